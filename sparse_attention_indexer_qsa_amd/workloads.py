"""Seeded synthetic workloads of the QSA indexer hot path.

This module only draws inputs: random numbers (numpy PCG64), their conversion to the
activation type T by torch's round-to-nearest-even cast, the cosSin table, context lengths and
page tables.  It holds none of the method's arithmetic, so the GPU library and the CPU oracle
can both be fed from it without sharing any code of the method.

T tensors are returned as numpy ``uint16`` bit patterns, cosSin as FP32, everything else int32.

The five workloads (shapes from the method's documented geometry: indexQk rows of 640 = four
128-dim q heads then one raw 128-dim key, cosSin rows of 64 = 32 cos then 32 sin, a pool
[2*numPages, 128, 2, 384] whose indexer columns start at 256):
  1  tiny prefill        B=1,  S=64,     bf16, ctx=[61]
  2  batched prefill     B=8,  S=2048,   fp16 and bf16, NaN padding
  3  long prefill        B=1,  S=131072, bf16, 1% outlier rows x30, theta=1e6
  4  decode sub-range    B=64, S=4 new-row slots, bf16, per-sequence ranges, paged pool
  5  mixed serving step  B=32, S=8192,   fp16, log-uniform lengths, paged pool
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

NUM_KV_HEADS = 2
POOL_HEAD_DIM = 384
HEAD_SIZE = 256
SENTINEL_U16 = 0xA5A5          # pools are pre-filled with bytes 0xA5
NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00}


@dataclass
class PoolSpec:
    numPages: int
    pageTable: np.ndarray          # int32 [B, 2, maxPagesPerSeq]
    numKVHeads: int = NUM_KV_HEADS
    poolHeadDim: int = POOL_HEAD_DIM
    headSize: int = HEAD_SIZE

    @property
    def maxPagesPerSeq(self):
        return self.pageTable.shape[2]

    @property
    def shape(self):
        return (2 * self.numPages, 128, self.numKVHeads, self.poolHeadDim)


@dataclass
class SubCall:
    """One k_compress call over a block sub-range, fed rows indexQk[:, pastLen:, :]."""
    blockBegin: int
    blockEnd: int
    pastLen: int


@dataclass
class Workload:
    name: str
    dt: str                        # "bf16" or "f16"
    indexQk: np.ndarray            # uint16 [B, S, 640]
    cosSin: np.ndarray             # float32 [maxPositions, 64]
    ctx: np.ndarray                # int32 [B]
    wQ: np.ndarray                 # uint16 [128]
    wK: np.ndarray                 # uint16 [128]
    eps: float
    numBlocks: int
    blockBegin: int
    blockEnd: int
    pastLen: int
    pool: Optional[PoolSpec]
    ranges: Optional[Tuple[np.ndarray, np.ndarray, np.ndarray, int]] = None
    run_q_prep: bool = True
    subcalls: list = field(default_factory=list)

    @property
    def B(self):
        return self.indexQk.shape[0]

    @property
    def S(self):
        return self.indexQk.shape[1]

    @property
    def maxPositions(self):
        return self.cosSin.shape[0]


def to_bits(values_f32, dt):
    """Round FP32 values to T with torch's round-to-nearest-even cast; return uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    return t.to(tdt).view(torch.int16).numpy().view(np.uint16)


def cos_sin_table(max_positions, theta):
    """cosSin [P, 64]: inverse frequency theta^(-2i/64), angle t*invf_i in FP64, then FP32."""
    i = np.arange(32, dtype=np.float64)
    invf = theta ** (-2.0 * i / 64.0)
    ang = np.arange(max_positions, dtype=np.float64)[:, None] * invf[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def _weights(rng, dt):
    wQ = to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt)
    wK = to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt)
    return wQ, wK


def _pad_nan(bits, ctx_rows, dt):
    """Fill rows t >= ctx_rows[b] of [B, S, 640] bits with T's quiet NaN (all columns)."""
    S = bits.shape[1]
    mask = np.arange(S)[None, :] >= np.asarray(ctx_rows)[:, None]
    bits[mask] = NAN_BITS[dt]
    return bits


def _perm_pages(rng, B, slots, numPages, offset):
    ids = rng.permutation(numPages)[: B * slots].astype(np.int32) + offset
    return ids.reshape(B, slots)


def config1():
    rng = np.random.default_rng(1)
    dt, B, S = "bf16", 1, 64
    x = rng.standard_normal((B, S, 640), dtype=np.float32)
    wQ, wK = _weights(rng, dt)
    pt = np.array([[[3], [1 + 4]]], dtype=np.int32)
    return Workload("tiny_prefill", dt, to_bits(x, dt), cos_sin_table(64, 1e4),
                    np.array([61], np.int32), wQ, wK, 1e-6, 16, 0, 16, 0, PoolSpec(4, pt))


def config2(dt="bf16", S=2048):
    """Batched prefill; both dtypes come from the same draw."""
    rng = np.random.default_rng(2)
    B = 8
    x = 1.5 * rng.standard_normal((B, S, 640), dtype=np.float32)
    wQ32 = 0.1 * rng.standard_normal(128, dtype=np.float32)
    wK32 = 0.1 * rng.standard_normal(128, dtype=np.float32)
    ctx = rng.integers(0, S + 1, B).astype(np.int32)
    ctx[0], ctx[1] = 0, S
    for j, r in zip((2, 3, 4), (1, 2, 3)):          # lengths that are 1, 2, 3 mod 4
        ctx[j] = min(S - 4 + r, max(r, ctx[j] - ctx[j] % 4 + r))
    bits = _pad_nan(to_bits(x, dt), ctx, dt)
    pages = S // 128
    numPages = B * pages
    pt = np.stack([_perm_pages(rng, B, pages, numPages, 0),
                   _perm_pages(rng, B, pages, numPages, numPages)], axis=1)
    nb = (S + 3) // 4
    return Workload(f"batched_prefill_{dt}", dt, bits, cos_sin_table(S, 1e4), ctx,
                    to_bits(wQ32, dt), to_bits(wK32, dt), 1e-6, nb, 0, nb, 0,
                    PoolSpec(numPages, pt))


def config3(S=131072):
    rng = np.random.default_rng(3)
    dt, B = "bf16", 1
    x = rng.standard_normal((B, S, 640), dtype=np.float32)
    n_out = max(1, round(0.01 * S))
    rows = rng.choice(S, n_out, replace=False)
    x[0, rows, :] *= 30.0
    wQ, wK = _weights(rng, dt)
    pages = (S + 127) // 128
    pt = np.stack([_perm_pages(rng, B, pages, pages, 0),
                   _perm_pages(rng, B, pages, pages, pages)], axis=1)
    nb = (S + 3) // 4
    return Workload("long_prefill", dt, to_bits(x, dt), cos_sin_table(S, 1e6),
                    np.array([S], np.int32), wQ, wK, 1e-6, nb, 0, nb, 0, PoolSpec(pages, pt))


def _drop_entries(rng, pt, frac):
    """Set `frac` of the entries of each plane to -1 (unused page)."""
    B, _, m = pt.shape
    for plane in range(2):
        flat = pt[:, plane, :].reshape(-1)
        k = int(round(frac * flat.size))
        flat[rng.choice(flat.size, k, replace=False)] = -1
        pt[:, plane, :] = flat.reshape(B, m)
    return pt


def config4(B=64, numPages=16384, maxPagesPerSeq=256, max_past=32768, dt="bf16"):
    """Decode: 1..4 new tokens per sequence, ranges cover only newly completed blocks (the same
    draws for either element type)."""
    rng = np.random.default_rng(4)
    S = 4
    past = rng.integers(4, max_past + 1, B).astype(np.int32)
    new = rng.integers(1, 5, B).astype(np.int32)
    ctx = (past + new).astype(np.int32)
    x = rng.standard_normal((B, S, 640), dtype=np.float32)
    wQ, wK = _weights(rng, dt)
    bits = _pad_nan(to_bits(x, dt), new, dt)
    pt = np.stack([rng.permutation(numPages)[: B * maxPagesPerSeq].reshape(B, maxPagesPerSeq),
                   rng.permutation(numPages)[: B * maxPagesPerSeq].reshape(B, maxPagesPerSeq)
                   + numPages], axis=1).astype(np.int32)
    pt = _drop_entries(rng, pt, 0.10)
    nb = int((ctx.max() + 3) // 4)
    ranges = (past.copy(), (past >> 2).astype(np.int32), (ctx >> 2).astype(np.int32), 1)
    return Workload("decode_subrange", dt, bits, cos_sin_table(4 * nb, 1e4), ctx, wQ, wK,
                    1e-6, nb, 0, 0, 0, PoolSpec(numPages, pt), ranges=ranges,
                    run_q_prep=False)


def config5(B=32, S=8192, numPages=8192):
    """Mixed serving step, fp16, log-uniform lengths, paged pool with 10% unused entries."""
    rng = np.random.default_rng(5)
    dt = "f16"
    ctx = np.clip(np.round(np.exp(rng.uniform(0.0, np.log(S), B))), 1, S).astype(np.int32)
    x = rng.standard_normal((B, S, 640), dtype=np.float32)
    wQ, wK = _weights(rng, dt)
    bits = _pad_nan(to_bits(x, dt), ctx, dt)
    pages = S // 128
    pt = np.stack([_perm_pages(rng, B, pages, numPages, 0),
                   _perm_pages(rng, B, pages, numPages, numPages)], axis=1)
    pt = _drop_entries(rng, pt, 0.10)
    nb = (S + 3) // 4
    cuts = np.sort(rng.choice(np.arange(1, nb), 3, replace=False))
    bounds = [0, *cuts.tolist(), nb]
    subcalls = []
    for i in range(4):
        if i == 0:
            p = 0
        else:
            p = 4 * bounds[i] - int(rng.integers(0, 2))   # 4c or 4c-1
        subcalls.append(SubCall(bounds[i], bounds[i + 1], p))
    return Workload("mixed_serving", dt, bits, cos_sin_table(S, 1e4), ctx, wQ, wK, 1e-6, nb,
                    0, nb, 0, PoolSpec(numPages, pt), subcalls=subcalls)


FLT_MAX = float(np.finfo(np.float32).max)


def _logit_values(rng, n, style):
    """n FP32 logits in a style: "scores" (non-negative, a ReLU's share of exact zeros, coarse
    quantisation so that equal values recur), "ties" (few distinct values), "normal"
    (both signs, continuous), "special" (normal plus +-0, subnormals, +-inf, NaNs of both signs,
    +-FLT_MAX), "special_ge" (as "special" without the values below -FLT_MAX: -inf and NaNs
    with the sign bit set)."""
    if style == "scores":
        v = np.maximum(rng.standard_normal(n) * 2.0, 0.0)
        return (np.round(v * 64.0) / 64.0).astype(np.float32)
    if style == "ties":
        return rng.integers(0, 4, n).astype(np.float32) * np.float32(0.5)
    v = rng.standard_normal(n).astype(np.float32)
    if style in ("special", "special_ge"):
        low = style == "special"
        specials = np.array([0.0, -0.0, 1e-45, -1e-45, np.inf, -FLT_MAX, FLT_MAX]
                            + ([-np.inf] if low else []), np.float32)
        pick = rng.random(n) < 0.05
        v[pick] = specials[rng.integers(0, len(specials), int(pick.sum()))]
        nan = rng.random(n) < 0.01
        neg = (rng.random(n) < 0.5) & low
        bits = np.where(neg, 0xFFC00001, 0x7FC00000).astype(np.uint32)
        v.view(np.uint32)[nan] = bits[nan]
    return v


def prefill_logits(seed, ctx, S, numBlocks, rowStart, numRows, styles=("scores",)):
    """Logits FP32 [numRows, numBlocks] laid out as the block scores of rows [rowStart,
    rowStart+numRows) are: row r = b*S + t has its first (t+1)//4 entries (capped at numBlocks)
    drawn in one of `styles` (cycled by row), the rest -FLT_MAX; padded rows (t >= ctx[b])
    are -FLT_MAX throughout."""
    rng = np.random.default_rng(seed)
    out = np.full((numRows, numBlocks), -FLT_MAX, np.float32)
    for i in range(numRows):
        r = rowStart + i
        b, t = divmod(r, S)
        if t >= ctx[b]:
            continue
        n = min((t + 1) // 4, numBlocks)
        out[i, :n] = _logit_values(rng, n, styles[i % len(styles)])
    return out


def decode_logits(seed, ctx, maxBlocks, styles=("scores", "ties", "normal", "special")):
    """Logits FP32 [B, maxBlocks] of one decode step: the first min(ctx/4, maxBlocks) entries of
    sequence b drawn in styles[b % len(styles)], the rest left NaN (never read)."""
    rng = np.random.default_rng(seed)
    B = len(ctx)
    out = np.full((B, maxBlocks), np.nan, np.float32)
    for b in range(B):
        n = max(0, min(int(ctx[b]) // 4, maxBlocks))
        out[b, :n] = _logit_values(rng, n, styles[b % len(styles)])
    return out


def decode_long_ctx(maxBlocks, B=64, seed=41):
    """Contexts of a decode batch over long sequences: B contexts uniform in [2 * maxBlocks,
    4 * maxBlocks + 3], so that every sequence holds between maxBlocks / 2 and maxBlocks
    complete blocks (128K to 256K tokens for maxBlocks = 65536, 512K to 1M for 262144)."""
    rng = np.random.default_rng(seed)
    return rng.integers(2 * maxBlocks, 4 * maxBlocks + 4, B).astype(np.int32)


def make(n, **kw):
    return {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}[n](**kw)
