"""An independent numpy re-derivation of K1a and K1b, used only to cross-check the C oracle.

Written separately from the oracle, vectorised over whole tensors: numpy binary32 arithmetic
(one rounding per operation, no FMA), the binary64 sum of squares rounded once, the binary64
reciprocal square root rounded once, and torch/numpy library casts for T <-> binary32.
Definitions: "Qsa Indexer Kernels", launchQsaIndexQPrep ("Exact numerics", "Padding
semantics") and launchQsaIndexKCompress (fixed-order block mean, cast, norm, rope at 4g).
"""
import numpy as np
import torch


def widen(bits, dt):
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dt == "bf16":
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    return bits.view(np.float16).astype(np.float32)


def narrow(values, dt):
    values = np.ascontiguousarray(values, dtype=np.float32)
    if dt == "bf16":
        return torch.from_numpy(values).to(torch.bfloat16).view(torch.int16).numpy() \
            .view(np.uint16)
    with np.errstate(over="ignore"):
        return values.astype(np.float16).view(np.uint16)


def _norm_rope(x, w1, c, s, eps):
    """x [..., 128] binary32; c, s [..., 32] broadcastable; returns pre-cast binary32."""
    sumsq = np.sum(x.astype(np.float64) ** 2, axis=-1).astype(np.float32)
    meanSq = sumsq / np.float32(128.0)
    v = meanSq + np.float32(eps)
    inv = (1.0 / np.sqrt(v.astype(np.float64))).astype(np.float32)
    y = (x * inv[..., None]) * w1
    lo, hi = y[..., :32], y[..., 32:64]
    o = y.copy()
    o[..., :32] = lo * c - hi * s
    o[..., 32:64] = hi * c + lo * s
    return o


def q_prep(indexQk, cosSin, ctx, wQ, eps, dt):
    B, S, _ = indexQk.shape
    x = widen(indexQk[..., :512], dt).reshape(B, S, 4, 128)
    w1 = np.float32(1.0) + widen(wQ, dt)
    c = cosSin[:S, None, :32]
    s = cosSin[:S, None, 32:]
    out = narrow(_norm_rope(x, w1, c[None], s[None], eps), dt)
    L = np.clip(np.asarray(ctx), 0, S)
    out[np.arange(S)[None, :] >= L[:, None]] = 0
    return out


def k_compress(indexQk, cosSin, ctx, wK, eps, numBlocks, dt):
    """Prefill form: blocks [0, numBlocks), pastLen 0."""
    B, S, _ = indexQk.shape
    nfull = S // 4
    k = widen(indexQk[:, :4 * nfull, 512:], dt).reshape(B, nfull, 4, 128)
    s = ((k[:, :, 0] + k[:, :, 1]) + k[:, :, 2]) + k[:, :, 3]
    m = widen(narrow(s * np.float32(0.25), dt), dt)
    w1 = np.float32(1.0) + widen(wK, dt)
    pos = 4 * np.arange(nfull)
    o = _norm_rope(m, w1, cosSin[pos, :32][None], cosSin[pos, 32:][None], eps)
    out = np.zeros((B, numBlocks, 128), np.uint16)
    out[:, :nfull] = narrow(o, dt)
    g = np.arange(numBlocks)
    invalid = (4 * g[None, :] + 3) >= np.asarray(ctx)[:, None]
    out[invalid] = 0
    return out
