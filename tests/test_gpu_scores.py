"""GPU parity of the block scores (qsa_index_scores on MFMA, qsa_index_scores_decode) through
the C ABI.  Masked and padded entries must be exactly -FLT_MAX; scores are compared within the
FP32 summation bound: |gpu - ref| <= c * 2^-16 * sum_h sum_d |q_hd k_d| + 2^-22 |ref|, where c =
1/sqrtf(128) (128-term dots in FP32: n*u = 2^-17 relative to the sum of |products|, doubled;
then three head additions and the scale)."""
import numpy as np
import pytest
import torch

from sparse_attention_indexer_qsa_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
NEG = np.float32(-np.finfo(np.float32).max)


@pytest.fixture(scope="module")
def qsa():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import sparse_attention_indexer_qsa_amd.qsa as q
    return q


@pytest.fixture(scope="module")
def O():
    from oracle.ref import default
    return default()


def _abs_bound(q, kb, dt, rows, ctx, S):
    """c * sum_h sum_d |q_hd k_d| for global `rows` against every block of its sequence, as
    (sum_h |q_h|) . |k| per sequence."""
    qsum = np.abs(G.widen(q.reshape(-1, 4, 128)[rows], dt)).sum(axis=1)   # [R, 128]
    kf = np.abs(G.widen(kb, dt))                                          # [B, nb, 128]
    b = rows // S
    out = np.empty((len(rows), kb.shape[1]))
    for bb in np.unique(b):
        sel = b == bb
        out[sel] = qsum[sel] @ kf[bb].T
    return (1 / np.sqrt(128.0)) * out


def check_logits(got, ref, bound, what):
    gbits, rbits = got.view(np.uint32), ref.view(np.uint32)
    neg = ref == NEG
    assert np.array_equal(gbits[neg], rbits[neg]), f"{what}: -FLT_MAX entries differ"
    assert np.all(got[~neg] != NEG), f"{what}: visible entry masked"
    err = np.abs(got[~neg].astype(np.float64) - ref[~neg].astype(np.float64))
    tol = 2.0 ** -16 * bound[~neg] + 2.0 ** -22 * np.abs(ref[~neg].astype(np.float64)) + 1e-30
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} beyond tolerance, max err/tol " \
        f"{float((err / tol).max()):.3g}"
    return int((gbits != rbits).sum()), float((err / tol).max()) if err.size else 0.0


def _inputs(O, wl):
    q = O.q_prep(wl.indexQk, wl.cosSin, wl.ctx, wl.wQ, wl.eps, wl.dt)
    kb = O.k_compress(wl.indexQk, wl.cosSin, wl.ctx, wl.wK, wl.eps, wl.numBlocks, 0,
                      wl.numBlocks, 0, wl.dt)
    return q, kb


def _gpu_scores(qsa, q, kb, ctx, dt, rowStart, numRows, nb):
    out = G.Guarded((numRows, nb), torch.float32, fill=float("nan"))
    qsa.qsa_index_scores(out.t, G.dev_bits(q), G.dev_bits(kb), G.dev(ctx), nb, rowStart,
                         numRows, dt=dt)
    torch.cuda.synchronize()
    out.check()
    return out.t.cpu().numpy()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_scores_batched_prefill_full(qsa, O, dt):
    """All 16384 rows x 512 blocks of the batched prefill (lengths 0, 2048, ragged, NaN
    padding), K1a/K1b outputs of the oracle as inputs."""
    wl = W.config2(dt)
    q, kb = _inputs(O, wl)
    rows = wl.B * wl.S
    got = _gpu_scores(qsa, q, kb, wl.ctx, dt, 0, rows, wl.numBlocks)
    ref = O.scores(q, kb, wl.ctx, 0, rows, dt)
    bound = _abs_bound(q, kb, dt, np.arange(rows), wl.ctx, wl.S)
    nd, worst = check_logits(got, ref, bound, f"batched {dt}")
    print(f"[parity] scores batched {dt}: {nd} of {got.size} differ in bits, worst err/tol "
          f"{worst:.3g}", flush=True)


def test_scores_long_prefill_chunk(qsa, O):
    """The long prefill (S=131072, 32768 blocks): a 2048-row chunk from the middle, sampled
    rows checked one by one against the oracle; every row's mask checked."""
    wl = W.config3()
    q, kb = _inputs(O, wl)
    r0, n = 65536 + 13, 2048
    got = _gpu_scores(qsa, q, kb, wl.ctx, wl.dt, r0, n, wl.numBlocks)
    t = r0 + np.arange(n)
    nvis = (t + 1) // 4
    g = np.arange(wl.numBlocks)
    assert np.all((got == NEG) == (g[None, :] >= nvis[:, None]))
    rng = np.random.default_rng(3)
    sample = np.sort(rng.choice(n, 24, replace=False))
    for i in sample:
        ref = O.scores(q, kb, wl.ctx, r0 + int(i), 1, wl.dt)
        bound = _abs_bound(q, kb, wl.dt, np.array([r0 + int(i)]), wl.ctx, wl.S)
        check_logits(got[i:i + 1], ref, bound, f"long row {r0 + i}")


def test_scores_long_prefill_bench_rows(qsa, O):
    """The launch the benchmark times: rows [65536, 73728) of the long prefill against all
    32768 blocks (128 tiles of 64 tokens x 8 ranges of 4096 blocks).  Every row's mask is
    checked; 32 sampled rows, the chunk's first and last among them, against the oracle."""
    wl = W.config3()
    q, kb = _inputs(O, wl)
    r0, n = 65536, 8192
    print(f"[gpu] scores rows [{r0}, {r0 + n}) x {wl.numBlocks}", flush=True)
    got = _gpu_scores(qsa, q, kb, wl.ctx, wl.dt, r0, n, wl.numBlocks)
    nvis = (r0 + np.arange(n) + 1) // 4
    for i0 in range(0, n, 1024):                 # the mask of every row, 1024 rows at a time
        blk = got[i0:i0 + 1024]
        masked = blk == NEG
        assert np.array_equal(masked, np.arange(wl.numBlocks)[None, :] >= nvis[i0:i0 + 1024, None])
    rng = np.random.default_rng(5)
    sample = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 30, replace=False)]))
    for i in sample:
        ref = O.scores(q, kb, wl.ctx, r0 + int(i), 1, wl.dt)
        bound = _abs_bound(q, kb, wl.dt, np.array([r0 + int(i)]), wl.ctx, wl.S)
        check_logits(got[i:i + 1], ref, bound, f"bench row {r0 + i}")
    print(f"[parity] scores bench rows: mask of {n} rows, {sample.size} rows vs oracle", flush=True)


def test_scores_chunks_and_edges(qsa, O):
    """Ragged S (not a multiple of the 32-token tile), chunks that start mid-tile and span
    sequences, a length-0 sequence: chunks equal slices of one GPU call bit for bit, and match
    the oracle."""
    rng = np.random.default_rng(97)
    dt = "bf16"
    B, S = 3, 203
    nb = (S + 3) // 4
    q = W.to_bits(rng.standard_normal((B, S, 4, 128), dtype=np.float32), dt)
    kb = W.to_bits(rng.standard_normal((B, nb, 128), dtype=np.float32), dt)
    ctx = np.array([203, 0, 150], np.int32)
    q[2, 150:] = 0x7FC0                      # padded rows are never read
    full = _gpu_scores(qsa, q, kb, ctx, dt, 0, B * S, nb)
    ref = O.scores(q, kb, ctx, 0, B * S, dt)
    check_logits(full, ref, _abs_bound(q, kb, dt, np.arange(B * S), ctx, S), "edges")
    for r0, n in ((0, 1), (5, 37), (190, 40), (201, 250), (600, 9)):
        part = _gpu_scores(qsa, q, kb, ctx, dt, r0, n, nb)
        assert np.array_equal(part.view(np.uint32), full[r0:r0 + n].view(np.uint32)), (r0, n)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_scores_ragged_ranges(qsa, O, dt):
    """numBlocks = 4103: one full 4096-block range and one of 7 blocks that the last rows of the
    first sequence reach; a row length that is not a multiple of 4, so the -FLT_MAX fill takes
    its scalar path; kbar rows beyond every row's reach; two sequences of different lengths;
    a chunk that crosses from the first sequence into the second mid-tile."""
    rng = np.random.default_rng(211)
    B, S, nb = 2, 16390, 4103
    q = W.to_bits(rng.standard_normal((B, S, 4, 128), dtype=np.float32), dt)
    kb = W.to_bits(rng.standard_normal((B, nb, 128), dtype=np.float32), dt)
    ctx = np.array([16390, 9001], np.int32)
    r0, n = 16000, 800
    print(f"[gpu] scores ragged ranges {dt} nb={nb} rows [{r0}, {r0 + n})", flush=True)
    got = _gpu_scores(qsa, q, kb, ctx, dt, r0, n, nb)
    ref = O.scores(q, kb, ctx, r0, n, dt)
    check_logits(got, ref, _abs_bound(q, kb, dt, r0 + np.arange(n), ctx, S), f"ragged {dt}")


def test_scores_narrow_numblocks(qsa, O):
    """numBlocks below a row's complete-block count (kbar holds only the first 50 blocks of a
    300-token sequence): rows see min((t+1)/4, numBlocks) blocks, the rest of no row exists."""
    rng = np.random.default_rng(223)
    dt, B, S, nb = "bf16", 2, 300, 50
    q = W.to_bits(rng.standard_normal((B, S, 4, 128), dtype=np.float32), dt)
    kb = W.to_bits(rng.standard_normal((B, nb, 128), dtype=np.float32), dt)
    ctx = np.array([300, 170], np.int32)
    got = _gpu_scores(qsa, q, kb, ctx, dt, 0, B * S, nb)
    ref = O.scores(q, kb, ctx, 0, B * S, dt)
    check_logits(got, ref, _abs_bound(q, kb, dt, np.arange(B * S), ctx, S), "narrow numBlocks")


def test_scores_row_groups_span_sequences(qsa, O):
    """A wide logits row (numBlocks = 32768, 128 slices of 256 blocks, so few row groups) over
    many short sequences: each row group walks bands of several sequences in turn (the kbar
    fragments are reloaded per sequence), lengths 0, 1, 4, 5 and ragged, a chunk that starts
    and ends mid-band; every row against the oracle."""
    rng = np.random.default_rng(227)
    dt, B, S, nb = "bf16", 9, 600, 32768
    q = W.to_bits(rng.standard_normal((B, S, 4, 128), dtype=np.float32), dt)
    kb = W.to_bits(rng.standard_normal((B, 160, 128), dtype=np.float32), dt)
    kbw = np.zeros((B, nb, 128), np.uint16)
    kbw[:, :160] = kb
    ctx = np.array([600, 0, 1, 4, 5, 333, 599, 17, 600], np.int32)
    r0, n = 7, B * S - 20
    print(f"[gpu] scores row groups over {B} sequences, nb={nb}", flush=True)
    got = _gpu_scores(qsa, q, kbw, ctx, dt, r0, n, nb)
    ref = O.scores(q, kbw, ctx, r0, n, dt)
    check_logits(got, ref, _abs_bound(q, kbw, dt, r0 + np.arange(n), ctx, S), "row groups")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_scores_decode(qsa, O, dt):
    """Decode scores of one query token per sequence against V-tails that the oracle's K1b
    wrote into a host pool (the same pool bits are uploaded for the GPU call); entries past
    each row's prefix keep their content; an unused V page entry, and one past the pool, score
    -FLT_MAX."""
    rng = np.random.default_rng(101)
    L = np.array([4000, 1031, 7, 3, 2048, 513, 0, 64], np.int32)
    B, Lmax = len(L), int(L.max())
    x = W.to_bits(rng.standard_normal((B, Lmax, 640), dtype=np.float32), dt)
    wK = W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt)
    m = (Lmax + 127) // 128
    numPages = B * m
    pt = np.stack([rng.permutation(numPages)[:B * m].reshape(B, m),
                   rng.permutation(numPages)[:B * m].reshape(B, m) + numPages], 1).astype(np.int32)
    pt[1, 1, 3] = -1
    pt[0, 1, 5] = 2 * numPages                  # past the pool: not a V page
    spec = W.PoolSpec(numPages, pt)
    cs = W.cos_sin_table(Lmax + 8, 1e4)
    nb = (Lmax + 3) // 4
    rpool = G.oracle_pool(spec)
    kbh = O.k_compress(x, cs, L, wK, 1e-6, nb, 0, nb, 0, dt, pool=rpool)
    pool = G.device_pool(spec)
    pool.pool.copy_(torch.from_numpy(rpool.data.view(np.int16)))
    qdec = W.to_bits(rng.standard_normal((B, 1, 4, 128), dtype=np.float32), dt)
    out = torch.full((B, nb), float("nan"), device="cuda")
    print(f"[gpu] scores_decode B={B} maxBlocks={nb}", flush=True)
    qsa.qsa_index_scores_decode(out, G.dev_bits(qdec), G.dev(L), pool, nb, dt=dt)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = O.scores_decode(qdec, L, rpool, nb, dt)
    for b in range(B):
        n = int(L[b]) // 4
        assert np.all(np.isnan(got[b, n:]))
        bound = (1 / np.sqrt(128.0)) * np.einsum(
            "hd,gd->g", np.abs(G.widen(qdec[b, 0], dt)), np.abs(G.widen(kbh[b, :n], dt)))
        check_logits(got[b, :n], ref[b, :n], bound, f"decode seq {b}")
    assert np.all(got[1, 96:128] == NEG)
    assert np.all(got[0, 160:192] == NEG)


def test_scores_decode_bench_batch(qsa, O):
    """The launch the benchmark times: the decode batch of 64 sequences (one new token each,
    contexts up to 32772, rows of (max ctx + 3) / 4 blocks) over the full paged pool of the
    decode workload (16384 pages per plane, 10 % of the entries unused).  The V pages that six
    sampled sequences reach hold seeded values, the rest of the pool zeros; those sequences are
    checked against the oracle on a host pool holding only their pages, renumbered."""
    wl = W.config4()
    ctx = (wl.ranges[0] + 1).astype(np.int32)
    B, mb, dt = len(ctx), int((ctx.max() + 3) // 4), "bf16"
    spec, hs = wl.pool, wl.pool.headSize
    rng = np.random.default_rng(61)
    sample = sorted({int(np.argmax(ctx)), int(np.argmin(ctx)),
                     *rng.choice(B, 4, replace=False).tolist()})
    hpt = np.full((len(sample), 2, spec.maxPagesPerSeq), -1, np.int32)
    dev_pages = []
    for k, b in enumerate(sample):
        nvis = min(int(ctx[b]) // 4, mb)
        for slot in range(min((4 * nvis + 127) // 128, spec.maxPagesPerSeq)):
            v = int(spec.pageTable[b, 1, slot])
            if v >= 0:
                hpt[k, 1, slot] = len(dev_pages)
                dev_pages.append(v)
    P = len(dev_pages)
    tails = W.to_bits(rng.standard_normal((P, 128, 128), dtype=np.float32), dt)
    from oracle.ref import Pool
    hdata = np.zeros((2 * ((P + 1) // 2), 128, 1, 128), np.uint16)
    hdata[:P, :, 0, :] = tails
    qdec = W.to_bits(rng.standard_normal((B, 1, 4, 128), dtype=np.float32), dt)
    ref = O.scores_decode(qdec[sample], ctx[sample], Pool(hdata, hpt, (P + 1) // 2, 0), mb, dt)
    pool = qsa.PoolState(torch.zeros(spec.shape, dtype=torch.int16, device="cuda"),
                         G.dev(spec.pageTable.astype(np.int32)), spec.numPages,
                         spec.numKVHeads, spec.poolHeadDim, hs)
    idx = torch.tensor(dev_pages, dtype=torch.long, device="cuda")
    pool.pool[idx, :, 0, hs:hs + 128] = torch.from_numpy(tails.view(np.int16)).cuda()
    out = torch.full((B, mb), float("nan"), device="cuda")
    print(f"[gpu] scores_decode bench batch B={B} maxBlocks={mb} sampled {sample}", flush=True)
    qsa.qsa_index_scores_decode(out, G.dev_bits(qdec), G.dev(ctx), pool, mb, dt=dt)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    del pool
    for k, b in enumerate(sample):
        n = min(int(ctx[b]) // 4, mb)
        assert np.all(np.isnan(got[b, n:]))
        kv = np.zeros((n, 128), np.uint16)
        for g in range(n):
            slot = (4 * g) // 128
            h = hpt[k, 1, slot] if slot < spec.maxPagesPerSeq else -1
            if h >= 0:
                kv[g] = tails[h, (4 * g) % 128]
        bound = (1 / np.sqrt(128.0)) * np.einsum(
            "hd,gd->g", np.abs(G.widen(qdec[b, 0], dt)), np.abs(G.widen(kv, dt)))
        check_logits(got[b, :n], ref[k, :n], bound, f"bench decode seq {b}")
    print(f"[parity] scores_decode bench batch: {len(sample)} sampled sequences", flush=True)

