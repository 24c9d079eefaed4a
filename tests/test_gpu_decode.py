"""GPU parity of the decode pre-pass (qsa_index_pre_decode, the page's
launchQsaIndexerPreDecode with n new tokens per sequence) through the C ABI."""
import numpy as np
import pytest
import torch

from sparse_attention_indexer_qsa_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qsa():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import sparse_attention_indexer_qsa_amd.qsa as q
    return q


@pytest.fixture(scope="module")
def O():
    from oracle.ref import default
    return default()


def _plant_past_keys(rng, wl, data):
    """Write finite random keys into the K-tails of the past tokens of each sequence's
    incomplete block (positions [4*floor(p/4), p)), which a decode step needs."""
    p = wl.ranges[0]
    view = data.reshape(data.shape[0], 128, data.shape[2], data.shape[3])
    for b in range(wl.B):
        for t in range(4 * (int(p[b]) // 4), int(p[b])):
            pid = wl.pool.pageTable[b, 0, t // 128]
            if pid >= 0:
                view[pid, t % 128, 0, 256:384] = W.to_bits(
                    rng.standard_normal(128, dtype=np.float32), wl.dt)


@pytest.mark.parametrize("shape,single,dt", [("small", False, "bf16"), ("small", True, "bf16"),
                                              ("small", False, "f16"), ("full", False, "bf16"),
                                              ("full", False, "f16")])
def test_pre_decode_vs_oracle(qsa, O, shape, single, dt):
    """A batch of 64 decoding sequences, 1..4 new tokens each (or one, with newLens = NULL),
    pool with 10 % unused entries.  "small": 4096 pages, 64 slots per sequence, past lengths up
    to 8188.  "full": the decode workload's own pool and the benchmark's launch, 16384 pages
    (6.44 GB, element offsets past 2^31), 256 slots, past lengths up to 32768.  q rows within
    1 ulp; the pool bit for bit except inside the V-tails the oracle writes, which are within
    1 ulp of the oracle's kbar."""
    if shape == "small":
        wl = W.config4(B=64, numPages=4096, maxPagesPerSeq=64, max_past=8188, dt=dt)
    else:
        wl = W.config4(dt=dt)
    past, new = wl.ranges[0], wl.ctx - wl.ranges[0]
    if single:
        wl.ctx = (past + 1).astype(np.int32)
        new = np.ones_like(new)
    rng = np.random.default_rng(44)
    data = np.full(wl.pool.shape, W.SENTINEL_U16, np.uint16)
    _plant_past_keys(rng, wl, data)
    from oracle.ref import Pool
    rpool = data.copy()
    rq = O.pre_decode(wl.indexQk, wl.cosSin, wl.ctx, None if single else new, wl.wQ, wl.wK,
                      wl.eps, Pool(rpool, wl.pool.pageTable, wl.pool.numPages, 256), wl.dt)
    pool = G.device_pool(wl.pool)
    pool.pool.copy_(torch.from_numpy(data.view(np.int16)))
    q = G.Guarded((wl.B, wl.S, 4, 128), torch.int16, fill=-1)
    print(f"[gpu] pre_decode {shape} B={wl.B} S={wl.S} pages={wl.pool.numPages} "
          f"single={single} {dt}", flush=True)
    qsa.qsa_index_pre_decode(q.t, G.dev_bits(wl.indexQk), G.dev(wl.cosSin), G.dev(wl.ctx),
                             G.dev_bits(wl.wQ), G.dev_bits(wl.wK), wl.eps, pool,
                             newLens=None if single else G.dev(new.astype(np.int32)), dt=wl.dt)
    torch.cuda.synchronize()
    q.check()
    qh = G.host_bits(q.t)
    nd = G.compare_T(qh, rq, wl.dt, what="qNormed")
    for b in range(wl.B):
        assert np.all(qh[b, new[b]:] == 0)
    ph = G.host_bits(pool.pool)
    del pool
    # cells the oracle wrote in V-plane rows: the only ones whose bits may differ
    rows_written = np.argwhere(np.any(rpool != data, axis=-1))
    v_rows = rows_written[rows_written[:, 0] >= wl.pool.numPages]
    # compare the V-tails within 1 ulp, then put the oracle's bits there and demand equality
    for page, row, head in v_rows:
        assert head == 0
        G.compare_T(ph[page, row, 0, 256:], rpool[page, row, 0, 256:], wl.dt, what="V-tail")
        ph[page, row, 0, 256:] = rpool[page, row, 0, 256:]
    diff = ph != rpool
    assert not diff.any(), f"pool differs outside the V-tails in {int(diff.sum())} elements, " \
        f"e.g. at {np.argwhere(diff)[:4].tolist()}"
    print(f"[parity] pre_decode {shape} single={single} {dt}: q bits differing {nd}, pool rows "
          f"written {len(rows_written)} ({len(v_rows)} V-tails)", flush=True)
    assert len(rows_written) > 0 and len(v_rows) > 0


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_pre_decode_equals_prefill_on_gpu(qsa, dt):
    """Prefill of a prefix, then decode steps of 1..4 tokens, all on the GPU, leaves in the
    V-tails exactly the kbar of one GPU prefill over the whole history and yields its q rows."""
    rng = np.random.default_rng(61)
    L = np.array([700, 513, 131, 260, 9, 4], np.int32)
    B, Lmax = len(L), int(L.max())
    x = W.to_bits(rng.standard_normal((B, Lmax, 640), dtype=np.float32), dt)
    wQ = W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt)
    wK = W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt)
    m = (Lmax + 127) // 128
    numPages = B * m
    pt = np.stack([rng.permutation(numPages)[:B * m].reshape(B, m),
                   rng.permutation(numPages)[:B * m].reshape(B, m) + numPages], 1).astype(np.int32)
    spec = W.PoolSpec(numPages, pt)
    cs = G.dev(W.cos_sin_table(Lmax + 8, 1e4))
    nb = (Lmax + 3) // 4
    xd, wq, wk = G.dev_bits(x), G.dev_bits(wQ), G.dev_bits(wK)
    # one prefill over the whole history
    q_full = torch.empty(B, Lmax, 4, 128, dtype=torch.int16, device="cuda")
    kb_full = torch.empty(B, nb, 128, dtype=torch.int16, device="cuda")
    qsa.qsa_index_prefill(q_full, kb_full, xd, cs, G.dev(L), wq, wk, 1e-6, nb, dt=dt)
    # prefix prefill, then decode steps
    pool = G.device_pool(spec)
    p0 = np.array([37, 128, 1, 259, 0, 3], np.int32)
    Spre = int(p0.max())
    xpre = xd[:, :Spre].contiguous()
    kb_tmp = torch.empty(B, nb, 128, dtype=torch.int16, device="cuda")
    qsa.qsa_index_k_compress(kb_tmp, xpre, cs, G.dev(p0), wk, 1e-6, nb, 0, nb, 0, pool=pool,
                             dt=dt)
    qsa.qsa_index_persist(pool, xpre, None, G.dev(p0), nb, 0, nb, 0, dt=dt)
    cur = p0.copy()
    qf = G.host_bits(q_full)
    while np.any(cur < L):
        n = np.minimum(rng.integers(1, 5, B), L - cur).astype(np.int32)
        rows = np.zeros((B, 4, 640), np.uint16)
        for b in range(B):
            rows[b, :n[b]] = x[b, cur[b]:cur[b] + n[b]]
        ctx = (cur + n).astype(np.int32)
        q = torch.empty(B, 4, 4, 128, dtype=torch.int16, device="cuda")
        qsa.qsa_index_pre_decode(q, G.dev_bits(rows), cs, G.dev(ctx), wq, wk, 1e-6, pool,
                                 newLens=G.dev(n), dt=dt)
        qh = G.host_bits(q)
        for b in range(B):
            assert np.array_equal(qh[b, :n[b]], qf[b, cur[b]:ctx[b]]), (b, cur[b])
        cur = ctx
    torch.cuda.synchronize()
    view = G.host_bits(pool.pool)
    kbf = G.host_bits(kb_full)
    for b in range(B):
        for g in range(int(L[b]) // 4):
            pid = pt[b, 1, (4 * g) // 128]
            assert np.array_equal(view[pid, (4 * g) % 128, 0, 256:], kbf[b, g]), (b, g)
