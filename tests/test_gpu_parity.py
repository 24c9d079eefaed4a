"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle on the same
seeded inputs (sparse_attention_indexer_qsa_amd.workloads).

Bars (from the method's exactness classes): padding rows, invalid blocks, raw-K tail copies,
pool addressing and the cast block mean are bit-exact; normed/roped outputs are within 1 ulp
of T (with the rope-cancellation allowance of gpu_util.compare_T); FP32 intermediates are
within 1e-6 relative.  Pools are compared whole and bit for bit (expected_pool): every cell
other than the targets must keep its sentinel, every K-tail must hold the raw key's bits and
every V-tail the bits of the GPU's own kbar row.  Every output buffer carries red zones.
"""
import numpy as np
import pytest
import torch

from sparse_attention_indexer_qsa_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

KBAR_FILL = 0x1357   # kbar rows outside the block range must keep this


@pytest.fixture(scope="module")
def qsa():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import sparse_attention_indexer_qsa_amd.qsa as q
    return q


@pytest.fixture(scope="module")
def O():
    from oracle.ref import default
    return default()


def _ranges_dev(qsa, wl):
    if wl.ranges is None:
        return None
    pl, bb, be, span = wl.ranges
    return qsa.SeqRanges(G.dev(pl), G.dev(bb), G.dev(be), span)


def run_gpu(qsa, wl, fused=False, with_pool=True):
    """The hot path on the GPU: three calls (K1a, K1b with the fused V-tail, raw-K tails) or the
    fused prefill.  Returns host copies (qNormed or None, kbar, pool tensor or None)."""
    print(f"[gpu] {wl.name} dt={wl.dt} B={wl.B} S={wl.S} fused={fused}", flush=True)
    x, cs, ctx = G.dev_bits(wl.indexQk), G.dev(wl.cosSin), G.dev(wl.ctx)
    wQ, wK = G.dev_bits(wl.wQ), G.dev_bits(wl.wK)
    pool = G.device_pool(wl.pool) if with_pool else None
    q = G.Guarded((wl.B, wl.S, 4, 128), torch.int16, fill=-1)
    kb = G.Guarded((wl.B, wl.numBlocks, 128), torch.int16, fill=KBAR_FILL)
    if fused:
        qsa.qsa_index_prefill(q.t, kb.t, x, cs, ctx, wQ, wK, wl.eps, wl.numBlocks, pool=pool,
                              dt=wl.dt)
    else:
        if wl.run_q_prep:
            qsa.qsa_index_q_prep(q.t, x, cs, ctx, wQ, wl.eps, dt=wl.dt)
        r = _ranges_dev(qsa, wl)
        qsa.qsa_index_k_compress(kb.t, x, cs, ctx, wK, wl.eps, wl.numBlocks, wl.blockBegin,
                                 wl.blockEnd, wl.pastLen, ranges=r, pool=pool, dt=wl.dt)
        if with_pool:
            qsa.qsa_index_persist(pool, x, None, ctx, wl.numBlocks, wl.blockBegin, wl.blockEnd,
                                  wl.pastLen, ranges=r, dt=wl.dt)
    torch.cuda.synchronize()
    q.check()
    kb.check()
    qh = G.host_bits(q.t) if (wl.run_q_prep or fused) else None
    return qh, G.host_bits(kb.t), (G.host_bits(pool.pool) if with_pool else None)


def run_oracle(O, wl, with_pool=True, debug=False):
    pool = G.oracle_pool(wl.pool) if with_pool else None
    q = qd = None
    if wl.run_q_prep:
        r = O.q_prep(wl.indexQk, wl.cosSin, wl.ctx, wl.wQ, wl.eps, wl.dt, debug=debug)
        q, qd = r if debug else (r, None)
    kinit = np.full((wl.B, wl.numBlocks, 128), KBAR_FILL, np.uint16)
    r = O.k_compress(wl.indexQk, wl.cosSin, wl.ctx, wl.wK, wl.eps, wl.numBlocks, wl.blockBegin,
                     wl.blockEnd, wl.pastLen, wl.dt, kbar=kinit, ranges=wl.ranges, pool=pool,
                     debug=debug)
    kb, kd = r if debug else (r, None)
    if with_pool:
        O.persist(pool, wl.indexQk, None, wl.ctx, wl.numBlocks, wl.blockBegin, wl.blockEnd,
                  wl.pastLen, ranges=wl.ranges)
    return q, kb, (pool.data if with_pool else None), qd, kd


def _q_rows_cs(wl):
    """cosSin row of every (b, t, h) vector of qNormed."""
    return np.broadcast_to(wl.cosSin[None, :wl.S, None, :], (wl.B, wl.S, 4, 64))


def _kb_rows_cs(wl):
    g = np.arange(wl.numBlocks)
    pos = np.minimum(4 * g, wl.cosSin.shape[0] - 1)
    return np.broadcast_to(wl.cosSin[pos][None], (wl.B, wl.numBlocks, 64))


def expected_pool(O, wl, gpu_kbar):
    """The pool the GPU call must leave, bit for bit: the oracle's raw-K tail writes, then the
    oracle's V-tail writes with the GPU's own dense kbar rows as the values (a bit copy of kbar
    is what the page's V-tail write is).  Which cells are written, and where, is the oracle's
    alone; only the 256 bytes inside a V-tail come from the GPU, and those are checked against
    the oracle's kbar separately."""
    exp = G.oracle_pool(wl.pool)
    O.persist(exp, wl.indexQk, gpu_kbar, wl.ctx, wl.numBlocks, wl.blockBegin, wl.blockEnd,
              wl.pastLen, ranges=wl.ranges)
    return exp.data


def check_against_oracle(O, wl, got, debug_pre=True):
    q, kb, pool = got
    rq, rkb, rpool, qd, kd = run_oracle(O, wl, with_pool=pool is not None, debug=debug_pre)
    ndiff, stats = {}, {}
    if rq is not None:
        L = np.clip(wl.ctx, 0, wl.S)
        pad = np.arange(wl.S)[None, :] >= L[:, None]
        assert np.all(q[pad] == 0), "padding rows must be exact +0"
        st = {}
        ndiff["q"] = G.compare_T(q, rq, wl.dt, qd and qd["preCast"], _q_rows_cs(wl),
                                 "qNormed", stats=st)
        stats["q"] = st
    zero_rows = np.all(rkb == 0, axis=-1)
    assert np.array_equal(kb[zero_rows], rkb[zero_rows]), "invalid blocks must be exact +0"
    keep = np.all(rkb == KBAR_FILL, axis=-1)
    assert np.array_equal(kb[keep], rkb[keep]), "kbar rows outside the range were written"
    st = {}
    ndiff["kbar"] = G.compare_T(kb, rkb, wl.dt, kd and kd["preCast"], _kb_rows_cs(wl), "kbar",
                                stats=st)
    stats["kbar"] = st
    if pool is not None:
        # oracle self-consistency: its K1b pool write equals its persist of its own kbar
        # (launchQsaIndexKCompressPaged: the V-tail write is a copy of the dense kbar row)
        own = expected_pool(O, wl, rkb)
        assert np.array_equal(own, rpool), "oracle: fused and unfused pool writes differ"
        exp = expected_pool(O, wl, kb)
        assert pool.shape == exp.shape
        diff = pool != exp
        assert not diff.any(), \
            f"pool differs from the expected pool in {int(diff.sum())} elements, e.g. at " \
            f"{np.argwhere(diff)[:4].tolist()}"
        ndiff["pool_vs_oracle_kbar"] = int((pool != rpool).sum())
    print(f"[parity] {wl.name}: bits differing {ndiff}; 1-ulp / cancellation-clause elements "
          f"{stats}", flush=True)
    return ndiff


# ------------------------------------------------------------------------- the configs ---

def test_config1_tiny_prefill(qsa, O):
    wl = W.config1()
    nd = check_against_oracle(O, wl, run_gpu(qsa, wl))
    assert nd["pool_vs_oracle_kbar"] == 0


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_config2_batched_prefill(qsa, O, dt):
    wl = W.config2(dt)
    check_against_oracle(O, wl, run_gpu(qsa, wl))


def test_config3_long_prefill_fused(qsa, O):
    """The launch configuration the benchmark times: the fused prefill at B=1, S=131072."""
    wl = W.config3()
    got = run_gpu(qsa, wl, fused=True)
    check_against_oracle(O, wl, got)


def test_config3_three_calls_equal_fused(qsa):
    wl = W.config3()
    a = run_gpu(qsa, wl, fused=True)
    b = run_gpu(qsa, wl, fused=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_config4_decode_subrange(qsa, O):
    wl = W.config4()
    check_against_oracle(O, wl, run_gpu(qsa, wl))


def test_config5_mixed_serving(qsa, O):
    wl = W.config5()
    check_against_oracle(O, wl, run_gpu(qsa, wl))


@pytest.mark.parametrize("cfg", ["1", "2bf16", "2f16", "5"])
def test_fused_equals_three_calls(qsa, cfg):
    wl = {"1": W.config1, "2bf16": lambda: W.config2("bf16"), "2f16": lambda: W.config2("f16"),
          "5": W.config5}[cfg]()
    a = run_gpu(qsa, wl, fused=True)
    b = run_gpu(qsa, wl, fused=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_config5_subrange_union_equals_one_call(qsa):
    """Four sub-range calls with pastLen > 0 (rows indexQk[:, pastLen:]) reproduce one call."""
    wl = W.config5()
    x, cs, ctx = G.dev_bits(wl.indexQk), G.dev(wl.cosSin), G.dev(wl.ctx)
    wK = G.dev_bits(wl.wK)
    one = torch.full((wl.B, wl.numBlocks, 128), KBAR_FILL, dtype=torch.int16, device="cuda")
    qsa.qsa_index_k_compress(one, x, cs, ctx, wK, wl.eps, wl.numBlocks, 0, wl.numBlocks, 0,
                             dt=wl.dt)
    acc = torch.full_like(one, KBAR_FILL)
    for sc in wl.subcalls:
        rows = x[:, sc.pastLen:].contiguous()
        qsa.qsa_index_k_compress(acc, rows, cs, ctx, wK, wl.eps, wl.numBlocks, sc.blockBegin,
                                 sc.blockEnd, sc.pastLen, dt=wl.dt)
    torch.cuda.synchronize()
    assert torch.equal(acc, one)


# ---------------------------------------------------------------- intermediates and pins ---

@pytest.mark.parametrize("cfg", ["1", "2f16"])
def test_debug_intermediates(qsa, O, cfg):
    """FP32 intermediates within 1e-6 relative of the oracle; the cast block mean bit-exact."""
    wl = W.config1() if cfg == "1" else W.config2("f16", S=512)
    x, cs, ctx = G.dev_bits(wl.indexQk), G.dev(wl.cosSin), G.dev(wl.ctx)
    B, S, nb = wl.B, wl.S, wl.numBlocks
    f32 = dict(dtype=torch.float32, device="cuda")
    qd = {"meanSq": torch.zeros(B, S, 4, **f32), "invRms": torch.zeros(B, S, 4, **f32),
          "preCast": torch.zeros(B, S, 4, 128, **f32)}
    kd = {"mT": torch.zeros(B, nb, 128, dtype=torch.int16, device="cuda"),
          "meanSq": torch.zeros(B, nb, **f32), "invRms": torch.zeros(B, nb, **f32),
          "preCast": torch.zeros(B, nb, 128, **f32)}
    q = torch.zeros(B, S, 4, 128, dtype=torch.int16, device="cuda")
    kb = torch.zeros(B, nb, 128, dtype=torch.int16, device="cuda")
    qsa.qsa_index_q_prep(q, x, cs, ctx, G.dev_bits(wl.wQ), wl.eps, dt=wl.dt, debug=qd)
    qsa.qsa_index_k_compress(kb, x, cs, ctx, G.dev_bits(wl.wK), wl.eps, nb, 0, nb, 0, dt=wl.dt,
                             debug=kd)
    torch.cuda.synchronize()
    _, rqd = O.q_prep(wl.indexQk, wl.cosSin, wl.ctx, wl.wQ, wl.eps, wl.dt, debug=True)
    _, rkd = O.k_compress(wl.indexQk, wl.cosSin, wl.ctx, wl.wK, wl.eps, nb, 0, nb, 0, wl.dt,
                          debug=True)
    assert np.array_equal(G.host_bits(kd["mT"]), rkd["mT"]), "cast block mean must be bit-exact"
    for name, got, ref in [("q.meanSq", qd["meanSq"], rqd["meanSq"]),
                           ("q.invRms", qd["invRms"], rqd["invRms"]),
                           ("k.meanSq", kd["meanSq"], rkd["meanSq"]),
                           ("k.invRms", kd["invRms"], rkd["invRms"])]:
        g = got.cpu().numpy()
        assert np.allclose(g, ref, rtol=1e-6, atol=0), name
    for name, got, ref, rows_cs in [("q.preCast", qd["preCast"], rqd["preCast"], _q_rows_cs(wl)),
                                    ("k.preCast", kd["preCast"], rkd["preCast"],
                                     _kb_rows_cs(wl))]:
        g = got.cpu().numpy().reshape(-1, 128).astype(np.float64)
        r = ref.reshape(-1, 128).astype(np.float64)
        M = G.rope_terms(r, rows_cs)        # |y_a c| + |y_b s| on roped dims
        M[:, 64:] = 0.0                      # dims [64, 128) are not roped: 1e-6 relative only
        tol = 1e-6 * np.abs(r) + 2.0 ** -22 * M
        assert np.all(np.abs(g - r) <= tol), name


def test_golden_pins_on_gpu(qsa):
    """The hand-worked block-mean and kbar values, through the GPU library."""
    from tests.oracle_pins import GOLDEN, H
    for c in GOLDEN["block_mean_order"]["cases"]:
        x = np.zeros((1, 4, 640), np.uint16)
        x[0, :, 512] = [H(v) for v in c["k"]]
        cs = np.zeros((4, 64), np.float32)
        cs[:, :32] = 1
        kd = {"mT": torch.zeros(1, 1, 128, dtype=torch.int16, device="cuda"),
              "meanSq": torch.zeros(1, 1, device="cuda"), "invRms": torch.zeros(1, 1, device="cuda"),
              "preCast": torch.zeros(1, 1, 128, device="cuda")}
        kb = torch.zeros(1, 1, 128, dtype=torch.int16, device="cuda")
        qsa.qsa_index_k_compress(kb, G.dev_bits(x), G.dev(cs), G.dev(np.array([4], np.int32)),
                                 torch.zeros(128, dtype=torch.int16, device="cuda"), 1e-6, 1, 0, 1,
                                 0, dt=c["dt"], debug=kd)
        assert G.host_bits(kd["mT"])[0, 0, 0] == H(c["mT"]), c
    means = {c["dt"]: c for c in GOLDEN["block_mean_order"]["cases"] if c["mT"] != c["k"][0]}
    for c in GOLDEN["kbar_order_end_to_end"]["cases"]:
        x = np.zeros((1, 4, 640), np.uint16)
        x[0, :, 512] = [H(v) for v in means[c["dt"]]["k"]]
        x[0, :, 513] = H(c["d1"])
        cs = np.zeros((4, 64), np.float32)
        cs[:, :32] = 1
        kb = torch.zeros(1, 1, 128, dtype=torch.int16, device="cuda")
        qsa.qsa_index_k_compress(kb, G.dev_bits(x), G.dev(cs), G.dev(np.array([4], np.int32)),
                                 torch.zeros(128, dtype=torch.int16, device="cuda"), 1e-6, 1, 0, 1,
                                 0, dt=c["dt"])
        got = G.host_bits(kb)[0, 0, :2].tolist()
        assert got == [H(v) for v in c["kbar01"]], (c, [hex(v) for v in got])
    for c in GOLDEN["norm_closed_forms"]["cases"]:
        one = 0x3F80 if c["dt"] == "bf16" else 0x3C00
        x = np.zeros((1, 1, 640), np.uint16)
        if "out_all" in c:
            x[0, 0, :512] = one
        else:
            x[0, 0, [0, 128, 256, 384]] = one
        cs = np.zeros((1, 64), np.float32)
        cs[:, :32] = 1
        q = torch.zeros(1, 1, 4, 128, dtype=torch.int16, device="cuda")
        qsa.qsa_index_q_prep(q, G.dev_bits(x), G.dev(cs), G.dev(np.array([1], np.int32)),
                             torch.zeros(128, dtype=torch.int16, device="cuda"), 1e-6, dt=c["dt"])
        qh = G.host_bits(q)
        if "out_all" in c:
            assert np.all(qh == H(c["out_all"])), c
        else:
            assert np.all(qh[0, 0, :, 0] == H(c["out0"])), c
            assert np.all((qh[0, 0, :, 1:] & 0x7FFF) == 0)


# ------------------------------------------------------------------------------ edges ---

def _small(S, ctx, dt="bf16", B=None, seed=99, numBlocks=None, pages=None):
    rng = np.random.default_rng(seed)
    ctx = np.asarray(ctx, np.int32)
    B = len(ctx) if B is None else B
    x = W.to_bits(rng.standard_normal((B, S, 640), dtype=np.float32), dt)
    wQ = W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt)
    wK = W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt)
    nb = (S + 3) // 4 if numBlocks is None else numBlocks
    m = max(1, (S + 127) // 128)
    numPages = B * m if pages is None else pages
    pt = np.stack([rng.permutation(numPages)[:B * m].reshape(B, m),
                   rng.permutation(numPages)[:B * m].reshape(B, m) + numPages], 1)
    return W.Workload(f"edge_S{S}", dt, x, W.cos_sin_table(max(S, 4 * nb), 1e4), ctx, wQ, wK,
                      1e-6, nb, 0, nb, 0, W.PoolSpec(numPages, pt.astype(np.int32)))


@pytest.mark.parametrize("S,ctx", [(1, [1]), (3, [2]), (4, [4]), (5, [5, 0, 3]), (61, [61]),
                                   (61, [60, 57, 1, 0]), (130, [130, 129, 128, 127]),
                                   (257, [257, 4, 255])])
@pytest.mark.parametrize("fused", [False, True])
def test_ragged_and_tiny(qsa, O, S, ctx, fused):
    wl = _small(S, ctx)
    got = run_gpu(qsa, wl, fused=fused)
    check_against_oracle(O, wl, got)


def test_kbar_stride_larger_than_blocks(qsa, O):
    """numBlocks > ceilDiv(S, 4): rows past the range keep their content."""
    wl = _small(64, [64, 33], numBlocks=40)
    wl.blockEnd = 16
    check_against_oracle(O, wl, run_gpu(qsa, wl))


def test_out_of_contract_device_values(qsa, O):
    """Lengths beyond S or negative, and page-table entries that are -1, negative or too large,
    never fault: lengths clamp (K1a) or make blocks invalid, bad entries skip the write."""
    wl = _small(256, [300, -7, 129, 256])
    pt = wl.pool.pageTable
    pt[0, 0, 1] = -1
    pt[2, 1, 0] = -5
    pt[3, 1, 1] = 2 * wl.pool.numPages + 3
    pt[2, 0, 1] = 2 ** 31 - 1
    check_against_oracle(O, wl, run_gpu(qsa, wl))


def test_empty_calls_touch_nothing(qsa):
    x = torch.zeros(0, 16, 640, dtype=torch.int16, device="cuda")
    cs = torch.zeros(16, 64, device="cuda")
    ctx = torch.zeros(0, dtype=torch.int32, device="cuda")
    w = torch.zeros(128, dtype=torch.int16, device="cuda")
    q = torch.zeros(0, 16, 4, 128, dtype=torch.int16, device="cuda")
    qsa.qsa_index_q_prep(q, x, cs, ctx, w, 1e-6, dt="bf16")
    kb = torch.full((1, 4, 128), 7, dtype=torch.int16, device="cuda")
    x1 = torch.zeros(1, 16, 640, dtype=torch.int16, device="cuda")
    ctx1 = torch.full((1,), 16, dtype=torch.int32, device="cuda")
    qsa.qsa_index_k_compress(kb, x1, cs, ctx1, w, 1e-6, 4, 2, 2, 0, dt="bf16")
    torch.cuda.synchronize()
    assert bool((kb == 7).all())


def test_validation_rejects_before_launch(qsa):
    x = torch.zeros(1, 16, 640, dtype=torch.int16, device="cuda")
    cs = torch.zeros(16, 64, device="cuda")
    ctx = torch.full((1,), 16, dtype=torch.int32, device="cuda")
    w = torch.zeros(128, dtype=torch.int16, device="cuda")
    kb = torch.full((1, 4, 128), 7, dtype=torch.int16, device="cuda")
    with pytest.raises(qsa.QsaError) as e:
        qsa.qsa_index_k_compress(kb, x, cs[:12], ctx, w, 1e-6, 4, 0, 4, 0, dt="bf16")
    assert e.value.code == qsa.QSA_E_INVALID and "maxPositions" in str(e.value)
    with pytest.raises(qsa.QsaError) as e:
        qsa.qsa_index_k_compress(kb, x, cs, ctx, w, 1e-6, 4, 0, 5, 0, dt="bf16")
    assert e.value.code == qsa.QSA_E_INVALID
    with pytest.raises(qsa.QsaError) as e:
        qsa.qsa_index_k_compress(kb, x, cs, ctx, w, float("nan"), 4, 0, 4, 0, dt="bf16")
    assert e.value.code == qsa.QSA_E_INVALID
    with pytest.raises(ValueError):   # the binding refuses a buffer smaller than the grid
        qsa.qsa_index_k_compress(kb[:, :2], x, cs, ctx, w, 1e-6, 4, 0, 4, 0, dt="bf16")
    torch.cuda.synchronize()
    assert bool((kb == 7).all())


def test_determinism_and_padding_never_read(qsa):
    """Two runs give identical bytes; refilling padding rows (NaN) with random bits changes
    nothing."""
    wl = W.config2("bf16", S=1024)
    a = run_gpu(qsa, wl, fused=True)
    b = run_gpu(qsa, wl, fused=True)
    rng = np.random.default_rng(5)
    L = np.clip(wl.ctx, 0, wl.S)
    pad = np.arange(wl.S)[None, :] >= L[:, None]
    wl.indexQk[pad] = rng.integers(0, 65536, (int(pad.sum()), 640)).astype(np.uint16)
    c = run_gpu(qsa, wl, fused=False)
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)
