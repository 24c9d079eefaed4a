"""Pins of the CPU oracle: checks that tie it to facts other than itself.

Each ``check_*`` takes an oracle object (``oracle.ref.Oracle``) and raises AssertionError when
the oracle breaks the fact it pins.  ``test_oracle_pins.py`` runs them on the real oracle;
``test_oracle_mutants.py`` runs them on deliberately broken builds of it and requires that each
break is caught.  The facts come from the "Qsa Indexer Kernels" page (TensorRT-Edge-LLM C++ API
documentation) and from mathematics:
  - hand-worked values (tests/golden/hand_worked.json),
  - closed forms (quarter-turn rope, w = -1, all-ones heads),
  - invariants (power-of-two scale invariance, padding never read, sub-range union, ranges
    mode = separate calls, thread-count independence, K1a/K1b agreement on constant blocks),
  - an independent numpy re-derivation on the tiny prefill workload,
  - the pool round trip through an independent tensor view of the addressing contract.
"""
import json
import os

import numpy as np

from tests import numpy_model as nm

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")))
H = lambda s: int(s, 16)  # noqa: E731


def _zero_row(B=1, S=4):
    return np.zeros((B, S, 640), np.uint16)


def _id_table(n):
    """cosSin rows with cos = 1, sin = 0 (rope is the identity)."""
    cs = np.zeros((n, 64), np.float32)
    cs[:, :32] = 1.0
    return cs


def _rand_bits(rng, shape, dt, scale=1.0):
    from sparse_attention_indexer_qsa_amd.workloads import to_bits
    return to_bits(scale * rng.standard_normal(shape, dtype=np.float32), dt)


def _is_zero(bits):
    return np.all((bits & 0x7FFF) == 0)


# ------------------------------------------------------------------------ hand-worked ----

def check_block_mean_order(O):
    for c in GOLDEN["block_mean_order"]["cases"]:
        x = _zero_row()
        x[0, :, 512] = [H(v) for v in c["k"]]
        cs = _id_table(4)
        _, dbg = O.k_compress(x, cs, np.array([4]), np.zeros(128, np.uint16), 1e-6, 1, 0, 1, 0,
                              c["dt"], debug=True)
        assert dbg["mT"][0, 0, 0] == H(c["mT"]), (c, hex(dbg["mT"][0, 0, 0]))


def check_kbar_order_end_to_end(O):
    means = {c["dt"]: c for c in GOLDEN["block_mean_order"]["cases"] if c["mT"] != c["k"][0]}
    for c in GOLDEN["kbar_order_end_to_end"]["cases"]:
        x = _zero_row()
        x[0, :, 512] = [H(v) for v in means[c["dt"]]["k"]]
        x[0, :, 513] = H(c["d1"])
        kb = O.k_compress(x, _id_table(4), np.array([4]), np.zeros(128, np.uint16), 1e-6, 1,
                          0, 1, 0, c["dt"])
        assert [int(v) for v in kb[0, 0, :2]] == [H(v) for v in c["kbar01"]], c
        assert _is_zero(kb[0, 0, 2:])
        # the fixture discriminates: an input whose fixed-order mean is the pairwise mean
        # gives the other answer
        x2 = x.copy()
        x2[0, :, 512] = H(means[c["dt"]]["mT_if_pairwise"])   # four equal rows: mean exact
        kb2 = O.k_compress(x2, _id_table(4), np.array([4]), np.zeros(128, np.uint16), 1e-6, 1,
                           0, 1, 0, c["dt"])
        assert [int(v) for v in kb2[0, 0, :2]] == [H(v) for v in c["kbar01_if_pairwise"]], c


def check_norm_closed_forms(O):
    for c in GOLDEN["norm_closed_forms"]["cases"]:
        one = 0x3F80 if c["dt"] == "bf16" else 0x3C00
        x = _zero_row(1, 1)
        if "out_all" in c:
            x[0, 0, :512] = one
        else:
            x[0, 0, [0, 128, 256, 384]] = one
        q = O.q_prep(x, _id_table(1), np.array([1]), np.zeros(128, np.uint16), 1e-6, c["dt"])
        if "out_all" in c:
            assert np.all(q == H(c["out_all"])), c
        else:
            assert np.all(q[0, 0, :, 0] == H(c["out0"])), (c, q[0, 0, :, 0])
            assert _is_zero(q[0, 0, :, 1:])


def check_gamma_minus_one_gives_zeros(O):
    rng = np.random.default_rng(7)
    for dt in ("bf16", "f16"):
        minus1 = 0xBF80 if dt == "bf16" else 0xBC00
        x = _rand_bits(rng, (1, 8, 640), dt)
        from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
        cs = cos_sin_table(32, 1e4)
        q = O.q_prep(x, cs, np.array([8]), np.full(128, minus1, np.uint16), 1e-6, dt)
        assert _is_zero(q)
        kb = O.k_compress(x, cs, np.array([8]), np.full(128, minus1, np.uint16), 1e-6, 2, 0, 2,
                          0, dt)
        assert _is_zero(kb)


# ------------------------------------------------------------------------- invariants ----

def check_scale_invariance(O):
    """With eps = 0, scaling x by 2^k scales meanSq by 4^k and rsqrt by 2^-k exactly, so the
    output bits do not change (no underflow or overflow in the chosen range)."""
    rng = np.random.default_rng(11)
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    cs = cos_sin_table(16, 1e4)
    for dt in ("bf16", "f16"):
        base = rng.standard_normal((1, 16, 640), dtype=np.float32)
        w = _rand_bits(rng, 128, dt, 0.1)
        ref_q = O.q_prep(_bits(base, dt), cs, np.array([16]), w, 0.0, dt)
        ref_k = O.k_compress(_bits(base, dt), cs, np.array([16]), w, 0.0, 4, 0, 4, 0, dt)
        for k in (-3, 2, 5):
            xs = _bits(base * np.float32(2.0 ** k), dt)
            assert np.array_equal(O.q_prep(xs, cs, np.array([16]), w, 0.0, dt), ref_q), (dt, k)
            assert np.array_equal(O.k_compress(xs, cs, np.array([16]), w, 0.0, 4, 0, 4, 0, dt),
                                  ref_k), (dt, k)


def _bits(values, dt):
    from sparse_attention_indexer_qsa_amd.workloads import to_bits
    return to_bits(values, dt)


def check_rope_quarter_turn(O):
    """cos = 0, sin = 1 is an exact quarter turn of each pair (i, i+32): o_i = -y_{i+32},
    o_{i+32} = y_i; dims 64..127 are untouched; compared with the identity row cos=1, sin=0."""
    rng = np.random.default_rng(13)
    for dt in ("bf16", "f16"):
        x = _rand_bits(rng, (1, 2, 640), dt)
        w = _rand_bits(rng, 128, dt, 0.1)
        ident = _id_table(2)
        turn = np.zeros((2, 64), np.float32)
        turn[:, 32:] = 1.0
        _, d0 = O.q_prep(x, ident, np.array([2]), w, 1e-6, dt, debug=True)
        _, d1 = O.q_prep(x, turn, np.array([2]), w, 1e-6, dt, debug=True)
        y, o = d0["preCast"], d1["preCast"]
        assert np.array_equal(o[..., :32], -y[..., 32:64])
        assert np.array_equal(o[..., 32:64], y[..., :32])
        assert np.array_equal(o[..., 64:], y[..., 64:])


def check_rope_position_and_pair_norm(O):
    """Token t uses cosSin row t (a one-row call on the table shifted to start at t gives the
    same bits), and each rope pair keeps its norm to binary32 rounding."""
    rng = np.random.default_rng(17)
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    cs = cos_sin_table(64, 1e4)
    dt = "bf16"
    x = _rand_bits(rng, (1, 64, 640), dt)
    w = _rand_bits(rng, 128, dt, 0.1)
    q, dq = O.q_prep(x, cs, np.array([64]), w, 1e-6, dt, debug=True)
    _, did = O.q_prep(x, _id_table(64), np.array([64]), w, 1e-6, dt, debug=True)
    for t in (1, 17, 63):
        qt = O.q_prep(x[:, t:t + 1], cs[t:t + 1], np.array([1]), w, 1e-6, dt)
        assert np.array_equal(qt[0, 0], q[0, t])
    y, o = did["preCast"].astype(np.float64), dq["preCast"].astype(np.float64)
    ny = y[..., :32] ** 2 + y[..., 32:64] ** 2
    no = o[..., :32] ** 2 + o[..., 32:64] ** 2
    assert np.allclose(no, ny, rtol=2e-6, atol=1e-30)
    assert not np.array_equal(o[..., :64], y[..., :64])


def check_padding_zero_and_never_read(O):
    """Rows t >= ctx (and blocks that are not complete inside the rows) are +0 and their input
    is never read: NaN or other garbage there changes no output bit."""
    rng = np.random.default_rng(19)
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    cs = cos_sin_table(32, 1e4)
    for dt in ("bf16", "f16"):
        nan = 0x7FC0 if dt == "bf16" else 0x7E00
        x = _rand_bits(rng, (4, 32, 640), dt)
        ctx = np.array([0, 13, 32, 30], np.int32)
        w = _rand_bits(rng, 128, dt, 0.1)
        xa, xb = x.copy(), x.copy()
        for b, c in enumerate(ctx):
            xa[b, c:] = nan
            xb[b, c:] = rng.integers(0, 65536, (32 - c, 640)).astype(np.uint16)
        qa = O.q_prep(xa, cs, ctx, w, 1e-6, dt)
        qb = O.q_prep(xb, cs, ctx, w, 1e-6, dt)
        assert np.array_equal(qa, qb)
        for b, c in enumerate(ctx):
            assert np.all(qa[b, c:] == 0)
            assert all(not _is_zero(qa[b, t]) for t in range(c))
        ka = O.k_compress(xa, cs, ctx, w, 1e-6, 8, 0, 8, 0, dt)
        kb = O.k_compress(xb, cs, ctx, w, 1e-6, 8, 0, 8, 0, dt)
        assert np.array_equal(ka, kb)
        for b, c in enumerate(ctx):
            nvalid = c // 4
            assert np.all(ka[b, nvalid:] == 0)
            assert all(not _is_zero(ka[b, g]) for g in range(nvalid))
        # lengths outside [0, S] are clamped for K1a
        q_over = O.q_prep(x, cs, np.array([40, -5, 32, 32]), w, 1e-6, dt)
        q_ref = O.q_prep(x, cs, np.array([32, 0, 32, 32]), w, 1e-6, dt)
        assert np.array_equal(q_over, q_ref)


def check_block_validity_rule(O):
    """launchQsaIndexKCompress: valid iff 4g+3 < ctx and 4g >= pastLen (and the block's rows
    lie inside the S provided rows); the raw key of token 4g+j is row 4g+j-pastLen."""
    rng = np.random.default_rng(23)
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    dt = "bf16"
    cs = cos_sin_table(64, 1e4)
    w = _rand_bits(rng, 128, dt, 0.1)
    full = _rand_bits(rng, (1, 64, 640), dt)
    ref = O.k_compress(full, cs, np.array([64]), w, 1e-6, 16, 0, 16, 0, dt)
    # (ctx, pastLen, S rows given, expected valid blocks among [0, 16))
    cases = [(64, 0, 64, set(range(16))), (63, 0, 64, set(range(15))),
             (64, 8, 56, set(range(2, 16))), (64, 9, 55, set(range(3, 16))),
             (40, 8, 20, set(range(2, 7))), (64, 12, 8, {3, 4}), (3, 0, 64, set())]
    for ctx, p, S, valid in cases:
        rows = full[:, p:p + S]
        kb = O.k_compress(rows, cs, np.array([ctx]), w, 1e-6, 16, 0, 16, p, dt)
        for g in range(16):
            if g in valid:
                assert np.array_equal(kb[0, g], ref[0, g]), (ctx, p, S, g)
            else:
                assert np.all(kb[0, g] == 0), (ctx, p, S, g)
    # rows outside [blockBegin, blockEnd) are untouched
    init = np.full((1, 16, 128), 0x1234, np.uint16)
    kb = O.k_compress(full, cs, np.array([64]), w, 1e-6, 16, 5, 9, 0, dt, kbar=init)
    assert np.all(kb[0, :5] == 0x1234) and np.all(kb[0, 9:] == 0x1234)
    assert np.array_equal(kb[0, 5:9], ref[0, 5:9])


def check_k1a_k1b_agree_on_constant_blocks(O):
    """A block of four identical key rows k has mean exactly k, so its kbar equals K1a's
    numerics applied to k with the K gamma at position 4g."""
    rng = np.random.default_rng(29)
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    cs = cos_sin_table(64, 1e4)
    for dt in ("bf16", "f16"):
        k = _rand_bits(rng, (16, 128), dt)
        w = _rand_bits(rng, 128, dt, 0.1)
        x = np.zeros((1, 64, 640), np.uint16)
        x[0, :, 512:] = np.repeat(k, 4, axis=0)
        kb = O.k_compress(x, cs, np.array([64]), w, 1e-6, 16, 0, 16, 0, dt)
        xq = np.zeros((1, 64, 640), np.uint16)
        xq[0, :, :128] = np.repeat(k, 4, axis=0)
        q = O.q_prep(xq, cs, np.array([64]), w, 1e-6, dt)
        assert np.array_equal(kb[0], q[0, ::4, 0]), dt


def check_subrange_union_equals_full(O):
    """The (blockBegin, blockEnd, pastLen) triplet compresses a sub-range of a longer sequence;
    sub-range calls that cover [0, numBlocks) reproduce one full call bit for bit."""
    rng = np.random.default_rng(31)
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    dt = "f16"
    S, nb = 256, 64
    cs = cos_sin_table(S, 1e4)
    x = _rand_bits(rng, (3, S, 640), dt)
    ctx = np.array([256, 201, 77], np.int32)
    w = _rand_bits(rng, 128, dt, 0.1)
    full = O.k_compress(x, cs, ctx, w, 1e-6, nb, 0, nb, 0, dt)
    acc = np.full((3, nb, 128), 0x5555, np.uint16)
    for bB, bE, p in [(0, 9, 0), (9, 30, 36), (30, 41, 119), (41, 64, 164)]:
        acc = O.k_compress(np.ascontiguousarray(x[:, p:]), cs, ctx, w, 1e-6, nb, bB, bE, p, dt,
                           kbar=acc)
    assert np.array_equal(acc, full)


def check_ranges_mode(O):
    """Per-sequence triplets: equal entries reproduce scalar mode; distinct entries reproduce
    separate one-sequence calls."""
    rng = np.random.default_rng(37)
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    dt = "bf16"
    S, nb, B = 8, 40, 5
    cs = cos_sin_table(4 * nb, 1e4)
    x = _rand_bits(rng, (B, S, 640), dt)
    w = _rand_bits(rng, 128, dt, 0.1)
    past = np.array([8, 12, 100, 151, 4], np.int32)
    ctx = past + np.array([8, 4, 7, 6, 1], np.int32)
    bB = past >> 2
    bE = (ctx + 3) >> 2
    span = int((bE - bB).max())
    r = O.k_compress(x, cs, ctx, w, 1e-6, nb, 0, 0, 0, dt, ranges=(past, bB, bE, span))
    for b in range(B):
        one = O.k_compress(x[b:b + 1], cs, ctx[b:b + 1], w, 1e-6, nb, int(bB[b]), int(bE[b]),
                           int(past[b]), dt)
        assert np.array_equal(r[b], one[0]), b
    same = O.k_compress(x, cs, np.full(B, 20, np.int32), w, 1e-6, nb, 0, 0, 0, dt,
                        ranges=(np.full(B, 8), np.full(B, 2), np.full(B, 5), 3))
    scal = O.k_compress(x, cs, np.full(B, 20, np.int32), w, 1e-6, nb, 2, 5, 8, dt)
    assert np.array_equal(same, scal)


def check_thread_count_independence(O):
    from sparse_attention_indexer_qsa_amd import workloads
    wl = workloads.config2("bf16", S=256)
    outs = []
    for n in (1, 3, 8):
        O.set_threads(n)
        q = O.q_prep(wl.indexQk, wl.cosSin, wl.ctx, wl.wQ, wl.eps, wl.dt)
        k = O.k_compress(wl.indexQk, wl.cosSin, wl.ctx, wl.wK, wl.eps, wl.numBlocks, 0,
                         wl.numBlocks, 0, wl.dt)
        outs.append((q, k))
    O.set_threads(8)
    for q, k in outs[1:]:
        assert np.array_equal(q, outs[0][0]) and np.array_equal(k, outs[0][1])


def check_numpy_rederivation(O):
    """An independent numpy binary32 re-derivation of the definitions (tests/numpy_model.py)
    matches the oracle bit for bit on the tiny prefill workload and a batched fp16 one."""
    from sparse_attention_indexer_qsa_amd import workloads
    for wl in (workloads.config1(), workloads.config2("f16", S=128)):
        q = O.q_prep(wl.indexQk, wl.cosSin, wl.ctx, wl.wQ, wl.eps, wl.dt)
        qn = nm.q_prep(wl.indexQk, wl.cosSin, wl.ctx, wl.wQ, wl.eps, wl.dt)
        assert np.array_equal(q, qn), wl.name
        k = O.k_compress(wl.indexQk, wl.cosSin, wl.ctx, wl.wK, wl.eps, wl.numBlocks, 0,
                         wl.numBlocks, 0, wl.dt)
        kn = nm.k_compress(wl.indexQk, wl.cosSin, wl.ctx, wl.wK, wl.eps, wl.numBlocks, wl.dt)
        assert np.array_equal(k, kn), wl.name


# ---------------------------------------------------------------------------- persist ----

def _pool(numPages, H=2, D=384):
    return np.full((2 * numPages, 128, H, D), 0xA5A5, np.uint16)


def check_pool_round_trip(O):
    """QsaIndexerPoolState addressing, checked through an independent view of the pool as a
    [2*numPages, 128, H, D] tensor: every written cell reads back the expected bits (K-tail =
    the raw key bits, V-tail = the dense kbar row), unused entries and out-of-range slots skip,
    and nothing else changes."""
    from oracle.ref import Pool
    rng = np.random.default_rng(41)
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    dt = "bf16"
    B, S, numPages, m = 3, 300, 12, 4
    nb = (S + 3) // 4
    cs = cos_sin_table(S, 1e4)
    x = _rand_bits(rng, (B, S, 640), dt)
    w = _rand_bits(rng, 128, dt, 0.1)
    ctx = np.array([300, 257, 130], np.int32)
    pt = np.stack([rng.permutation(numPages)[:B * m].reshape(B, m),
                   rng.permutation(numPages)[:B * m].reshape(B, m) + numPages], 1).astype(np.int32)
    pt[1, 0, 2] = -1          # K tail page of sequence 1's tokens 256.. unused
    pt[2, 1, 0] = -1          # V page of sequence 2's first 32 blocks unused
    pt[0, 1, 1] = 2 * numPages + 5   # out of range id: skipped
    data = _pool(numPages)
    pool = Pool(data, pt, numPages, 256)
    kb = O.k_compress(x, cs, ctx, w, 1e-6, nb, 0, nb, 0, dt, pool=pool)
    O.persist(pool, x, None, ctx, nb, 0, nb, 0)
    view = data.reshape(2 * numPages, 128, 2, 384)
    expect = np.full_like(data, 0xA5A5)
    ev = expect.reshape(view.shape)
    for b in range(B):
        c = int(ctx[b])
        for t in range(c - c % 4, c):
            pid = pt[b, 0, t // 128]
            if pid >= 0:
                ev[pid, t % 128, 0, 256:384] = x[b, t, 512:640]
        for g in range(c // 4):
            pid = pt[b, 1, (4 * g) // 128]
            if 0 <= pid < 2 * numPages:
                ev[pid, (4 * g) % 128, 0, 256:384] = kb[b, g]
    assert np.array_equal(view, ev)
    # persist with the dense kbar writes the same V-tails as the fused pool write
    data2 = _pool(numPages)
    pool2 = Pool(data2, pt, numPages, 256)
    O.persist(pool2, x, kb, ctx, nb, 0, nb, 0)
    assert np.array_equal(data2, data)


def check_tail_rule_with_past(O):
    """Raw-K tails: tokens [max(pastLen, ctx - ctx%4), ctx) inside the provided rows, copied
    bit-unmodified; none when ctx % 4 == 0."""
    from oracle.ref import Pool
    rng = np.random.default_rng(43)
    numPages, B, S = 8, 4, 4
    x = rng.integers(0, 65536, (B, S, 640)).astype(np.uint16)
    past = np.array([10, 13, 16, 127], np.int32)
    new = np.array([3, 4, 4, 2], np.int32)
    ctx = past + new
    pt = np.stack([np.arange(B * 2).reshape(B, 2), np.arange(B * 2).reshape(B, 2) + numPages],
                  1).astype(np.int32)
    data = _pool(numPages)
    pool = Pool(data, pt, numPages, 256)
    O.persist(pool, x, None, ctx, 40, 0, 0, 0, ranges=(past, past >> 2, ctx >> 2, 1))
    view = data.reshape(2 * numPages, 128, 2, 384)
    written = {}
    for b in range(B):
        c, p = int(ctx[b]), int(past[b])
        for t in range(max(p, c - c % 4), c):
            written[(int(pt[b, 0, t // 128]), t % 128)] = x[b, t - p, 512:]
    # 10+3=13: token 12; 13+4=17: token 16; 16+4=20: none; 127+2=129: token 128
    assert len(written) == 3
    for (pid, row), bits in written.items():
        assert np.array_equal(view[pid, row, 0, 256:], bits)
    assert np.count_nonzero(data != 0xA5A5) == np.count_nonzero(
        np.stack(list(written.values())) != 0xA5A5)


# ------------------------------------------------------------------- decode pre-pass ----

def _history(rng, dt, lengths, numPages=None):
    """Random full histories [B, Lmax, 640], gammas, cosSin table and a page table with
    unique ids (V ids offset by numPages)."""
    from sparse_attention_indexer_qsa_amd.workloads import cos_sin_table
    B, Lmax = len(lengths), int(max(lengths))
    m = (Lmax + 127) // 128
    numPages = B * m if numPages is None else numPages
    x = _rand_bits(rng, (B, Lmax, 640), dt)
    wQ, wK = _rand_bits(rng, 128, dt, 0.1), _rand_bits(rng, 128, dt, 0.1)
    pt = np.stack([rng.permutation(numPages)[:B * m].reshape(B, m),
                   rng.permutation(numPages)[:B * m].reshape(B, m) + numPages], 1).astype(np.int32)
    return x, wQ, wK, cos_sin_table(Lmax + 8, 1e4), pt, numPages


def check_pre_decode_equals_prefill(O):
    """launchQsaIndexerPreDecode: the raw key is stored bit-unmodified so that decode-time
    compression is bit-identical to prefill K1b.  Prefill of a prefix, then decode steps of 1..4
    new tokens, must leave in the V-tails exactly the kbar rows of one prefill over the whole
    history, and give the same q rows as K1a over the whole history."""
    from oracle.ref import Pool
    rng = np.random.default_rng(53)
    for dt in ("bf16", "f16"):
        L = np.array([300, 257, 131, 9], np.int32)
        x, wQ, wK, cs, pt, numPages = _history(rng, dt, L)
        B, Lmax = x.shape[:2]
        nb = (Lmax + 3) // 4
        kb_full = O.k_compress(x, cs, L, wK, 1e-6, nb, 0, nb, 0, dt)
        q_full = O.q_prep(x, cs, L, wQ, 1e-6, dt)
        data = np.full((2 * numPages, 128, 2, 384), 0xA5A5, np.uint16)
        pool = Pool(data, pt, numPages, 256)
        p0 = np.array([37, 128, 1, 0], np.int32)
        Spre = int(p0.max())
        O.k_compress(np.ascontiguousarray(x[:, :Spre]), cs, p0, wK, 1e-6, nb, 0, nb, 0, dt,
                     pool=pool)
        O.persist(pool, np.ascontiguousarray(x[:, :Spre]), None, p0, nb, 0, nb, 0)
        cur = p0.copy()
        single = dt == "f16"   # the page's form: one new token per step, newLens = NULL
        while np.any(cur < L):
            n = np.minimum(1 if single else rng.integers(1, 5, B), L - cur).astype(np.int32)
            rows = np.zeros((B, 4, 640), np.uint16)
            for b in range(B):
                rows[b, :n[b]] = x[b, cur[b]:cur[b] + n[b]]
            ctx = (cur + n).astype(np.int32)
            if single:
                live = n > 0
                q = O.pre_decode(rows[live], cs, ctx[live], None, wQ, wK, 1e-6,
                                 Pool(data, pt[live], numPages, 256), dt)
                qq = np.zeros((B, 4, 4, 128), np.uint16)
                qq[live] = q
                q = qq
            else:
                q = O.pre_decode(rows, cs, ctx, n, wQ, wK, 1e-6, pool, dt)
            for b in range(B):
                assert np.array_equal(q[b, :n[b]], q_full[b, cur[b]:ctx[b]]), (dt, b, cur[b])
                assert np.all(q[b, n[b]:] == 0)
            cur = ctx
        view = data.reshape(2 * numPages, 128, 2, 384)
        for b in range(B):
            for g in range(int(L[b]) // 4):
                pid = pt[b, 1, (4 * g) // 128]
                assert np.array_equal(view[pid, (4 * g) % 128, 0, 256:], kb_full[b, g]), (dt, b, g)


def check_pre_decode_guards(O):
    """Lengths <= 0 write zero q rows and touch no pool cell; a K-tail page marked unused makes
    the completed block uncomputable (no V-tail write) while its q rows are still produced; the
    default of one new token equals newLens = 1."""
    from oracle.ref import Pool
    rng = np.random.default_rng(59)
    dt = "bf16"
    L = np.array([8, 12, 40], np.int32)
    x, wQ, wK, cs, pt, numPages = _history(rng, dt, L)
    rows = np.ascontiguousarray(x[:, :4])
    data = np.full((2 * numPages, 128, 2, 384), 0xA5A5, np.uint16)
    q = O.pre_decode(rows, cs, np.array([0, -3, 0], np.int32), None, wQ, wK, 1e-6,
                     Pool(data, pt, numPages, 256), dt)
    assert np.all(q == 0) and np.all(data == 0xA5A5)
    ctx = np.array([4, 8, 12], np.int32)            # each completes a block
    pt2 = pt.copy()
    pt2[1, 0, 0] = -1                              # sequence 1: earlier keys not in the pool
    q1 = O.pre_decode(rows, cs, ctx, None, wQ, wK, 1e-6, Pool(data, pt2, numPages, 256), dt)
    view = data.reshape(2 * numPages, 128, 2, 384)
    assert np.all(view[pt2[1, 1, 0], 4, 0, 256:] == 0xA5A5)
    assert not np.all(q1[1, 0] == 0)
    # exactly two cells changed: the V-tails of sequences 0 and 2 (no K-tail: blocks complete)
    rows_written = np.unique(np.argwhere(view != 0xA5A5)[:, :2], axis=0)
    assert len(rows_written) == 2, rows_written
    data2 = np.full_like(data, 0xA5A5)
    q2 = O.pre_decode(rows, cs, ctx, np.ones(3, np.int32), wQ, wK, 1e-6,
                      Pool(data2, pt2, numPages, 256), dt)
    assert np.array_equal(q1, q2) and np.array_equal(data, data2)


# ---------------------------------------------------------------------- block scores ----

NEG_FLT_MAX_BITS = 0xFF7FFFFF


def _bf16(x):
    from sparse_attention_indexer_qsa_amd.workloads import to_bits
    return to_bits(np.asarray(x, np.float32), "bf16")


def check_score_scale(O):
    """The scale 1/sqrtf(128) is the binary32 value numpy computes with float32 sqrt and
    divide."""
    assert np.float32(O.score_scale()) == np.float32(1) / np.sqrt(np.float32(128))


def check_scores_closed_forms(O):
    """launchQsaIndexScores: ReLU per head (not after the sum), heads summed, scale after the
    sum.  One-hot q heads against a one-hot kbar row give exact head dots (a_h * b)."""
    c = np.float32(1) / np.sqrt(np.float32(128))
    for dots, expect_sum in [((0.5, 1.0, -2.0, -0.5), 1.5), ((3.0, 5.0, -7.0, 1.0), 9.0),
                             ((-1.0, -2.0, -3.0, -4.0), 0.0)]:
        q = np.zeros((1, 4, 4, 128), np.uint16)
        kb = np.zeros((1, 1, 128), np.uint16)
        for h, a in enumerate(dots):
            q[0, 3, h, 7] = _bf16([a])[0]          # token 3 sees block 0
        kb[0, 0, 7] = _bf16([1.0])[0]
        lg = O.scores(q, kb, np.array([4]), 3, 1, "bf16")
        assert lg[0, 0] == np.float32(expect_sum) * c, (dots, lg[0, 0])
    # scale after the sum: head dots 2.40625 and 3.765625 (both bf16 values) round differently
    # when scaled before summing: c*(x+y) = 0.5455218, c*x + c*y = 0.54552186
    x, y = np.float32(2.40625), np.float32(3.765625)
    assert np.float32(c * np.float32(x + y)) != np.float32(np.float32(c * x) + np.float32(c * y))
    q = np.zeros((1, 4, 4, 128), np.uint16)
    kb = np.zeros((1, 1, 128), np.uint16)
    q[0, 3, 0, 5], q[0, 3, 1, 9] = _bf16([x])[0], _bf16([y])[0]
    kb[0, 0, 5] = kb[0, 0, 9] = _bf16([1.0])[0]
    lg = O.scores(q, kb, np.array([4]), 3, 1, "bf16")
    assert lg[0, 0] == np.float32(c * np.float32(x + y))


def check_scores_mask_and_padding(O):
    """Invisible blocks (g >= (t+1)/4) and padded rows (t >= ctx, ctx <= 0) are exactly -FLT_MAX;
    padded q rows and invisible kbar rows are never read (NaN there changes nothing)."""
    rng = np.random.default_rng(67)
    B, S = 3, 40
    nb = S // 4
    q = _bf16(rng.standard_normal((B, S, 4, 128)))
    kb = _bf16(rng.standard_normal((B, nb, 128)))
    ctx = np.array([40, 17, 0], np.int32)
    lg = O.scores(q, kb, ctx, 0, B * S, "bf16").reshape(B, S, nb)
    bits = lg.view(np.uint32)
    for b in range(B):
        for t in range(S):
            nvis = (t + 1) // 4 if t < ctx[b] else 0
            assert np.all(bits[b, t, nvis:] == NEG_FLT_MAX_BITS), (b, t)
            assert np.all(np.isfinite(lg[b, t, :nvis])) and np.all(lg[b, t, :nvis] >= 0)
    q2, kb2 = q.copy(), kb.copy()
    q2[1, 17:] = 0x7FC0
    q2[2] = 0x7FC0
    kb2[1, 4:] = 0x7FC0        # t < 17 sees blocks < 4 only
    assert np.array_equal(O.scores(q2, kb2, ctx, 0, B * S, "bf16").view(np.uint32),
                          bits.reshape(B * S, nb))


def check_scores_chunks_and_permutation(O):
    """Row chunks (rowStart, numRows) are slices of the full matrix; permuting the 128 dims of
    q and kbar together changes no logit (each head dot is exact before its one rounding)."""
    rng = np.random.default_rng(71)
    for dt in ("bf16", "f16"):
        B, S = 2, 64
        nb = S // 4
        from sparse_attention_indexer_qsa_amd.workloads import to_bits
        q = to_bits(rng.standard_normal((B, S, 4, 128), dtype=np.float32), dt)
        kb = to_bits(rng.standard_normal((B, nb, 128), dtype=np.float32), dt)
        ctx = np.array([64, 50], np.int32)
        full = O.scores(q, kb, ctx, 0, B * S, dt)
        parts = [O.scores(q, kb, ctx, r0, n, dt) for r0, n in ((0, 37), (37, 60), (97, 31))]
        assert np.array_equal(np.concatenate(parts).view(np.uint32), full.view(np.uint32))
        perm = rng.permutation(128)
        qp = np.ascontiguousarray(q[..., perm])
        kp = np.ascontiguousarray(kb[..., perm])
        assert np.array_equal(O.scores(qp, kp, ctx, 0, B * S, dt).view(np.uint32),
                              full.view(np.uint32))


def check_scores_numpy(O):
    """An independent numpy derivation (float64 matmul of the widened values, one rounding to
    float32 per head, ReLU, ascending head sum, scale) matches bit for bit."""
    rng = np.random.default_rng(73)
    dt = "bf16"
    B, S = 2, 48
    nb = S // 4
    q = _bf16(rng.standard_normal((B, S, 4, 128)))
    kb = _bf16(rng.standard_normal((B, nb, 128)))
    ctx = np.array([48, 30], np.int32)
    got = O.scores(q, kb, ctx, 0, B * S, dt).reshape(B, S, nb)
    qf, kf = nm.widen(q, dt).astype(np.float64), nm.widen(kb, dt).astype(np.float64)
    dots = np.einsum("bthd,bgd->bthg", qf, kf).astype(np.float32)
    r = np.maximum(dots, np.float32(0))
    ssum = ((r[:, :, 0] + r[:, :, 1]) + r[:, :, 2]) + r[:, :, 3]
    ref = np.float32(1) / np.sqrt(np.float32(128)) * ssum
    t = np.arange(S)[:, None]
    g = np.arange(nb)[None, :]
    vis = (g < (t + 1) // 4)[None] & (t < ctx[:, None, None])
    ref = np.where(vis, ref, np.float32(-np.finfo(np.float32).max))
    assert np.array_equal(got.view(np.uint32), ref.astype(np.float32).view(np.uint32))


def check_scores_decode_matches_prefill(O):
    """launchQsaIndexScoresDecode: the decode token t = ctx-1 scored against kbar gathered from
    the V-tails equals row t of the prefill scores over [0, ctx/4); entries past the prefix are
    not written; blocks whose V page is unused score -FLT_MAX."""
    from oracle.ref import Pool
    rng = np.random.default_rng(79)
    dt = "bf16"
    L = np.array([300, 131, 8, 3], np.int32)
    x, wQ, wK, cs, pt, numPages = _history(rng, dt, L)
    B, Lmax = x.shape[:2]
    nb = (Lmax + 3) // 4
    data = np.full((2 * numPages, 128, 2, 384), 0xA5A5, np.uint16)
    pool = Pool(data, pt, numPages, 256)
    kb = O.k_compress(x, cs, L, wK, 1e-6, nb, 0, nb, 0, dt, pool=pool)
    q = O.q_prep(x, cs, L, wQ, 1e-6, dt)
    full = O.scores(q, kb, L, 0, B * Lmax, dt).reshape(B, Lmax, nb)
    qdec = np.stack([q[b, L[b] - 1] for b in range(B)])
    lg = O.scores_decode(qdec, L, pool, nb, dt)
    for b in range(B):
        n = L[b] // 4
        assert np.array_equal(lg[b, :n].view(np.uint32), full[b, L[b] - 1, :n].view(np.uint32))
        assert np.all(np.isnan(lg[b, n:]))
    pt2 = pt.copy()
    pt2[0, 1, 1] = -1                       # blocks 32..63 of sequence 0 lose their V page
    lg2 = O.scores_decode(qdec, L, Pool(data, pt2, numPages, 256), nb, dt)
    assert np.all(lg2[0, 32:64].view(np.uint32) == NEG_FLT_MAX_BITS)
    assert np.array_equal(lg2[0, :32], lg[0, :32]) and np.array_equal(lg2[0, 64:75], lg[0, 64:75])


# ----------------------------------------------------------------- selection + expand ----

def _orderable_np(lg):
    """The page's map u = bits >= 0 ? bits | 0x80000000 : ~bits, in numpy (int64 keys)."""
    b = np.ascontiguousarray(lg, np.float32).view(np.uint32).astype(np.int64)
    return np.where(b & 0x80000000, (~b) & 0xFFFFFFFF, b | 0x80000000)


def check_ids_fill(O):
    """launchQsaIndexIdsFill: every row of the segmented sort's id array is 0, 1, ...,
    numBlocks-1 (the page's ids[r * numBlocks + c] = c), whatever the row; empty shapes give
    empty arrays.  The 3 x 5 case is written out by hand."""
    assert O.ids_fill(3, 5).tolist() == [[0, 1, 2, 3, 4]] * 3
    assert O.ids_fill(1, 1).tolist() == [[0]]
    assert O.ids_fill(0, 7).shape == (0, 7) and O.ids_fill(4, 0).shape == (4, 0)
    big = O.ids_fill(37, 1031)
    assert np.all(big[:, 0] == 0) and np.all(np.diff(big, axis=1) == 1)
    assert np.all(big == big[:1])


def check_expand_hand_worked(O):
    """launchQsaIndexExpand on hand-worked rows: t=0 is only its tail token; t=3 one block; t=6
    one block plus tail 4,5,6; t=2050 fills all 2051 slots (4*512 + 3); a padded row is -1."""
    S = 2051
    sorted_ids = np.tile(np.arange(512, dtype=np.int32)[::-1], (5, 1))  # any order: 511, 510, ..
    rows = {0: [0], 3: [511 * 4 + j for j in range(4)],
            6: [511 * 4 + j for j in range(4)] + [4, 5, 6]}
    for t, expect in rows.items():
        out = O.expand(sorted_ids[:1], np.array([S]), 1, S, t, 1)[t]
        assert out[:len(expect)].tolist() == expect and np.all(out[len(expect):] == -1), t
    out = O.expand(sorted_ids[:1], np.array([S]), 1, S, 2050, 1)[2050]
    assert np.all(out >= 0) and out[-3:].tolist() == [2048, 2049, 2050]
    assert sorted(out[:2048].tolist()) == list(range(2048))
    out = O.expand(sorted_ids[:1], np.array([100]), 1, S, 100, 1)[100]
    assert np.all(out == -1)


def check_expand_invariants(O):
    """Every expanded row lists distinct tokens in [0, t]: 4 per selected block, then the tail
    [4*nVis, t]; the count is 4*min(512, nVis) + (t+1)%4."""
    rng = np.random.default_rng(83)
    B, S = 2, 3000
    nb = S // 4
    ts = rng.choice(S, 40, replace=False)
    for t in ts:
        nvis = (t + 1) // 4
        srt = np.zeros((1, nb), np.int32)
        srt[0, :nvis] = rng.permutation(nvis)
        out = O.expand(srt, np.array([S, S]), B, S, S + int(t), 1)[S + t]
        n = 4 * min(512, nvis) + (t + 1) % 4
        v = out[:n]
        assert np.all(out[n:] == -1) and len(set(v.tolist())) == n
        assert np.all((v >= 0) & (v <= t))
        assert v[4 * min(512, nvis):].tolist() == list(range(4 * nvis, t + 1))


def check_orderable_map(O):
    """The selection's key order is the float order (non-NaN), with -0 just below +0."""
    rng = np.random.default_rng(89)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32) * 1e3,
                        np.array([0.0, -0.0, np.inf, -np.inf, 1e-45, -1e-45,
                                  np.finfo(np.float32).max, -np.finfo(np.float32).max],
                                 np.float32)])
    # the oracle's ordering through a one-row prefill selection over all of x
    S = 4 * len(x)
    out, srt = O.topk_expand(x[None, :], np.array([S]), 1, S, S - 1, 1)
    order = x[srt[0]]
    assert np.all(order[:-1] >= order[1:])
    pz, nz = np.where((x == 0) & ~np.signbit(x))[0][0], np.where((x == 0) & np.signbit(x))[0][0]
    assert list(srt[0]).index(pz) < list(srt[0]).index(nz)
    assert np.array_equal(np.argsort(-_orderable_np(x), kind="stable"), srt[0])


def check_topk_vs_numpy(O):
    """The prefill selection equals numpy's stable argsort of the descending keys (ties in
    ascending id) followed by the expand rule; a padded row is -1."""
    rng = np.random.default_rng(97)
    B, S = 2, 2400
    nb = S // 4
    lg = (rng.standard_normal((B * S, nb)) ** 2).astype(np.float32)
    lg[:, ::7] = lg[:, 3:4]             # many exact ties
    ctx = np.array([2400, 2100], np.int32)
    rows = np.sort(rng.choice(B * S, 64, replace=False))
    for r in rows:
        out, srt = O.topk_expand(lg[r:r + 1], ctx, B, S, int(r), 1)
        ref = np.argsort(-_orderable_np(lg[r]), kind="stable")
        assert np.array_equal(srt[0], ref)
        b, t = divmod(int(r), S)
        if t >= ctx[b]:
            assert np.all(out[r] == -1)
            continue
        nvis = (t + 1) // 4
        k = min(512, nvis)
        exp = (ref[:k, None] * 4 + np.arange(4)).reshape(-1).tolist() + \
            list(range(4 * nvis, t + 1))
        assert out[r, :len(exp)].tolist() == exp and np.all(out[r, len(exp):] == -1)


def check_topk_ties_and_decode_set(O):
    """launchQsaTopKExpandDecode: equal keys at the threshold are taken in ascending block id;
    nVis <= 512 takes every block without reading logits; the decode selection is the same
    block set as the prefill selection of the same logits, emitted in ascending id order."""
    rng = np.random.default_rng(101)
    B, mb = 6, 4000
    lg = np.full((B, mb), np.nan, np.float32)
    ctx = np.array([4000 * 4, 2051, 513 * 4 + 2, 9, 0, 3000], np.int32)
    for b in range(B):
        n = max(0, min(mb, int(ctx[b]) // 4))
        lg[b, :n] = rng.integers(0, 50, n).astype(np.float32)   # heavy ties
    lg[1, :] = np.nan                                            # nVis = 512: never read
    out = O.topk_expand_decode(lg, ctx)
    out2, sc = O.topk_expand_decode(lg, ctx, np.full((B, 3), 7, np.int32))
    assert np.array_equal(out2, out) and np.all(sc == 0)         # step a.: counters zeroed
    for b in range(B):
        c = int(ctx[b])
        if c <= 0:
            assert np.all(out[b] == -1)
            continue
        nvis = min(mb, c // 4)
        k = min(512, nvis)
        sel = out[b, :4 * k:4] // 4
        assert np.all(np.diff(sel) > 0)                          # ascending id order
        assert out[b, 4 * k:4 * k + c % 4].tolist() == list(range(4 * nvis, 4 * nvis + c % 4))
        if nvis <= 512:
            assert sel.tolist() == list(range(nvis))
            continue
        key = _orderable_np(lg[b, :nvis])
        thr = np.sort(key)[::-1][k - 1]
        assert np.all(key[sel] >= thr) and np.sum(key > thr) <= k
        eq = np.where(key == thr)[0]
        need = k - int(np.sum(key > thr))
        assert np.array_equal(np.intersect1d(sel, eq), eq[:need])   # ascending id at the tie
        # same set as the prefill selection of row t = c - 1 with the same logits
        S = c
        row = np.full((1, nvis), 0, np.float32)
        row[0] = lg[b, :nvis]
        pout, _ = O.topk_expand(row, np.array([S]), 1, S, S - 1, 1)
        assert set(pout[S - 1, :4 * k].tolist()) == set(out[b, :4 * k].tolist())


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
