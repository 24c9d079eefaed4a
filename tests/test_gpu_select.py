"""GPU parity of the block selection and expansion (qsa_index_ids_fill, qsa_index_expand,
qsa_index_topk_expand, qsa_index_topk_expand_decode) through the C ABI.  All outputs are
integers and are compared bit-exactly with the oracle: the page's full-row stable descending
sort + expand for prefill, the top-512 set emitted in ascending id for decode."""
import numpy as np
import pytest
import torch

from sparse_attention_indexer_qsa_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu
WIDTH = 2051
POISON = 0x5A5A5A5A


@pytest.fixture(scope="module")
def qsa():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import sparse_attention_indexer_qsa_amd.qsa as q
    return q


@pytest.fixture(scope="module")
def O():
    from oracle.ref import default
    return default()


def _host(g):
    torch.cuda.synchronize()
    g.check()
    return g.t.cpu().numpy()


def _check_chunk(got, ref, rowStart, numRows, what):
    """Rows of the chunk equal the oracle's, rows outside it keep the poison."""
    inside = np.zeros(got.shape[0], bool)
    inside[rowStart:rowStart + numRows] = True
    assert np.all(got[~inside] == POISON), f"{what}: rows outside the chunk written"
    bad = np.flatnonzero(np.any(got[inside] != ref[inside], axis=1))
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first global row {rowStart + bad[0]}"


def test_ids_fill(qsa, O):
    for rows, nb in [(37, 1000), (1, 1), (5, 4097)]:
        g = G.Guarded((rows, nb), torch.int32, fill=POISON)
        print(f"[gpu] ids_fill rows={rows} nb={nb}", flush=True)
        qsa.qsa_index_ids_fill(g.t, rows, nb)
        assert np.array_equal(_host(g), O.ids_fill(rows, nb))


# name: (B, S, numBlocks, ctx, rowStart, numRows, logit styles cycled by row)
PREFILL_CASES = {
    "ragged": (3, 2600, 650, [2600, 0, 1999], 0, 3 * 2600, ("scores", "ties")),
    "chunk": (2, 4096, 1024, [4096, 3001], 2500, 4000, ("scores", "ties", "normal",
                                                         "special_ge")),
    "narrow": (1, 4096, 700, [4096], 1500, 2596, ("scores", "normal")),
    "tiny": (2, 9, 3, [9, 5], 0, 18, ("scores",)),
    "zeros": (1, 3000, 750, [3000], 2040, 960, ("ties",)),
}


def _prefill_case(case):
    B, S, nb, ctx, r0, n, styles = PREFILL_CASES[case]
    ctx = np.array(ctx, np.int32)
    logits = W.prefill_logits(11, ctx, S, nb, r0, n, styles)
    if case == "zeros":
        logits[logits > -W.FLT_MAX] = 0.0       # every complete block ties
    return B, S, nb, ctx, r0, n, logits


@pytest.mark.parametrize("case", list(PREFILL_CASES))
def test_topk_expand_prefill(qsa, O, case):
    """Fused selection + K4 over a row chunk: rows below and above 512 complete blocks, a
    numBlocks narrower than the rows' complete blocks, ties, +-0, NaN, +-inf, -FLT_MAX in
    complete blocks, padded rows and a sequence of length 0."""
    B, S, nb, ctx, r0, n, logits = _prefill_case(case)
    ref, _ = O.topk_expand(logits, ctx, B, S, r0, n)
    out = G.Guarded((B * S, WIDTH), torch.int32, fill=POISON)
    print(f"[gpu] topk_expand case={case} B={B} S={S} nb={nb} rows=[{r0},{r0 + n})", flush=True)
    qsa.qsa_index_topk_expand(out.t, G.dev(logits), G.dev(ctx), B, S, nb, r0, n)
    got = _host(out)
    ref[:r0] = POISON
    ref[r0 + n:] = POISON
    _check_chunk(got, ref, r0, n, f"topk_expand {case}")
    sel = int(np.count_nonzero(got[r0:r0 + n] >= 0))
    print(f"[parity] topk_expand {case}: {n} rows bit-exact ({sel} indices)", flush=True)


# Long rows: name -> (B, S, numBlocks, ctx, rowStart, numRows, styles).  Their outputs span
# B*S rows, so rows outside the chunk are checked on the device and only the chunk is copied.
LONG_CASES = {
    # rows of 32758-32768 blocks at the end of a 131072-token sequence (one wave per row)
    "full32k": (1, 131072, 32768, [131072], 131072 - 40, 40,
                ("scores", "normal", "ties", "special_ge", "zeros")),
    # 20 keys per thread (24 registers), mid-sequence rows
    "mid": (1, 40000, 10000, [40000], 20000, 64, ("scores", "normal", "ties", "special_ge")),
    # a chunk across two sequences: short rows of sequence 1 beside long rows of sequence 0
    "cross": (2, 12000, 3000, [12000, 11000], 11990, 30, ("scores", "normal")),
    # rows of 19999-20000 blocks beside every length from 0 to 1100 blocks of a second sequence
    # (the 1024-entry candidate buffer of rows up to 32768 blocks) and its padded rows
    "mid_buffer_edge": (2, 80000, 20000, [80000, 4400], 80000 - 4, 4 + 4500,
                        ("scores", "ties", "normal", "special_ge")),
    # rows of 18484-18500 blocks: just past the register kernel's 72 keys per thread
    "past_registers": (1, 74000, 18500, [74000], 74000 - 64, 64,
                       ("scores", "ties", "normal", "special_ge")),
    # rows longer than 32768 blocks (one wave per row, candidate buffer in LDS)
    "stream": (1, 140000, 35000, [140000], 140000 - 6, 6, ("scores", "normal", "ties")),
    # rows of about 70000 blocks: several cuts of the candidate buffer per row, with all keys
    # equal ("zeros") and with few distinct values, so that ties straddle every cut
    "very_long": (1, 280000, 70000, [280000], 280000 - 5, 5,
                  ("scores", "ties", "normal", "special_ge", "zeros")),
    # the same kernel on numBlocks not a multiple of 4: four rows of 32768-32771 blocks beside
    # every length from 0 to 2049 blocks of a second sequence (one candidate buffer holds
    # 2048), and its padded rows
    "long_unaligned": (2, 131080, 32771, [131080, 8196], 131080 - 4, 4 + 8250,
                       ("scores", "ties", "normal", "special_ge")),
    # the 1024-entry candidate buffer on numBlocks not a multiple of 4 (one load per key):
    # eight rows of 19999-20001 blocks beside every length from 0 to 775 blocks of a second
    # sequence, and its padded rows
    "wave_unaligned": (2, 80004, 20001, [80004, 3100], 80004 - 8, 8 + 3200,
                       ("scores", "ties", "normal", "special_ge")),
    # numBlocks not a multiple of 4 (one load per key): eight rows of 2249-2251 blocks beside
    # every length from 0 to 1750 blocks of a second sequence, and its padded rows
    "unaligned": (2, 9004, 2251, [9004, 7000], 9004 - 8, 8 + 7100,
                  ("scores", "ties", "normal", "special_ge")),
    # rows of 2045 to 2050 blocks: around one full candidate buffer of the long-row kernel
    "buffer_edge": (1, 8200, 2100, [8200], 8180, 20, ("scores", "ties", "normal")),
}


def _long_case(case):
    B, S, nb, ctx, r0, n, styles = LONG_CASES[case]
    ctx = np.array(ctx, np.int32)
    styles = tuple("ties" if s == "zeros" else s for s in styles)
    logits = W.prefill_logits(17, ctx, S, nb, r0, n, styles)
    if "zeros" in LONG_CASES[case][6]:
        k = LONG_CASES[case][6].index("zeros")
        for i in range(k, n, len(LONG_CASES[case][6])):
            logits[i][logits[i] > -W.FLT_MAX] = 0.0
    return B, S, nb, ctx, r0, n, logits


def _run_long(qsa, O, B, S, nb, ctx, r0, n, logits, what):
    ref, _ = O.topk_expand(logits, ctx, B, S, r0, n)   # rows outside the chunk stay untouched
    out = G.Guarded((B * S, WIDTH), torch.int32, fill=POISON)
    print(f"[gpu] topk_expand {what} B={B} S={S} nb={nb} rows=[{r0},{r0 + n})", flush=True)
    qsa.qsa_index_topk_expand(out.t, G.dev(logits), G.dev(ctx), B, S, nb, r0, n)
    torch.cuda.synchronize()
    out.check()
    assert bool((out.t[:r0] == POISON).all()) and bool((out.t[r0 + n:] == POISON).all()), \
        f"{what}: rows outside the chunk written"
    got = out.t[r0:r0 + n].cpu().numpy()
    bad = np.flatnonzero(np.any(got != ref[r0:r0 + n], axis=1))
    assert bad.size == 0, f"{what}: {bad.size} rows differ, first global row {r0 + bad[0]}"
    print(f"[parity] topk_expand {what}: {n} rows bit-exact", flush=True)


@pytest.mark.parametrize("case", list(LONG_CASES))
def test_topk_expand_long_rows(qsa, O, case):
    """Rows of up to 35000 complete blocks: chunks across two sequences (long rows beside short
    and padded ones), numBlocks not a multiple of 4, rows around one candidate buffer and past
    32768 blocks; value styles with recurring values, many ties at the threshold (all equal
    included), +-0, +-inf, NaN and -FLT_MAX."""
    _run_long(qsa, O, *_long_case(case), case)


def test_topk_expand_long_prefill_bench_rows(qsa, O):
    """The launch the benchmark times: rows [65536, 73728) of the long prefill (16384 to 18432
    complete blocks each, 72 register keys per thread), scores-like logits with recurring
    values; all 8192 rows bit-exact against the oracle's full stable sort."""
    S, nb, r0, n = 131072, 32768, 65536, 8192
    ctx = np.array([S], np.int32)
    logits = W.prefill_logits(23, ctx, S, nb, r0, n, ("scores",))
    _run_long(qsa, O, 1, S, nb, ctx, r0, n, logits, "bench rows")


def test_topk_expand_rank_paths(qsa, O):
    """Rows of about 17500 blocks (72 register keys per thread) built so that the ranking of
    the selected keys takes each of its paths: 600 keys tied at the maximum (every selected
    key in one bucket: the bitonic fallback on the candidates); 700 distinct keys one ulp apart
    at the top (buckets one ulp wide); 1200 keys tied at the threshold under 300 distinct ones
    (too many candidates: the exact threshold, the ordered pass over the row, one large bucket);
    900 tied under 100 distinct (1000 candidates, one large bucket); and 1100 distinct keys
    one ulp apart (more than 1024 candidates: the exact threshold from the LDS passes, then the
    ranks of the keys at or above it); and a row whose only large keys sit where the register
    kernel samples (the first key of every other register group), so that the sample's estimate
    leaves fewer than 512 keys above it and the exact select runs instead."""
    B, S, nb = 1, 70000, 17500
    ctx = np.array([S], np.int32)
    r0, n = S - 6, 6
    rng = np.random.default_rng(31)
    logits = rng.standard_normal((n, nb)).astype(np.float32)
    five = np.array([5.0], np.float32).view(np.uint32)[0]

    def above(k, start=0):  # k distinct keys, one ulp apart, from 5.0 + start ulps up
        return (five + np.uint32(start) + np.arange(k, dtype=np.uint32)).view(np.float32)

    for row, (tied, distinct) in enumerate([(600, 0), (0, 700), (1200, 300), (900, 100),
                                            (0, 1100)]):
        pos = rng.choice(nb, tied + distinct, replace=False)
        logits[row, pos[:tied]] = np.float32(5.0)
        if distinct:
            logits[row, pos[tied:]] = above(distinct, 1 if tied else 0)
    ids = np.arange(nb)
    sampled = (ids % 4 == 0) & ((ids // 1024) % 2 == 0)  # 256 threads x 4 keys per group
    logits[5, sampled] += np.float32(10.0)
    _run_long(qsa, O, B, S, nb, ctx, r0, n, logits, "rank paths")


def test_topk_expand_estimate_boundary(qsa, O):
    """One launch of the 48-keys-per-thread register kernel over rows of 8200 to 8500 blocks in
    four value styles: rows below about 8330 blocks take the exact select (the sample's k would
    exceed half the threads), longer ones the sampled first pass; bit-exact against the oracle
    either way, on 16-byte aligned rows and on rows of one load per key."""
    for nb in (8528, 8525):
        S = 34100
        ctx = np.array([S], np.int32)
        r0, n = 32800, 1200
        logits = W.prefill_logits(19, ctx, S, nb, r0, n,
                                  ("scores", "normal", "ties", "special_ge"))
        _run_long(qsa, O, 1, S, nb, ctx, r0, n, logits, f"estimate boundary nb={nb}")


def test_topk_expand_wave_estimate_fallback(qsa, O):
    """Rows past the register kernel (one wave per row) whose only large keys sit in runs of
    256 at each eighth of the row, which include the runs the walk samples for its start
    threshold (one at each quarter): the estimate then leaves fewer than 512 keys above it and
    the row is walked again from the plain start.
    Beside each, a row of the same length with the large keys elsewhere; 16-byte aligned rows
    and rows of one load per key."""
    for S, nb in ((80000, 20000), (80004, 20001)):
        ctx = np.array([S], np.int32)
        r0, n = S - 4, 4
        rng = np.random.default_rng(37)
        logits = rng.standard_normal((n, nb)).astype(np.float32)
        for row in range(n):
            nv = min((r0 + row + 1) // 4, nb)
            runs = np.zeros(nb, bool)
            for j in range(8):
                p = (j * nv // 8) & ~3
                runs[p:p + 256] = True
            if row % 2 == 0:
                logits[row, runs] += np.float32(10.0)
            else:
                logits[row, np.flatnonzero(~runs[:nv])[:2048]] += np.float32(10.0)
        _run_long(qsa, O, 1, S, nb, ctx, r0, n, logits, f"wave estimate fallback nb={nb}")


def test_topk_expand_all_ones_nan(qsa, O):
    """Keys at the bottom of the order (FP32 bits 0xFFFFFFFF map to 0): a row made only of
    them (the threshold is 0 and padding keys equal it), a row where one thread's keys are all
    such NaNs (the radix window then starts at 0), and a row that is mostly NaN with 600
    ordinary values.  numBlocks < nVis, so every entry is a complete block."""
    B, S, nb = 1, 12100, 3000
    ctx = np.array([S], np.int32)
    r0, n = S - 9, 9
    rng = np.random.default_rng(23)
    logits = rng.standard_normal((n, nb)).astype(np.float32)
    bits = logits.view(np.uint32)
    bits[0::3] = 0xFFFFFFFF
    bits[1::3, 1200:1204] = 0xFFFFFFFF
    for i in range(2, n, 3):
        keep = rng.choice(nb, 600, replace=False)
        row = np.full(nb, 0xFFFFFFFF, np.uint32)
        row[keep] = bits[i, keep]
        bits[i] = row
    _run_long(qsa, O, B, S, nb, ctx, r0, n, logits, "all-ones NaN")
    # the same with a row of 700 blocks (a single register group, row-minimum window)
    nb2 = 700
    lg2 = np.ascontiguousarray(logits[:, :nb2])
    _run_long(qsa, O, B, S, nb2, ctx, r0, n, lg2, "all-ones NaN, 700 blocks")


@pytest.mark.parametrize("case", ["ragged", "chunk"])
def test_expand_prefill(qsa, O, case):
    """K4 alone, fed with the oracle's sorted ids (the page's sort output)."""
    B, S, nb, ctx, r0, n, logits = _prefill_case(case)
    ref, srt = O.topk_expand(logits, ctx, B, S, r0, n)
    out = G.Guarded((B * S, WIDTH), torch.int32, fill=POISON)
    print(f"[gpu] expand case={case}", flush=True)
    qsa.qsa_index_expand(out.t, G.dev(srt), G.dev(ctx), B, S, nb, r0, n)
    got = _host(out)
    ref[:r0] = POISON
    ref[r0 + n:] = POISON
    _check_chunk(got, ref, r0, n, f"expand {case}")
    # and the oracle's expand of the same sorted ids agrees with its fused form
    ref2 = O.expand(srt, ctx, B, S, r0, n, outIdx=np.full((B * S, WIDTH), POISON, np.int32))
    assert np.array_equal(ref2, ref)


@pytest.mark.parametrize("maxBlocks", [4096, 512, 600, 2000, 1001, 9000, 16384, 32768, 40000, 0, 1, 3])
def test_topk_expand_decode(qsa, O, maxBlocks):
    """64 sequences: ctx <= 0, ctx/4 below, at and above 512, above 4*maxBlocks (capped), all
    four logit styles including -inf and NaNs of both signs."""
    rng = np.random.default_rng(7 + maxBlocks)
    ctx = rng.integers(1, 4 * maxBlocks + 40, 64).astype(np.int32)
    ctx[:6] = [0, -5, 2048, 2051, 2052, 4 * maxBlocks + 3]
    ctx[6] = 1
    logits = W.decode_logits(13, ctx, maxBlocks)
    ref, ref_sc = O.topk_expand_decode(logits, ctx, np.full((64, 2), 9, np.int32))
    out = G.Guarded((64, WIDTH), torch.int32, fill=POISON)
    sc = G.Guarded((64, 2), torch.int32, fill=9)
    print(f"[gpu] topk_expand_decode maxBlocks={maxBlocks}", flush=True)
    qsa.qsa_index_topk_expand_decode(out.t, G.dev(logits), G.dev(ctx), maxBlocks,
                                     splitCounters=sc.t, numKVHeads=2)
    got = _host(out)
    assert np.array_equal(_host(sc), ref_sc)
    bad = np.flatnonzero(np.any(got != ref, axis=1))
    assert bad.size == 0, f"{bad.size} sequences differ, first {bad[0]} (ctx {ctx[bad[0]]})"
    print(f"[parity] topk_expand_decode maxBlocks={maxBlocks}: 64 rows bit-exact", flush=True)


def test_topk_expand_decode_bench_batch(qsa, O):
    """The launch the benchmark times: the decode batch of 64 sequences (one new token each,
    contexts up to 32772), rows of (max ctx + 3) / 4 blocks, scores-like logits."""
    wl = W.config4()
    ctx = (wl.ranges[0] + 1).astype(np.int32)
    mb = int((ctx.max() + 3) // 4)
    logits = W.decode_logits(5, ctx, mb, styles=("scores",))
    ref = O.topk_expand_decode(logits, ctx)
    out = G.Guarded((len(ctx), WIDTH), torch.int32, fill=POISON)
    print(f"[gpu] topk_expand_decode bench batch maxBlocks={mb}", flush=True)
    qsa.qsa_index_topk_expand_decode(out.t, G.dev(logits), G.dev(ctx), mb)
    got = _host(out)
    bad = np.flatnonzero(np.any(got != ref, axis=1))
    assert bad.size == 0, f"{bad.size} sequences differ, first {bad[0]} (ctx {ctx[bad[0]]})"
    print(f"[parity] topk_expand_decode bench batch: {len(ctx)} rows bit-exact", flush=True)


# Rows cut into chunks (maxBlocks above 32768): chunk lengths 8192, 16384 and 32768 occur;
# rows above 262144 blocks take the streaming kernel (the last two cases).
SPLIT_CASES = [(32772, 64), (65536, 64), (131071, 32), (200001, 24), (262144, 64),
               (262148, 8), (300001, 8)]


@pytest.mark.parametrize("maxBlocks,B", SPLIT_CASES)
def test_topk_expand_decode_long_rows(qsa, O, maxBlocks, B):
    """Long decode rows: contexts around every chunk boundary a row of these lengths can have
    (a chunk of 1, 512 and 513 keys, a row ending on a boundary), ctx <= 0, rows of <= 512
    blocks, capped contexts, and all four logit styles (ties spread across chunks, -inf, NaNs
    of both signs); aligned and unaligned rows."""
    rng = np.random.default_rng(11 + maxBlocks)
    ctx = rng.integers(1, 4 * maxBlocks + 40, B).astype(np.int32)
    special = [0, -5, 2048, 2052, 4 * maxBlocks + 3, 1]
    for c in (8192, 16384, 32768):
        for n in (c - 1, c, c + 1, c + 512, c + 513, 2 * c + 7, 7 * c + 300):
            if n <= maxBlocks:
                special.append(4 * n + int(rng.integers(0, 4)))
    special = special[:B]
    ctx[:len(special)] = special
    logits = W.decode_logits(17, ctx, maxBlocks)
    ref, ref_sc = O.topk_expand_decode(logits, ctx, np.full((B, 3), 9, np.int32))
    out = G.Guarded((B, WIDTH), torch.int32, fill=POISON)
    sc = G.Guarded((B, 3), torch.int32, fill=9)
    print(f"[gpu] topk_expand_decode long rows maxBlocks={maxBlocks} B={B}", flush=True)
    qsa.qsa_index_topk_expand_decode(out.t, G.dev(logits), G.dev(ctx), maxBlocks,
                                     splitCounters=sc.t, numKVHeads=3)
    got = _host(out)
    assert np.array_equal(_host(sc), ref_sc)
    bad = np.flatnonzero(np.any(got != ref, axis=1))
    assert bad.size == 0, f"{bad.size} sequences differ, first {bad[0]} (ctx {ctx[bad[0]]})"
    print(f"[parity] topk_expand_decode long rows maxBlocks={maxBlocks}: {B} rows bit-exact",
          flush=True)


@pytest.mark.parametrize("maxBlocks", [65536, 262144])
def test_topk_expand_decode_long_bench_batch(qsa, O, maxBlocks):
    """The launches the benchmark times for long decode rows: 64 sequences of maxBlocks / 2 to
    maxBlocks complete blocks, scores-like logits."""
    ctx = W.decode_long_ctx(maxBlocks)
    logits = W.decode_logits(5, ctx, maxBlocks, styles=("scores",))
    ref = O.topk_expand_decode(logits, ctx)
    out = G.Guarded((len(ctx), WIDTH), torch.int32, fill=POISON)
    print(f"[gpu] topk_expand_decode long bench batch maxBlocks={maxBlocks}", flush=True)
    qsa.qsa_index_topk_expand_decode(out.t, G.dev(logits), G.dev(ctx), maxBlocks)
    got = _host(out)
    bad = np.flatnonzero(np.any(got != ref, axis=1))
    assert bad.size == 0, f"{bad.size} sequences differ, first {bad[0]} (ctx {ctx[bad[0]]})"
    print(f"[parity] topk_expand_decode long bench batch maxBlocks={maxBlocks}: "
          f"{len(ctx)} rows bit-exact", flush=True)


def test_topk_expand_decode_all_ones_nan(qsa, O):
    """Decode rows holding FP32 bits 0xFFFFFFFF (the smallest key): all of them (threshold 0,
    padding keys equal to it), one register group of them inside ordinary values, and a few
    hundred ordinary values among them; rows of 700, 3000 and 9000 blocks."""
    rng = np.random.default_rng(29)
    maxBlocks = 9000
    ctx = np.array([4 * 700 + 1, 4 * 3000 + 2, 4 * 9000 + 3] * 3, np.int32)
    B = len(ctx)
    logits = rng.standard_normal((B, maxBlocks)).astype(np.float32)
    bits = logits.view(np.uint32)
    bits[0:3] = 0xFFFFFFFF
    bits[3:6, 1200:1204] = 0xFFFFFFFF
    for b in range(6, 9):
        keep = rng.choice(min(int(ctx[b]) // 4, maxBlocks), 600, replace=False)
        row = np.full(maxBlocks, 0xFFFFFFFF, np.uint32)
        row[keep] = bits[b, keep]
        bits[b] = row
    ref = O.topk_expand_decode(logits, ctx)
    out = G.Guarded((B, WIDTH), torch.int32, fill=POISON)
    print("[gpu] topk_expand_decode all-ones NaN", flush=True)
    qsa.qsa_index_topk_expand_decode(out.t, G.dev(logits), G.dev(ctx), maxBlocks)
    got = _host(out)
    bad = np.flatnonzero(np.any(got != ref, axis=1))
    assert bad.size == 0, f"{bad.size} sequences differ, first {bad[0]} (ctx {ctx[bad[0]]})"
    print(f"[parity] topk_expand_decode all-ones NaN: {B} rows bit-exact", flush=True)
