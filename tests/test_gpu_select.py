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


@pytest.mark.parametrize("maxBlocks", [4096, 512, 600])
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
