"""The entry points enqueue on the caller's stream and neither synchronise nor allocate, so a
caller can capture them in a HIP graph.  A captured prefill -> scores -> selection sequence,
replayed several times on fresh inputs copied into the captured input buffer, with eager calls
and synchronisations between the replays, must give the eager calls' bits every time."""
import numpy as np
import pytest
import torch

from sparse_attention_indexer_qsa_amd import workloads as W
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager_calls():
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import sparse_attention_indexer_qsa_amd.qsa as qsa
    dt, B, S = "bf16", 2, 4096
    nb = S // 4
    rng = np.random.default_rng(5)
    cs = G.dev(W.cos_sin_table(S, 1e4))
    wq = G.dev_bits(W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt))
    wk = G.dev_bits(W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt))
    ctx = G.dev(np.array([4096, 3333], np.int32))

    def draw(seed):
        r = np.random.default_rng(seed)
        return G.dev_bits(W.to_bits(r.standard_normal((B, S, 640), dtype=np.float32), dt))

    x = draw(0)                      # the captured input buffer
    q = torch.empty(B, S, 4, 128, dtype=torch.int16, device="cuda")
    kb = torch.empty(B, nb, 128, dtype=torch.int16, device="cuda")
    logits = torch.empty(B * S, nb, dtype=torch.float32, device="cuda")
    out = torch.empty(B * S, qsa.INDEX_WIDTH, dtype=torch.int32, device="cuda")

    def step():                      # on the current stream
        qsa.qsa_index_prefill(q, kb, x, cs, ctx, wq, wk, 1e-6, nb, dt=dt)
        qsa.qsa_index_scores(logits, q, kb, ctx, nb, 0, B * S, dt=dt)
        qsa.qsa_index_topk_expand(out, logits, ctx, B, S, nb, 0, B * S)

    def outputs():
        return [q.clone(), kb.clone(), logits.view(torch.int32).clone(), out.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):    # every kernel runs once before the capture
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("[gpu] capturing prefill -> scores -> selection", flush=True)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for seed in (1, 2, 3, 4):
        fresh = draw(seed)
        x.copy_(fresh)
        step()                       # eager reference on these inputs
        torch.cuda.synchronize()
        ref = outputs()
        for t in (q, kb, out):       # poison the outputs, then replay on the same inputs
            t.fill_(-7)
        logits.fill_(1.5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        for name, a, b in zip(("qNormed", "kbar", "logits", "indices"), got, ref):
            assert torch.equal(a, b), f"replay {seed}: {name} differs from the eager call"
        print(f"[parity] graph replay {seed}: all four outputs equal the eager calls", flush=True)


def test_decode_graph_replays_match_eager_calls():
    """The serving loop's decode step (pre-pass -> decode scores -> decode selection) captured
    once and replayed on fresh new-token rows: q rows, logits, indices, split counters and the
    whole pool equal those of eager calls from the same pool state, every replay."""
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import sparse_attention_indexer_qsa_amd.qsa as qsa
    dt, B = "bf16", 8
    rng = np.random.default_rng(9)
    ctx_np = np.array([4097, 9, 2050, 700, 1, 3000, 4096, 513], np.int32)
    m = 33                                              # pages per sequence (4224 tokens)
    numPages = B * m
    pt = np.stack([rng.permutation(numPages).reshape(B, m),
                   rng.permutation(numPages).reshape(B, m) + numPages], 1).astype(np.int32)
    pt[2, 1, 5] = -1
    spec = W.PoolSpec(numPages, pt)
    pool = G.device_pool(spec)
    init = G.dev_bits(W.to_bits(rng.standard_normal(spec.shape, dtype=np.float32), dt))
    pool.pool.copy_(init)
    mb = int((ctx_np.max() + 3) // 4)
    cs = G.dev(W.cos_sin_table(4 * mb + 8, 1e4))
    wq = G.dev_bits(W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt))
    wk = G.dev_bits(W.to_bits(0.1 * rng.standard_normal(128, dtype=np.float32), dt))
    ctx = G.dev(ctx_np)

    def draw(seed):
        r = np.random.default_rng(seed)
        return G.dev_bits(W.to_bits(r.standard_normal((B, 1, 640), dtype=np.float32), dt))

    x = draw(0)
    q = torch.empty(B, 1, 4, 128, dtype=torch.int16, device="cuda")
    logits = torch.zeros(B, mb, dtype=torch.float32, device="cuda")
    out = torch.empty(B, qsa.INDEX_WIDTH, dtype=torch.int32, device="cuda")
    sc = torch.empty(B, 2, dtype=torch.int32, device="cuda")

    def step():
        qsa.qsa_index_pre_decode(q, x, cs, ctx, wq, wk, 1e-6, pool, dt=dt)
        qsa.qsa_index_scores_decode(logits, q, ctx, pool, mb, dt=dt)
        qsa.qsa_index_topk_expand_decode(out, logits, ctx, mb, splitCounters=sc, numKVHeads=2)

    def outputs():
        return [q.clone(), logits.view(torch.int32).clone(), out.clone(), sc.clone(),
                pool.pool.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("[gpu] capturing pre-pass -> decode scores -> decode selection", flush=True)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for seed in (1, 2, 3):
        x.copy_(draw(seed))
        pool.pool.copy_(init)
        logits.zero_()
        step()
        torch.cuda.synchronize()
        ref = outputs()
        pool.pool.copy_(init)
        logits.zero_()
        q.fill_(-7)
        out.fill_(-7)
        sc.fill_(5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        for name, a, b in zip(("qNormed", "logits", "indices", "split counters", "pool"), got,
                              ref):
            assert torch.equal(a, b), f"replay {seed}: {name} differs from the eager calls"
        print(f"[parity] decode graph replay {seed}: all outputs equal the eager calls", flush=True)


def test_split_decode_selection_graph_replays():
    """The decode selection of rows past 32768 blocks (a chunk launch that stages candidates in
    the output rows, then a merge launch) captured once and replayed on fresh logits: every
    replay equals an eager call, and the output rows hold no staging left over."""
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import sparse_attention_indexer_qsa_amd.qsa as qsa
    mb, B = 65536, 16
    ctx_np = W.decode_long_ctx(mb, B=B, seed=5)
    ctx_np[:3] = [0, 2051, 4 * mb + 2]
    ctx = G.dev(ctx_np)
    logits = G.dev(W.decode_logits(21, ctx_np, mb))
    out = torch.empty(B, qsa.INDEX_WIDTH, dtype=torch.int32, device="cuda")
    sc = torch.empty(B, 3, dtype=torch.int32, device="cuda")

    def step():
        qsa.qsa_index_topk_expand_decode(out, logits, ctx, mb, splitCounters=sc, numKVHeads=3)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print("[gpu] capturing the split decode selection", flush=True)
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for seed in (31, 32, 33):
        logits.copy_(G.dev(W.decode_logits(seed, ctx_np, mb, styles=("scores", "ties"))))
        step()
        torch.cuda.synchronize()
        ref = [out.clone(), sc.clone()]
        out.fill_(-7)
        sc.fill_(5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(sc, ref[1]), f"replay {seed}"
        assert torch.all(sc == 0)
    print("[parity] split decode selection: 3 graph replays equal eager calls", flush=True)
