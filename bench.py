"""Benchmark of the QSA indexer hot path on one MI355X.

A step is one pass of the whole path (index-Q norm + rope, index-K block compression, kbar
V-tail and raw-K tail persistence) over the long single-sequence prefill workload: B = 1,
S = 131072 tokens, T = bf16, rope theta 1e6, pool of 1024 + 1024 pages.  It is one launch of
qsa_index_prefill through the C ABI.  The three-call sequence (qsa_index_q_prep,
qsa_index_k_compress with the pool, qsa_index_persist) is timed beside it.

Inputs are seeded synthetic data already resident in HBM.  Steps rotate over --sets copies of
every buffer, so no step finds its inputs in the 256 MB Infinity Cache.

Prints one JSON line: rows/s (value), ms per step, the roofline of the kernel (algorithmic
bytes per launch / average launch time from HIP events recorded on the launch stream, against
the 8 TB/s HBM peak), HBM traffic measured by rocprofv3 counters when a committed profile of
the current kernel source exists, and the CPU oracle timed on the host's cores.  Beside the
headline: the block-scores and selection legs, the decode legs, and each of the other four
workloads (tiny prefill, batched prefill in bf16 and fp16, decode sub-range compression,
mixed serving step) timed with a cold cache per rep.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer rows/s and achieved HBM GB/s (% of peak), bf16, QPrep+KCompress+persist"
HBM_PEAK_GBPS = 8000.0
KERNEL_SRCS = [os.path.join(ROOT, "sparse_attention_indexer_qsa_amd", "csrc", f)
               for f in ("qsa_kernels.hip", "qsa_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill_kernel_long_prefill.json")


def kernel_source_hash():
    """Hash of the sources of the fused prefill kernel (its kernel file and device helpers)."""
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl):
    """Bytes the fused prefill must move for workload `wl` (each consumed input byte once, each
    output byte once): valid q rows, distinct cosSin rows, every qNormed row (zeros included),
    raw keys of valid blocks, every dense kbar row of the range, the raw-K tails (read +
    write), kbar V-tails, the page-table entries those writes read, weights and lengths."""
    import numpy as np
    S, B = wl.S, wl.B
    L = np.clip(wl.ctx.astype(np.int64), 0, S)
    k1a = 1024 * int(L.sum()) + 256 * int(L.max()) + 1024 * B * S
    valid_blocks = L // 4
    k1b = 1024 * int(valid_blocks.sum()) + 256 * B * wl.numBlocks
    tails = L % 4
    pt = wl.pool.pageTable
    v_pages = sum(len(set(range(0, int(v) * 4, 128))) for v in valid_blocks) if len(L) else 0
    k_pages = int((tails > 0).sum())
    persist = 512 * int(tails.sum()) + 256 * int(valid_blocks.sum()) + 4 * (v_pages + k_pages)
    del pt
    return k1a + k1b + persist + 2 * 256 + 4 * B


def _triplets(wl):
    """Each sequence's block range [gB, gE) and past length: the call's scalars, or the
    per-sequence arrays (the range capped at maxBlockSpan blocks)."""
    import numpy as np
    B = wl.B
    if wl.ranges is None:
        return (np.full(B, wl.blockBegin, np.int64), np.full(B, wl.blockEnd, np.int64),
                np.full(B, wl.pastLen, np.int64))
    pl, bb, be, span = wl.ranges
    bb = bb.astype(np.int64)
    return bb, np.minimum(be.astype(np.int64), bb + span), pl.astype(np.int64)


def path_bytes(wl, q_prep=True):
    """Algorithmic bytes of one pass of the path over workload `wl`, from its seeded lengths
    and page table (an unfused sequence of calls is scored against the same count):
      q-prep   1024 per valid q row read + 256 per distinct cosSin row + 1024 per qNormed row
               written (padding zeros included);
      compress 1024 per valid block's raw keys + 256 per distinct cosSin row 4g + 256 per dense
               kbar row of the range written (invalid zeros included);
      persist  512 per raw-K tail token copied + 256 per kbar V-tail written + 4 per distinct
               page-table entry read;
      plus the two gammas (512) and the lengths (4 per sequence).
    Writes whose page entry is unused or out of range are not counted (nothing moves)."""
    import numpy as np
    B, S, nb = wl.B, wl.S, wl.numBlocks
    ctx = wl.ctx.astype(np.int64)
    pt = wl.pool.pageTable.astype(np.int64)
    mp, ids = pt.shape[2], 2 * wl.pool.numPages
    k1a = 0
    if q_prep:
        L = np.clip(ctx, 0, S)
        k1a = 1024 * int(L.sum()) + 256 * int(L.max(initial=0)) + 1024 * B * S
    gB, gE, p = _triplets(wl)
    valid_rows, dense, n_tail, n_kbar, entries = set(), 0, 0, 0, set()
    n_valid = 0

    def guard(b, plane, pos):
        slot = pos >> 7
        if slot < 0 or slot >= mp:
            return False
        entries.add((b, plane, slot))
        e = int(pt[b, plane, slot])
        return 0 <= e < ids

    for b in range(B):
        g = np.arange(max(gB[b], 0), min(gE[b], nb), dtype=np.int64)
        dense += len(g)
        t0 = 4 * g
        ok = (t0 + 3 < ctx[b]) & (t0 >= p[b]) & (t0 + 3 - p[b] < S)
        if wl.ranges is not None:
            ok &= t0 < wl.maxPositions
        gv = g[ok]
        n_valid += len(gv)
        valid_rows.update((4 * gv).tolist())
        for pos in (4 * gv).tolist():
            n_kbar += guard(b, 1, pos)
        c = int(ctx[b])
        if c > 0:
            for t in range(max(int(p[b]), c - c % 4), c):
                if 0 <= t - p[b] < S:
                    n_tail += guard(b, 0, t)
    k1b = 1024 * n_valid + 256 * len(valid_rows) + 256 * dense
    persist = 512 * int(n_tail) + 256 * int(n_kbar) + 4 * len(entries)
    return int(k1a + k1b + persist + 2 * 256 + 4 * B)


SCORE_ROWS = (65536, 8192)   # the long prefill's query rows [65536, 73728) scored and selected
INDEX_WIDTH = 2051           # token slots per selected row: 4 * 512 + 3


def scores_alg(S, nb, rowStart, numRows):
    """Algorithmic bytes of one qsa_index_scores call (FP32 logits of every (row, block), the
    rows' q, the kbar rows any row sees), the visible (row, block) pairs and their flops."""
    import numpy as np
    t = rowStart + np.arange(numRows)
    visible = int(np.minimum((t + 1) // 4, nb).sum())
    nvis_max = int(min((rowStart + numRows) // 4, nb))
    return 4 * numRows * nb + 1024 * numRows + 256 * nvis_max, visible, 2 * 4 * 128 * visible


def select_alg(S, nb, rowStart, numRows):
    """Algorithmic bytes of one qsa_index_topk_expand call: each row's complete-block logits
    read once, its 2051 token slots written."""
    import numpy as np
    t = rowStart + np.arange(numRows)
    return 4 * int(np.minimum((t + 1) // 4, nb).sum()) + 4 * INDEX_WIDTH * numRows


def cpu_baseline(wl, seconds):
    """The oracle (plain C, OpenMP) on the host: the whole path on the same inputs, repeated
    for about `seconds` of CPU work (at least 3 passes); the median pass is reported."""
    import numpy as np
    from oracle.ref import Pool, default
    O = default()
    threads = O.max_threads()
    pool = Pool(np.full(wl.pool.shape, 0xA5A5, np.uint16), wl.pool.pageTable, wl.pool.numPages,
                wl.pool.headSize)

    def run():
        O.q_prep(wl.indexQk, wl.cosSin, wl.ctx, wl.wQ, wl.eps, wl.dt)
        O.k_compress(wl.indexQk, wl.cosSin, wl.ctx, wl.wK, wl.eps, wl.numBlocks, 0, wl.numBlocks,
                     0, wl.dt, pool=pool)
        O.persist(pool, wl.indexQk, None, wl.ctx, wl.numBlocks, 0, wl.numBlocks, 0)

    def timed(budget):
        run()  # warm-up
        times = []
        t_start = time.perf_counter()
        while len(times) < 3 or time.perf_counter() - t_start < budget:
            t0 = time.perf_counter()
            run()
            times.append(time.perf_counter() - t0)
        return sorted(times)[len(times) // 2], len(times), time.perf_counter() - t_start

    t, passes, spent = timed(seconds)
    O.set_threads(1)
    t1, passes1, _ = timed(seconds / 3)
    O.set_threads(threads)
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": wl.B * wl.S / t, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole long-prefill workload (B={wl.B}, S={wl.S}) through the oracle's "
                      f"q_prep + k_compress(pool) + persist, {passes} passes in {spent:.1f} s "
                      f"after 1 warm-up, median pass {t * 1e3:.1f} ms, {threads} OpenMP threads",
            "single_thread": {"value": wl.B * wl.S / t1, "median_pass_ms": t1 * 1e3,
                              "passes": passes1},
            "cpu_model": model}


def decode_leg(qsa, torch, steps, warmup):
    """The decode pre-pass (qsa_index_pre_decode) on the decode workload's shape: 64 sequences,
    past lengths up to 32768, one new token each (the page's form), a pool of 16384 + 16384
    pages.  Latency-bound; reported beside the prefill figure, not as the headline."""
    import numpy as np
    from sparse_attention_indexer_qsa_amd import workloads as W
    wl = W.config4()
    ctx = (wl.ranges[0] + 1).astype(np.int32)
    B, S = wl.B, wl.S

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    x, cs, c = bits(wl.indexQk), torch.from_numpy(wl.cosSin).cuda(), torch.from_numpy(ctx).cuda()
    wQ, wK = bits(wl.wQ), bits(wl.wK)
    pool = torch.zeros(wl.pool.shape, dtype=torch.int16, device="cuda")
    ps = qsa.PoolState(pool, torch.from_numpy(wl.pool.pageTable).cuda(), wl.pool.numPages,
                       wl.pool.numKVHeads, wl.pool.poolHeadDim, wl.pool.headSize)
    q = torch.empty(B, S, 4, 128, dtype=torch.int16, device="cuda")
    pst = ps.c_struct(B)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()  # inputs made on the default stream are complete
    args = (q.data_ptr(), x.data_ptr(), cs.data_ptr(), cs.shape[0], c.data_ptr(), None,
            wQ.data_ptr(), wK.data_ptr(), wl.eps, ctypes.byref(pst), B, S, qsa.QSA_BF16,
            stream.cuda_stream)
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            assert qsa.lib.qsa_index_pre_decode(*args) == 0, qsa.qsa_last_error()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            qsa.lib.qsa_index_pre_decode(*args)
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    blocks = int(np.sum(ctx % 4 == 0))
    return {"workload": "decode pre-pass, B=64, one new token each, bf16",
            "entry": "qsa_index_pre_decode", "us_per_call": us, "tokens_per_s": B / us * 1e6,
            "blocks_compressed_per_call": blocks}


CONFIG_LEGS = ("tiny_prefill", "batched_prefill_bf16", "batched_prefill_f16", "decode_subrange",
               "mixed_serving")
SCRATCH_BYTES = 512 << 20    # written between cold-cache reps: twice the 256 MB Infinity Cache


def _config_workload(name):
    from sparse_attention_indexer_qsa_amd import workloads as W
    return {"tiny_prefill": W.config1, "batched_prefill_bf16": lambda: W.config2("bf16"),
            "batched_prefill_f16": lambda: W.config2("f16"), "decode_subrange": W.config4,
            "mixed_serving": W.config5}[name]()


def config_leg(qsa, torch, name, reps, warmup):
    """One of the five workloads through the C ABI, each rep with a cold cache: a 512 MiB
    scratch write (outside the timed span) evicts the Infinity Cache, then HIP events on the
    launch stream bracket the rep.  Prefills run as one fused launch (qsa_index_prefill) and
    as the three calls (q-prep, block compression with the pool, persist); the decode
    sub-range runs block compression with per-sequence ranges and the pool, then persist.
    Median, p10 and p90 over `reps`; GB/s on path_bytes of the run's seeded lengths."""
    import numpy as np
    wl = _config_workload(name)
    T = qsa.QSA_BF16 if wl.dt == "bf16" else qsa.QSA_F16
    B, S, nb = wl.B, wl.S, wl.numBlocks

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    x, cs = bits(wl.indexQk), torch.from_numpy(wl.cosSin).cuda()
    ctx, wQ, wK = torch.from_numpy(wl.ctx).cuda(), bits(wl.wQ), bits(wl.wK)
    pool = torch.full(wl.pool.shape, 0xA5A5 - 65536, dtype=torch.int16, device="cuda")
    ps = qsa.PoolState(pool, torch.from_numpy(wl.pool.pageTable).cuda(), wl.pool.numPages,
                       wl.pool.numKVHeads, wl.pool.poolHeadDim, wl.pool.headSize)
    pst = ps.c_struct(B)
    q = torch.empty(B, S, 4, 128, dtype=torch.int16, device="cuda")
    kb = torch.empty(B, nb, 128, dtype=torch.int16, device="cuda")
    rng = None
    if wl.ranges is not None:
        pl, bb, be, span = wl.ranges
        rt = [torch.from_numpy(a).cuda() for a in (pl, bb, be)]
        rng = qsa.qsa_seq_ranges_t(rt[0].data_ptr(), rt[1].data_ptr(), rt[2].data_ptr(), span)
    rp = ctypes.byref(rng) if rng is not None else None
    scratch = torch.empty(SCRATCH_BYTES // 4, dtype=torch.float32, device="cuda")
    L = qsa.lib
    alg = path_bytes(wl, wl.run_q_prep)

    def fused(st):
        return L.qsa_index_prefill(q.data_ptr(), kb.data_ptr(), x.data_ptr(), cs.data_ptr(),
                                   cs.shape[0], ctx.data_ptr(), wQ.data_ptr(), wK.data_ptr(),
                                   wl.eps, ctypes.byref(pst), B, S, nb, T, st)

    def three(st):
        rc = 0
        if wl.run_q_prep:
            rc |= L.qsa_index_q_prep(q.data_ptr(), x.data_ptr(), cs.data_ptr(), cs.shape[0],
                                     ctx.data_ptr(), wQ.data_ptr(), wl.eps, B, S, T, st)
        rc |= L.qsa_index_k_compress(kb.data_ptr(), x.data_ptr(), cs.data_ptr(), cs.shape[0],
                                     ctx.data_ptr(), wK.data_ptr(), wl.eps, B, S, nb,
                                     wl.blockBegin, wl.blockEnd, wl.pastLen, rp,
                                     ctypes.byref(pst), T, st)
        rc |= L.qsa_index_persist(ctypes.byref(pst), x.data_ptr(), None, ctx.data_ptr(), B, S, nb,
                                  wl.blockBegin, wl.blockEnd, wl.pastLen, rp, T, st)
        return rc

    def cold(fn):
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for _ in range(warmup):
                assert fn(stream.cuda_stream) == 0, qsa.qsa_last_error()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(reps)]
            for i, (a, b) in enumerate(ev):
                scratch.fill_(float(i))
                a.record(stream)
                fn(stream.cuda_stream)
                b.record(stream)
            torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
        p10, p50, p90 = us[len(us) // 10], us[len(us) // 2], us[(9 * len(us)) // 10]
        return {"us_p10_p50_p90": [p10, p50, p90], "rows_per_s": B * S / p50 * 1e6,
                "GBps": alg / p50 / 1e3, "hbm_frac": alg / p50 / 1e3 / HBM_PEAK_GBPS}

    out = {"workload": f"{wl.name}: B={B}, S={S}, {wl.dt}, numBlocks={nb}, "
                       f"numPages={wl.pool.numPages}", "alg_bytes": alg,
           "valid_rows": int(np.clip(wl.ctx, 0, S).sum()) if wl.run_q_prep else None}
    if wl.ranges is None:
        out["fused"] = cold(fused)
        out["fused"]["entry"] = "qsa_index_prefill"
    out["three_call"] = cold(three)
    out["three_call"]["entry"] = ("qsa_index_q_prep + " if wl.run_q_prep else "") + \
        "qsa_index_k_compress (pool" + (", per-sequence ranges" if rng is not None else "") + \
        ") + qsa_index_persist"
    del pool, scratch, x, q, kb
    torch.cuda.empty_cache()
    return out


# Each leg's warm-up lasts at least this long as well as `warmup` calls: the first tens of
# milliseconds of a leg on a freshly allocated output run measurably slower (the scores call
# 245 against 210 us over its first 55 calls, the selection 134 against 126), and the legs
# report steady-state calls.
WARM_S = 0.1


def _warm(torch, call, warmup):
    """Run call() `warmup` times and then until WARM_S seconds have passed, synchronised."""
    t0 = time.perf_counter()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < WARM_S:
        for _ in range(8):
            call()
        torch.cuda.synchronize()


def _time_stream(torch, fn, steps, warmup):
    """Average microseconds per call of fn() on a fresh stream, timed with stream events."""
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()  # inputs made on the default stream are complete
    with torch.cuda.stream(stream):
        _warm(torch, lambda: fn(stream.cuda_stream), warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn(stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / steps


def select_leg(qsa, torch, wl, logits, steps, warmup, rowStart=SCORE_ROWS[0]):
    """Top-512 selection + expand (qsa_index_topk_expand) of the long-prefill rows whose block
    scores the scores leg produced.  Reads each row's complete blocks, writes 2051 indices."""
    import numpy as np
    S, nb = wl.S, wl.numBlocks
    numRows = logits.shape[0]
    out = torch.empty(S, qsa.INDEX_WIDTH, dtype=torch.int32, device="cuda")
    ctx = torch.tensor([S], dtype=torch.int32, device="cuda")

    def call(st):
        rc = qsa.lib.qsa_index_topk_expand(out.data_ptr(), logits.data_ptr(), ctx.data_ptr(), 1,
                                           S, nb, rowStart, numRows, st)
        assert rc == 0, qsa.qsa_last_error()
    us = _time_stream(torch, call, steps, warmup)
    alg = select_alg(S, nb, rowStart, numRows)
    blocks = int(np.minimum((np.arange(rowStart, rowStart + numRows) + 1) // 4, nb).sum())
    del out
    return {"workload": f"long prefill rows [{rowStart}, {rowStart + numRows}) x {nb} blocks",
            "entry": "qsa_index_topk_expand", "us_per_call": us, "alg_bytes": alg,
            "GBps": alg / us / 1e3, "hbm_frac": alg / us / 1e3 / HBM_PEAK_GBPS,
            "blocks": blocks, "ps_per_block": us * 1e6 / blocks}


def select_long_leg(qsa, torch, steps, warmup):
    """Top-512 selection + expand on rows longer than 32768 blocks (one wave per row, an LDS
    candidate buffer): the last 2048 rows of a 262144-token sequence, 65024 to 65536 complete
    blocks each, scores-like logits (a ReLU's share of zeros, quantised so that values recur;
    -FLT_MAX past each row's complete blocks, as the scores call writes them)."""
    S, nb, numRows = 262144, 65536, 2048
    rowStart = S - numRows
    g = torch.Generator(device="cuda").manual_seed(7)
    # relu(2 x) quantised to 1/64, by divisions only: a multiply would launch the kernel the
    # counter calibration identifies as its reference (torch.mul, --copy-calib)
    logits = torch.randn(numRows, nb, generator=g, device="cuda")
    logits = torch.round(torch.relu(logits) / 0.0078125) / 64.0
    nvis = (torch.arange(rowStart, S, device="cuda") + 1) // 4
    cols = torch.arange(nb, device="cuda")
    logits[cols[None, :] >= nvis[:, None]] = -3.4028234663852886e38
    out = torch.empty(S, qsa.INDEX_WIDTH, dtype=torch.int32, device="cuda")
    ctx = torch.tensor([S], dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def call(st):
        rc = qsa.lib.qsa_index_topk_expand(out.data_ptr(), logits.data_ptr(), ctx.data_ptr(), 1,
                                           S, nb, rowStart, numRows, st)
        assert rc == 0, qsa.qsa_last_error()
    us = _time_stream(torch, call, steps, warmup)
    alg = select_alg(S, nb, rowStart, numRows)
    del out, logits
    return {"workload": f"rows [{rowStart}, {S}) of a {S}-token sequence x {nb} blocks",
            "entry": "qsa_index_topk_expand", "us_per_call": us, "alg_bytes": alg,
            "GBps": alg / us / 1e3, "hbm_frac": alg / us / 1e3 / HBM_PEAK_GBPS}


def scores_decode_leg(qsa, torch, steps, warmup):
    """Decode block scores (qsa_index_scores_decode) for the decode workload's 64 sequences,
    one new token each (contexts up to 32772): kbar gathered from the V-tails of the paged
    pool.  Latency-bound; reported beside the prefill figure."""
    import numpy as np
    from sparse_attention_indexer_qsa_amd import workloads as W
    wl = W.config4()
    ctx = (wl.ranges[0] + 1).astype(np.int32)
    B = len(ctx)
    mb = int((ctx.max() + 3) // 4)
    g = torch.Generator(device="cuda").manual_seed(6)
    q = torch.randn((B, 4, 128), generator=g, device="cuda").to(torch.bfloat16)
    pool = torch.randn(wl.pool.shape, generator=g, device="cuda", dtype=torch.bfloat16)
    ps = qsa.PoolState(pool, torch.from_numpy(wl.pool.pageTable).cuda(), wl.pool.numPages,
                       wl.pool.numKVHeads, wl.pool.poolHeadDim, wl.pool.headSize)
    pst = ps.c_struct(B)
    c = torch.from_numpy(ctx).cuda()
    lg = torch.empty(B, mb, dtype=torch.float32, device="cuda")

    def call(st):
        rc = qsa.lib.qsa_index_scores_decode(lg.data_ptr(), q.data_ptr(), c.data_ptr(),
                                             ctypes.byref(pst), B, mb, qsa.QSA_BF16, st)
        assert rc == 0, qsa.qsa_last_error()
    us = _time_stream(torch, call, steps, warmup)
    blocks = int(np.minimum(ctx // 4, mb).sum())
    alg = 260 * blocks + 1024 * B
    del pool, ps
    return {"workload": f"decode, B={B}, context up to {int(ctx.max())}, bf16",
            "entry": "qsa_index_scores_decode", "us_per_call": us, "alg_bytes": alg,
            "GBps": alg / us / 1e3}


def select_decode_leg(qsa, torch, steps, warmup):
    """Decode top-512 selection + expand (qsa_index_topk_expand_decode) for the decode
    workload's 64 sequences (context lengths up to 32772, scores-like logits)."""
    import numpy as np
    from sparse_attention_indexer_qsa_amd import workloads as W
    wl = W.config4()
    ctx = (wl.ranges[0] + 1).astype(np.int32)
    mb = int((ctx.max() + 3) // 4)
    lg = torch.from_numpy(W.decode_logits(5, ctx, mb, styles=("scores",))).cuda()
    c = torch.from_numpy(ctx).cuda()
    out = torch.empty(len(ctx), qsa.INDEX_WIDTH, dtype=torch.int32, device="cuda")

    def call(st):
        rc = qsa.lib.qsa_index_topk_expand_decode(out.data_ptr(), lg.data_ptr(), c.data_ptr(),
                                                  None, 0, len(ctx), mb, st)
        assert rc == 0, qsa.qsa_last_error()
    us = _time_stream(torch, call, steps, warmup)
    alg = 4 * int(np.minimum(ctx // 4, mb)[ctx // 4 > 512].sum()) + 4 * qsa.INDEX_WIDTH * len(ctx)
    blocks = int(np.minimum(ctx // 4, mb).sum())
    return {"workload": f"decode, B={len(ctx)}, context up to {int(ctx.max())}",
            "entry": "qsa_index_topk_expand_decode", "us_per_call": us, "alg_bytes": alg,
            "GBps": alg / us / 1e3, "blocks": blocks, "ps_per_block": us * 1e6 / blocks}


def select_decode_long_leg(qsa, torch, steps, warmup, maxBlocks):
    """Decode top-512 selection + expand (qsa_index_topk_expand_decode) over long rows: 64
    sequences of maxBlocks / 2 to maxBlocks complete blocks, scores-like logits.  Rows this
    long are cut into chunks selected by workgroups of their own and then merged."""
    import numpy as np
    from sparse_attention_indexer_qsa_amd import workloads as W
    ctx = W.decode_long_ctx(maxBlocks)
    lg = torch.from_numpy(W.decode_logits(5, ctx, maxBlocks, styles=("scores",))).cuda()
    c = torch.from_numpy(ctx).cuda()
    out = torch.empty(len(ctx), qsa.INDEX_WIDTH, dtype=torch.int32, device="cuda")

    def call(st):
        rc = qsa.lib.qsa_index_topk_expand_decode(out.data_ptr(), lg.data_ptr(), c.data_ptr(),
                                                  None, 0, len(ctx), maxBlocks, st)
        assert rc == 0, qsa.qsa_last_error()
    us = _time_stream(torch, call, steps, warmup)
    blocks = int(np.minimum(ctx // 4, maxBlocks).sum())
    alg = 4 * blocks + 4 * qsa.INDEX_WIDTH * len(ctx)
    del lg
    return {"workload": f"decode, B={len(ctx)}, rows of {maxBlocks // 2} to {maxBlocks} blocks",
            "entry": "qsa_index_topk_expand_decode", "us_per_call": us, "alg_bytes": alg,
            "GBps": alg / us / 1e3, "hbm_frac": alg / us / 1e3 / HBM_PEAK_GBPS,
            "blocks": blocks, "ps_per_block": us * 1e6 / blocks}


def scores_leg(qsa, torch, s, wl, steps, warmup, rowStart=SCORE_ROWS[0], numRows=SCORE_ROWS[1]):
    """Block scores (qsa_index_scores, MFMA) over a chunk of the long prefill's query rows,
    on the qNormed and kbar the fused prefill produced.  Bound by the FP32 logits it writes."""
    import numpy as np
    S, nb = wl.S, wl.numBlocks
    logits = torch.empty(numRows, nb, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()  # inputs made on the default stream are complete
    args = (logits.data_ptr(), s["q"].data_ptr(), s["kb"].data_ptr(), s["ctx"].data_ptr(), 1, S,
            nb, rowStart, numRows, qsa.QSA_BF16, stream.cuda_stream)
    with torch.cuda.stream(stream):
        assert qsa.lib.qsa_index_scores(*args) == 0, qsa.qsa_last_error()
        _warm(torch, lambda: qsa.lib.qsa_index_scores(*args), warmup)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            qsa.lib.qsa_index_scores(*args)
        e1.record(stream)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    alg, visible, flops = scores_alg(S, nb, rowStart, numRows)
    # the write floor of this output on this machine: torch fill_ of the same logits tensor
    fill_us = _time_stream(torch, lambda st: logits.fill_(-3.4028234663852886e38), steps, warmup)
    out_bytes = logits.numel() * 4
    write_ref = {"what": f"torch fill_ of the {out_bytes:,} B logits tensor", "us_per_fill": fill_us,
                 "GBps": out_bytes / fill_us / 1e3,
                 "frac_of_peak": out_bytes / fill_us / 1e3 / HBM_PEAK_GBPS}
    # the fills overwrote the logits that the select leg reads: compute them once more
    with torch.cuda.stream(stream):
        assert qsa.lib.qsa_index_scores(*args) == 0, qsa.qsa_last_error()
    torch.cuda.synchronize()
    return logits, {"workload": f"long prefill rows [{rowStart}, {rowStart + numRows}) x {nb} blocks, "
                        f"bf16, FP32 logits", "entry": "qsa_index_scores", "us_per_call": us,
            "alg_bytes": alg, "GBps": alg / us / 1e3, "hbm_frac": alg / us / 1e3 / HBM_PEAK_GBPS,
            "visible_scores": visible, "TFLOPs": flops / us / 1e6,
            "mfma_bf16_frac": flops / us / 1e6 / 2500.0, "write_reference": write_ref}


COPY_BYTES = 256 << 20


def copy_reference(qsa, torch, nbytes, steps, warmup, sets=4):
    """Plain device-to-device copies moving the same bytes as one fused launch (nbytes/2 read,
    nbytes/2 written), rotated over `sets` buffer pairs and timed with events like the kernel:
    the library's own plain copy (qsa_stream_copy: one 16-byte chunk per thread, non-temporal
    loads and stores, the fastest copy form measured on this machine) and torch's copy_.  The
    rate at which this box streams these bytes at all, for reading roofline.frac."""
    n = nbytes // 2 // 16 * 4
    bufs = [(torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0),
             torch.empty(n, dtype=torch.float32, device="cuda")) for _ in range(sets)]
    torch.cuda.synchronize()

    def timed(fn):
        stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i in range(warmup):
                fn(i, stream)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(steps):
                fn(i, stream)
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    us = timed(lambda i, st: qsa.qsa_stream_copy(bufs[i % sets][1], bufs[i % sets][0], st))
    assert torch.equal(bufs[0][1], bufs[0][0]), "qsa_stream_copy did not copy"
    tus = timed(lambda i, st: bufs[i % sets][1].copy_(bufs[i % sets][0]))
    del bufs
    moved = 2 * n * 4
    return {"what": f"qsa_stream_copy of {n * 4:,} B (read + write = {moved:,} B), {sets} "
                    f"rotating buffer pairs", "us_per_copy": us, "GBps": moved / us / 1e3,
            "frac_of_peak": moved / us / 1e3 / HBM_PEAK_GBPS,
            "torch_copy_us": tus, "torch_copy_GBps": moved / tus / 1e3}


def _csv_rows(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    assert files, f"no *{suffix} under {d}"
    return [r for f in files for r in csv.DictReader(open(f))]


def _counter(d, name):
    """Mean value of counter `name` per dispatch, by kernel name (rocprofv3 --pmc output)."""
    from collections import defaultdict
    acc = defaultdict(list)
    for r in _csv_rows(d, "counter_collection.csv"):
        if r["Counter_Name"] == name:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


PROFILE_MD = os.path.join(ROOT, "profiles", "prefill_kernel_long_prefill.md")
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d $OUT/ptrace -o run -- "
             "python3 $R/bench.py --steps 50 --warmup 10 --no-cpu --no-configs",
    "fetch": "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/pfetch -o run "
             "-- python3 $R/bench.py --steps 10 --warmup 2 --no-cpu --no-three-call --no-decode "
             "--no-configs --copy-calib",
    "write": "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/pwrite -o run "
             "-- python3 $R/bench.py --steps 10 --warmup 2 --no-cpu --no-three-call --no-decode "
             "--no-configs --copy-calib",
}


def summarize(trace_dir, fetch_dir, write_dir):
    """profiles/ summary of the fused prefill kernel: per-kernel durations from the kernel
    trace, HBM bytes from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what
    the same counter reads for a plain 256 MiB streaming kernel (torch.mul, --copy-calib)."""
    from sparse_attention_indexer_qsa_amd import workloads as W
    stats = _csv_rows(trace_dir, "kernel_stats.csv")
    fetch, write = _counter(fetch_dir, "FETCH_SIZE"), _counter(write_dir, "WRITE_SIZE")

    def pick(d, key):
        ks = [k for k in d if key in k]
        assert ks, (key, list(d))
        return d[ks[0]][0]

    copy_key = "MulFunctor"   # torch.mul over 256 MiB of float32 (--copy-calib); no other
    #                           leg of a counter run may launch a float multiply
    f_copy, w_copy = pick(fetch, copy_key), pick(write, copy_key)
    f_scale, w_scale = COPY_BYTES / (f_copy * 1024), COPY_BYTES / (w_copy * 1024)
    f_k, w_k = pick(fetch, "prefill_kernel"), pick(write, "prefill_kernel")
    fb, wb = f_k * 1024 * f_scale, w_k * 1024 * w_scale
    alg = algorithmic_bytes(W.config3())
    alg_path = path_bytes(W.config3())
    rec = {"kernel": "prefill_kernel<Bf16, pool> on the long-prefill workload",
           "kernel_source_sha256_16": kernel_source_hash(), "fetch_bytes_per_launch": fb,
           "write_bytes_per_launch": wb, "bytes_per_launch": fb + wb,
           "fetch_scale_from_copy": f_scale, "write_scale_from_copy": w_scale}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    pre = [r for r in stats if "prefill_kernel" in r["Name"]][0]
    avg_us = float(pre["AverageNs"]) / 1e3
    md = [f"# prefill_kernel (fused K1a + K1b + persist) — long prefill, B=1, S=131072, bf16", "",
          f"Kernel source hash (first 16 hex of sha256 of `qsa_kernels.hip` + `qsa_device.h`): "
          f"`{kernel_source_hash()}`.  MI355X (gfx950), one GPU.",
          f"Algorithmic bytes per launch: {alg:,}.", "", "## Kernel durations", "",
          "Command (run from `/tmp` with `TMPDIR=/tmp`; `R` is the repository root, `OUT` the "
          "directory that collects the profiler output):", "",
          "    " + PROFILE_CMDS["trace"], "",
          "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"].replace("qsa::(anonymous namespace)::", "").split("(")[0]
        md.append(f"| `{name[:80]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    md += ["", f"Fused kernel, on the path's algorithmic bytes (the three-call count, which "
           f"charges the block positions' cosSin rows once per consuming call): {alg_path:,} B / "
           f"{avg_us:.2f} us = {alg_path / avg_us / 1e6:.2f} TB/s = "
           f"{100 * alg_path / avg_us / 1e6 / 8:.1f} % of the 8 TB/s HBM peak.",
           f"On the bytes the fused launch itself must move: {alg:,} B / {avg_us:.2f} us = "
           f"{alg / avg_us / 1e6:.2f} TB/s = {100 * alg / avg_us / 1e6 / 8:.1f} %.", "",
           "## HBM traffic (counters)", "",
           "One counter per run; each run includes `torch.mul` over 256 MiB of float32, a "
           "reference kernel that reads and writes 268,435,456 B:", "",
           "    " + PROFILE_CMDS["fetch"], "    " + PROFILE_CMDS["write"], "",
           "| counter (KiB per dispatch) | reference kernel | scale | prefill_kernel | bytes |",
           "|---|---|---|---|---|",
           f"| FETCH_SIZE | {f_copy:,.0f} (for 262,144 read) | x {f_scale:.3f} | {f_k:,.0f} | "
           f"{fb:,.0f} |",
           f"| WRITE_SIZE | {w_copy:,.0f} (for 262,144 written) | x {w_scale:.3f} | {w_k:,.0f} | "
           f"{wb:,.0f} |", "",
           f"Measured {fb + wb:,.0f} B per launch against {alg:,} algorithmic "
           f"({100 * (fb + wb - alg) / alg:+.2f} %).", "",
           "Written by `python bench.py --summarize $OUT/ptrace $OUT/pfetch $OUT/pwrite`"
           " (also writes `traffic_prefill_kernel_long_prefill.json`)."]
    open(PROFILE_MD, "w").write("\n".join(md) + "\n")
    print("\n".join(md))
    summarize_next(stats, fetch, write, f_scale, w_scale)


NEXT_MD = os.path.join(ROOT, "profiles", "scores_select_long_prefill.md")


def summarize_next(stats, fetch, write, f_scale, w_scale):
    """profiles/ summary of the block-scores and top-512 selection kernels on the long
    prefill's rows [65536, 73728): durations from the same kernel trace, HBM bytes from the
    same FETCH_SIZE / WRITE_SIZE runs, against their algorithmic bytes."""
    S, nb = 131072, 32768
    r0, nr = SCORE_ROWS
    legs = [("scores_kernel", "`scores_kernel<Bf16>` (qsa_index_scores)",
             scores_alg(S, nb, r0, nr)[0]),
            ("topk_expand_reg_kernel", "`topk_expand_reg_kernel` (qsa_index_topk_expand)",
             select_alg(S, nb, r0, nr)),
            ("topk_expand_wave_kernel", "`topk_expand_wave_kernel` (qsa_index_topk_expand; "
             "rows [260096, 262144) of a 262144-token sequence x 65536 blocks)",
             select_alg(262144, 65536, 262144 - 2048, 2048))]
    md = ["# Block scores and top-512 selection — long prefill rows [65536, 73728) x 32768 "
          "blocks, bf16 (and the selection on rows past 32768 blocks)", "",
          "MI355X (gfx950), one GPU.  Kernel durations from the trace, HBM bytes from the "
          "counter runs of `prefill_kernel_long_prefill.md` (same commands, same scale factors "
          f"x {f_scale:.3f} for FETCH_SIZE and x {w_scale:.3f} for WRITE_SIZE).", "",
          "| kernel | avg us | algorithmic bytes | achieved | % of 8 TB/s | measured bytes "
          "(fetch + write) | vs algorithmic |", "|---|---|---|---|---|---|---|"]
    for key, label, alg in legs:
        rows = [r for r in stats if key in r["Name"]]
        if not rows:
            continue
        us = float(rows[0]["AverageNs"]) / 1e3
        fk = [v for k, v in fetch.items() if key in k]
        wk = [v for k, v in write.items() if key in k]
        meas = "—"
        rel = "—"
        if fk and wk:
            mb = fk[0][0] * 1024 * f_scale + wk[0][0] * 1024 * w_scale
            meas = f"{mb:,.0f} ({fk[0][0] * 1024 * f_scale:,.0f} + {wk[0][0] * 1024 * w_scale:,.0f})"
            rel = f"{100 * (mb - alg) / alg:+.1f} %"
        md.append(f"| {label} | {us:.1f} | {alg:,} | {alg / us / 1e6:.2f} TB/s | "
                  f"{100 * alg / us / 1e6 / 8:.1f} | {meas} | {rel} |")
    # decode kernels: the 64-sequence decode batch and the long-row decode batches
    import numpy as np
    from sparse_attention_indexer_qsa_amd import workloads as W
    wl4 = W.config4()
    dctx = (wl4.ranges[0] + 1).astype(np.int64)
    dmb = int((dctx.max() + 3) // 4)
    dn = np.minimum(dctx // 4, dmb)
    dec = [("scores_decode_kernel", "`scores_decode_kernel<Bf16>` (qsa_index_scores_decode, "
            "decode batch: 64 sequences, contexts up to 32772)", 260 * int(dn.sum()) + 1024 * 64),
           ("topk_expand_decode_reg_kernel", "`topk_expand_decode_reg_kernel` "
            "(qsa_index_topk_expand_decode, the same batch)",
            4 * int(dn[dn > 512].sum()) + 4 * 2051 * 64)]
    for mb, kpt in ((65536, 16), (262144, 64)):
        c = W.decode_long_ctx(mb).astype(np.int64)
        n = np.minimum(c // 4, mb)
        dec.append((f"topk_decode_chunk_kernel<{kpt}", f"`topk_decode_chunk_kernel<{kpt}>` "
                    f"(qsa_index_topk_expand_decode, 64 rows of {mb // 2} to {mb} blocks: "
                    f"chunk pass; the 16-bit candidate ids it stages are not counted)",
                    4 * int(n.sum())))
    dec.append(("topk_decode_merge_kernel", "`topk_decode_merge_kernel<8>` (merge pass of both "
                "long-row batches; its bytes: the staged ids, the candidates' keys and the "
                "8204-byte rows, not counted above)", None))
    md += ["", "## Decode kernels", "",
           "| kernel | calls | avg us | algorithmic bytes | achieved | % of 8 TB/s | measured "
           "bytes (fetch + write) |", "|---|---|---|---|---|---|---|"]
    for key, label, alg in dec:
        rows = [r for r in stats if key in r["Name"]]
        if not rows:
            continue
        us = float(rows[0]["AverageNs"]) / 1e3
        fk = [v for k, v in fetch.items() if key in k]
        wk = [v for k, v in write.items() if key in k]
        meas = "—"
        if fk and wk:
            mb_ = fk[0][0] * 1024 * f_scale + wk[0][0] * 1024 * w_scale
            meas = f"{mb_:,.0f} ({fk[0][0] * 1024 * f_scale:,.0f} + {wk[0][0] * 1024 * w_scale:,.0f})"
        ach = "—" if alg is None else f"{alg / us / 1e6:.2f} TB/s"
        frac = "—" if alg is None else f"{100 * alg / us / 1e6 / 8:.1f}"
        md.append(f"| {label} | {rows[0]['Calls']} | {us:.2f} | "
                  f"{'—' if alg is None else f'{alg:,}'} | {ach} | {frac} | {meas} |")
    md += ["", "Algorithmic bytes: scores = 4 B per (row, block) logit written + 1024 B of q per "
           "row + 256 B per kbar row any row sees; selection = 4 B per complete-block logit read "
           "+ 4 x 2051 B of token slots per row; decode scores = 256 B of V-tail read + 4 B "
           "written per visible block + 1024 B of q per sequence.", "",
           "Written by `python bench.py --summarize $OUT/ptrace $OUT/pfetch $OUT/pwrite`"
           "."]
    open(NEXT_MD, "w").write("\n".join(md) + "\n")
    print("\n".join(md))


CONFIG_MD = os.path.join(ROOT, "profiles", "config_legs.md")
CONFIG_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d $OUT/ctrace_$LEG -o run -- "
             "python3 $R/bench.py --only $LEG --steps 50 --warmup 5",
    "fetch": "timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE -f csv -d $OUT/cfetch_$LEG -o run "
             "-- python3 $R/bench.py --only $LEG --steps 10 --warmup 2 --copy-calib",
    "write": "timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE -f csv -d $OUT/cwrite_$LEG -o run "
             "-- python3 $R/bench.py --only $LEG --steps 10 --warmup 2 --copy-calib",
}


def summarize_configs(out_dir):
    """profiles/ summary of the five-workload legs: for each, the library's kernels from its
    own kernel trace and FETCH_SIZE / WRITE_SIZE runs (CONFIG_CMDS), counters scaled by what
    they read for the 256 MiB torch.mul reference of the same run; per step, the kernels of the
    fused launch and of the call sequence against the path's algorithmic bytes."""
    md = ["# The five workloads: kernel durations and HBM traffic", "",
          "MI355X (gfx950), one GPU.  One profiler run per workload and per counter; commands "
          "(from `/tmp`, `TMPDIR=/tmp`; `R` the repository root, `OUT` the profiler output "
          "directory, `LEG` the workload name):", ""]
    md += ["    " + c for c in CONFIG_CMDS.values()]
    md += ["", "Algorithmic bytes: the path's count for the run's seeded lengths and page table "
           "(`bench.path_bytes`): q rows read, distinct cosSin rows, every qNormed row written, "
           "raw keys of valid blocks, distinct cosSin rows of block positions, every kbar row "
           "of the range, raw-K tails (read + write), V-tails written, page entries read, "
           "gammas and lengths.  A kernel's 'measured' bytes are FETCH_SIZE and WRITE_SIZE per "
           "dispatch, scaled.", ""]
    ours = ("prefill_kernel", "q_prep_kernel", "k_compress_kernel", "persist_kernel")
    for leg in CONFIG_LEGS:
        tdir = os.path.join(out_dir, f"ctrace_{leg}")
        if not os.path.isdir(tdir):
            continue
        wl = _config_workload(leg)
        alg = path_bytes(wl, wl.run_q_prep)
        stats = _csv_rows(tdir, "kernel_stats.csv")
        fetch = _counter(os.path.join(out_dir, f"cfetch_{leg}"), "FETCH_SIZE")
        write = _counter(os.path.join(out_dir, f"cwrite_{leg}"), "WRITE_SIZE")

        def pick(d, key):
            ks = [k for k in d if key in k]
            return d[ks[0]][0] if ks else None
        f_scale = COPY_BYTES / (pick(fetch, "MulFunctor") * 1024)
        w_scale = COPY_BYTES / (pick(write, "MulFunctor") * 1024)
        md += [f"## {leg}: B={wl.B}, S={wl.S}, {wl.dt}", "",
               f"Algorithmic bytes per step: {alg:,}.  Counter scales: FETCH_SIZE x "
               f"{f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}.", "",
               "| kernel | calls | avg us | measured bytes (fetch + write) |", "|---|---|---|---|"]
        fused_us = seq_us = 0.0
        fused_b = seq_b = 0.0
        for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
            key = next((k for k in ours if k in r["Name"]), None)
            if key is None:
                continue
            name = r["Name"].replace("qsa::(anonymous namespace)::", "").split("(")[0]
            us = float(r["AverageNs"]) / 1e3
            fk = [v for k, v in fetch.items() if k == r["Name"]]
            wk = [v for k, v in write.items() if k == r["Name"]]
            mb = None
            if fk and wk:
                mb = fk[0][0] * 1024 * f_scale + wk[0][0] * 1024 * w_scale
            md.append(f"| `{name[:70]}` | {r['Calls']} | {us:.2f} | "
                      + (f"{mb:,.0f} ({fk[0][0] * 1024 * f_scale:,.0f} + "
                         f"{wk[0][0] * 1024 * w_scale:,.0f})" if mb is not None else "—") + " |")
            if key == "prefill_kernel":
                fused_us += us
                fused_b += mb or 0.0
            else:
                seq_us += us
                seq_b += mb or 0.0
        md.append("")
        for label, us, b in (("fused launch", fused_us, fused_b), ("call sequence", seq_us,
                                                                    seq_b)):
            if us > 0:
                md.append(f"- {label}: {us:.2f} us of kernel time per step = "
                          f"{alg / us / 1e3:,.0f} GB/s = {100 * alg / us / 1e3 / HBM_PEAK_GBPS:.1f} % "
                          f"of 8 TB/s on the algorithmic bytes; measured {b:,.0f} B "
                          f"({100 * (b - alg) / alg:+.1f} % vs algorithmic).")
        md.append("")
    md += ["Written by `python bench.py --summarize-configs $OUT`."]
    open(CONFIG_MD, "w").write("\n".join(md) + "\n")
    print("\n".join(md))


def _json_default(o):
    """numpy scalars in the result record become plain numbers."""
    if hasattr(o, "item"):
        return o.item()
    raise TypeError(f"{type(o)} is not JSON serializable")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=4, help="rotating buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="CPU oracle baseline: seconds of repeated passes (at least 3)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-three-call", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode pre-pass leg")
    ap.add_argument("--no-scores", action="store_true", help="skip the block-scores leg")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the cold-cache legs of the five workloads")
    ap.add_argument("--only", default=None,
                    help="comma-separated workload legs to run alone (of: "
                         + ", ".join(CONFIG_LEGS) + "); prints their results only")
    ap.add_argument("--summarize", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summary and traffic record from rocprofv3 output "
                         "(kernel trace, FETCH_SIZE run, WRITE_SIZE run) and exit")
    ap.add_argument("--summarize-configs", metavar="OUT",
                    help="write profiles/config_legs.md from the per-workload rocprofv3 runs "
                         "under OUT (ctrace_LEG, cfetch_LEG, cwrite_LEG) and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(*args.summarize)
        return
    if args.summarize_configs:
        summarize_configs(args.summarize_configs)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}): the indexer hot path needs no exchange between GPUs; run it once "
              f"per GPU, each on its own shard of sequences.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_indexer_qsa_amd.qsa as qsa
    from sparse_attention_indexer_qsa_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    def copy_calib():
        # a plain streaming kernel of known traffic: reads COPY_BYTES, writes COPY_BYTES
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 2.0, out=dst)
        torch.cuda.synchronize()

    def config_legs(names):
        res = {}
        for name in names:
            print(f"[bench] timing the {name} workload (cold cache)", file=sys.stderr,
                  flush=True)
            res[name] = config_leg(qsa, torch, name, min(args.steps, 50), min(args.warmup, 5))
        return res

    if args.only:
        names = [n for n in args.only.split(",") if n]
        assert all(n in CONFIG_LEGS for n in names), (names, CONFIG_LEGS)
        if args.copy_calib:
            copy_calib()
        print(json.dumps({"configs": config_legs(names)}, default=_json_default), flush=True)
        return

    print("[bench] generating the long-prefill workload", file=sys.stderr, flush=True)
    wl = W.config3()
    B, S, nb = wl.B, wl.S, wl.numBlocks
    dt = qsa.QSA_BF16

    def bits(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    wQ, wK = bits(wl.wQ), bits(wl.wK)
    host_x = torch.from_numpy(wl.indexQk.view(np.int16))
    host_cs = torch.from_numpy(wl.cosSin)
    sets = []
    for i in range(args.sets):
        x = host_x.cuda()
        cs = host_cs.cuda()
        ctx = torch.from_numpy(wl.ctx).cuda()
        pt = torch.from_numpy(wl.pool.pageTable).cuda()
        pool = torch.full(wl.pool.shape, 0xA5A5 - 65536, dtype=torch.int16, device="cuda")
        q = torch.empty(B, S, 4, 128, dtype=torch.int16, device="cuda")
        kb = torch.empty(B, nb, 128, dtype=torch.int16, device="cuda")
        ps = qsa.PoolState(pool, pt, wl.pool.numPages, wl.pool.numKVHeads, wl.pool.poolHeadDim,
                           wl.pool.headSize)
        sets.append(dict(x=x, cs=cs, ctx=ctx, pool=ps, q=q, kb=kb, pstruct=ps.c_struct(B)))
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()  # inputs made on the default stream are complete
    sh = stream.cuda_stream
    L = qsa.lib

    # arguments are marshalled once per buffer set; the timed loop only calls the C ABI
    def fused_args(s):
        return (s["q"].data_ptr(), s["kb"].data_ptr(), s["x"].data_ptr(), s["cs"].data_ptr(),
                S, s["ctx"].data_ptr(), wQ.data_ptr(), wK.data_ptr(), wl.eps,
                ctypes.byref(s["pstruct"]), B, S, nb, dt, sh)

    fa = [fused_args(s) for s in sets]

    def three_calls(s):
        rc = L.qsa_index_q_prep(s["q"].data_ptr(), s["x"].data_ptr(), s["cs"].data_ptr(), S,
                                s["ctx"].data_ptr(), wQ.data_ptr(), wl.eps, B, S, dt, sh)
        rc |= L.qsa_index_k_compress(s["kb"].data_ptr(), s["x"].data_ptr(), s["cs"].data_ptr(), S,
                                     s["ctx"].data_ptr(), wK.data_ptr(), wl.eps, B, S, nb, 0, nb,
                                     0, None, ctypes.byref(s["pstruct"]), dt, sh)
        rc |= L.qsa_index_persist(ctypes.byref(s["pstruct"]), s["x"].data_ptr(), None,
                                  s["ctx"].data_ptr(), B, S, nb, 0, nb, 0, None, dt, sh)
        return rc

    torch.cuda.synchronize()

    def timed(fn, steps, warmup):
        with torch.cuda.stream(stream):
            for i in range(warmup):
                assert fn(i % args.sets) == 0, qsa.qsa_last_error()
            torch.cuda.synchronize()          # barrier (one rank) + device sync
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0 = time.perf_counter()
            e0.record(stream)
            for i in range(steps):
                fn(i % args.sets)
            e1.record(stream)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
        return (t1 - t0) / steps, e0.elapsed_time(e1) / 1e3 / steps

    print("[bench] timing the fused prefill", file=sys.stderr, flush=True)
    wall, ev = timed(lambda i: L.qsa_index_prefill(*fa[i]), args.steps, args.warmup)
    # per-launch distribution (events around each launch, same stream)
    per = []
    with torch.cuda.stream(stream):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(min(args.steps, 100))]
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            L.qsa_index_prefill(*fa[i % args.sets])
            b.record(stream)
        torch.cuda.synchronize()
        per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    three = None
    if not args.no_three_call:
        print("[bench] timing the three-call sequence", file=sys.stderr, flush=True)
        w3, e3 = timed(lambda i: three_calls(sets[i]), args.steps, args.warmup)
        three = {"ms_per_step": w3 * 1e3, "event_ms_per_step": e3 * 1e3,
                 "rows_per_s": B * S / w3, "GBps_alg": path_bytes(wl) / e3 / 1e9}
    if args.copy_calib:
        copy_calib()

    scores = select = select_long = select_decode = scores_decode = select_decode_long = None
    if not args.no_scores:
        print("[bench] timing the block scores", file=sys.stderr, flush=True)
        logits, scores = scores_leg(qsa, torch, sets[0], wl, min(args.steps, 50),
                                    min(args.warmup, 5))
        print("[bench] timing the top-512 selection", file=sys.stderr, flush=True)
        select = select_leg(qsa, torch, wl, logits, min(args.steps, 50), min(args.warmup, 5))
        del logits
        print("[bench] timing the selection on rows past 32768 blocks", file=sys.stderr,
              flush=True)
        select_long = select_long_leg(qsa, torch, min(args.steps, 50), min(args.warmup, 5))
        select_decode = select_decode_leg(qsa, torch, min(args.steps, 100), min(args.warmup, 10))
        print("[bench] timing the decode selection on long rows", file=sys.stderr, flush=True)
        select_decode_long = [select_decode_long_leg(qsa, torch, min(args.steps, 50),
                                                     min(args.warmup, 5), mb)
                              for mb in (65536, 262144)]
        scores_decode = scores_decode_leg(qsa, torch, min(args.steps, 100), min(args.warmup, 10))
    decode = None
    if not args.no_decode:
        print("[bench] timing the decode pre-pass", file=sys.stderr, flush=True)
        del sets, fa
        torch.cuda.empty_cache()
        decode = decode_leg(qsa, torch, args.steps, args.warmup)

    configs = None
    if not args.no_configs:
        configs = config_legs(CONFIG_LEGS)

    alg = path_bytes(wl)                 # the path's algorithmic bytes of one step
    alg_fused = algorithmic_bytes(wl)    # what the fused launch itself must move
    achieved = alg / ev / 1e9
    print("[bench] timing the copy reference", file=sys.stderr, flush=True)
    copy_ref = copy_reference(qsa, torch, alg_fused, min(args.steps, 100), min(args.warmup, 10))
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        t = json.load(open(TRAFFIC_FILE))
        if t.get("kernel_source_sha256_16") == kernel_source_hash():
            traffic = t["bytes_per_launch"]
    out = {
        "metric": METRIC, "value": B * S / wall, "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "long_prefill", "B": B, "S": S, "T": "bf16", "theta": 1e6,
                   "numBlocks": nb, "numPages": wl.pool.numPages, "entry": "qsa_index_prefill",
                   "buffer_sets": args.sets,
                   "timers": "value and ms_per_step: host wall clock around the timed launches "
                             "(synchronised before and after); roofline.achieved: HIP events "
                             "on the launch stream over the same launches"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "alg_bytes": alg, "event_us": ev * 1e6,
                     "fused_launch_bytes": alg_fused,
                     "frac_on_fused_launch_bytes": alg_fused / ev / 1e9 / HBM_PEAK_GBPS},
        "kernel": {"name": "prefill_kernel<Bf16, pool>", "alg_bytes_per_launch": alg,
                   "fused_launch_bytes": alg_fused,
                   "event_us_per_launch": ev * 1e6,
                   "us_p10_p50_p90": [per[len(per) // 10], per[len(per) // 2],
                                      per[(9 * len(per)) // 10]],
                   "source_sha256_16": kernel_source_hash(), "copy_reference": copy_ref},
        "three_call": three,
        "decode_pre_pass": decode,
        "scores": scores,
        "select": select,
        "select_long_rows": select_long,
        "scores_decode": scores_decode,
        "select_decode": select_decode,
        "select_decode_long_rows": select_decode_long,
        "configs": configs,
    }
    if not args.no_cpu:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out, default=_json_default), flush=True)


if __name__ == "__main__":
    main()
