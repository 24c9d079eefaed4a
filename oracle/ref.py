"""ctypes front end of the CPU oracle (``libqsa_ref.so``) — TEST INFRASTRUCTURE ONLY.

Arrays are numpy, C-contiguous; T tensors travel as ``uint16`` bit patterns.  The parameter
lists mirror the GPU library's entry points, with host arrays in place of device pointers.
Each function returns new output arrays; pools are updated in place, like the device pool.

``Oracle(path)`` binds a specific build of the oracle (the tests also build deliberately
broken copies to show that the pins catch them); the module-level functions use the default
build.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F16, BF16 = 0, 1
DTYPES = {"f16": F16, "fp16": F16, "bf16": BF16}


class RefPool(ctypes.Structure):
    """The oracle's own mirror of the page's QsaIndexerPoolState."""
    _fields_ = [("poolPtr", ctypes.c_void_p), ("pageTable", ctypes.c_void_p),
                ("maxPagesPerSeq", ctypes.c_int32), ("numPages", ctypes.c_int32),
                ("numKVHeads", ctypes.c_int32), ("poolHeadDim", ctypes.c_int32),
                ("headSize", ctypes.c_int32)]


def _dt(dt):
    return DTYPES[dt] if isinstance(dt, str) else int(dt)


def _p(a):
    """Pointer to a C-contiguous numpy array (None stays NULL)."""
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


class Pool:
    """Host pool of the oracle: ``data`` is uint16 [2*numPages, 128, H, D]."""

    def __init__(self, data, pageTable, numPages, headSize):
        self.data = data
        self.pageTable = _i32(pageTable)
        self.numPages = int(numPages)
        self.headSize = int(headSize)
        assert data.dtype == np.uint16 and data.flags["C_CONTIGUOUS"]
        assert data.shape[0] == 2 * numPages and data.shape[1] == 128
        assert self.pageTable.ndim == 3 and self.pageTable.shape[1] == 2

    def c_struct(self):
        return RefPool(self.data.ctypes.data, self.pageTable.ctypes.data,
                       self.pageTable.shape[2], self.numPages, self.data.shape[2],
                       self.data.shape[3], self.headSize)


def _ranges(ranges):
    if ranges is None:
        return None, None, None, 0
    pastLens, blockBegins, blockEnds, maxSpan = ranges
    return _i32(pastLens), _i32(blockBegins), _i32(blockEnds), int(maxSpan)


class Oracle:
    def __init__(self, path=None):
        path = path or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        self.path = path
        L = ctypes.CDLL(path)
        P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        L.ref_q_prep.argtypes = [P, P, P, I32, P, P, F32, I32, I32, ctypes.c_int, P, P, P]
        L.ref_k_compress.argtypes = [P, P, P, I32, P, P, F32, I32, I32, I32, I32, I32, I32,
                                     P, P, P, I32, P, ctypes.c_int, P, P, P, P]
        L.ref_persist.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, I32]
        L.ref_pre_decode.argtypes = [P, P, P, I32, P, P, P, P, F32, P, I32, I32, ctypes.c_int]
        L.ref_scores.argtypes = [P, P, P, P, I32, I32, I32, I32, I32, ctypes.c_int]
        L.ref_scores_decode.argtypes = [P, P, P, P, I32, I32, ctypes.c_int]
        L.ref_score_scale.restype = ctypes.c_float
        L.ref_ids_fill.argtypes = [P, I32, I32]
        L.ref_expand.argtypes = [P, P, P, I32, I32, I32, I32, I32]
        L.ref_topk_expand.argtypes = [P, P, P, P, I32, I32, I32, I32, I32]
        L.ref_topk_expand_decode.argtypes = [P, P, P, P, I32, I32, I32]
        L.ref_widen.argtypes = [P, P, I64, ctypes.c_int]
        L.ref_narrow.argtypes = [P, P, I64, ctypes.c_int]
        L.ref_set_threads.argtypes = [ctypes.c_int]
        L.ref_max_threads.restype = ctypes.c_int
        for f in (L.ref_q_prep, L.ref_k_compress, L.ref_persist, L.ref_widen, L.ref_narrow,
                  L.ref_set_threads, L.ref_pre_decode, L.ref_scores, L.ref_scores_decode,
                  L.ref_ids_fill, L.ref_expand, L.ref_topk_expand, L.ref_topk_expand_decode):
            f.restype = None
        self.L = L

    def set_threads(self, n):
        self.L.ref_set_threads(int(n))

    def max_threads(self):
        return self.L.ref_max_threads()

    def widen(self, bits, dt):
        bits = _u16(bits)
        out = np.empty(bits.shape, np.float32)
        self.L.ref_widen(_p(bits), _p(out), bits.size, _dt(dt))
        return out

    def narrow(self, values, dt):
        values = np.ascontiguousarray(values, dtype=np.float32)
        out = np.empty(values.shape, np.uint16)
        self.L.ref_narrow(_p(values), _p(out), values.size, _dt(dt))
        return out

    def q_prep(self, indexQk, cosSin, ctx, wQ, eps, dt, debug=False):
        """K1a.  indexQk uint16 [B,S,640] -> qNormed uint16 [B,S,4,128] (and debug dict)."""
        indexQk, wQ = _u16(indexQk), _u16(wQ)
        cosSin = np.ascontiguousarray(cosSin, dtype=np.float32)
        ctx = _i32(ctx)
        B, S, W = indexQk.shape
        assert W == 640 and wQ.shape == (128,) and cosSin.shape[1] == 64
        assert ctx.shape == (B,)
        q = np.empty((B, S, 4, 128), np.uint16)
        dbg = None
        if debug:
            dbg = {"meanSq": np.empty((B, S, 4), np.float32),
                   "invRms": np.empty((B, S, 4), np.float32),
                   "preCast": np.empty((B, S, 4, 128), np.float32)}
        d = dbg or {}
        self.L.ref_q_prep(_p(q), _p(indexQk), _p(cosSin), cosSin.shape[0], _p(ctx), _p(wQ),
                          float(eps), B, S, _dt(dt), _p(d.get("meanSq")), _p(d.get("invRms")),
                          _p(d.get("preCast")))
        return (q, dbg) if debug else q

    def k_compress(self, indexQk, cosSin, ctx, wK, eps, numBlocks, blockBegin, blockEnd,
                   pastLen, dt, kbar=None, ranges=None, pool=None, debug=False,
                   maxPositions=None):
        """K1b.  Returns kbar uint16 [B,numBlocks,128]; rows outside the range keep `kbar`'s
        initial content (zeros when `kbar` is None).  `ranges` = (pastLens, blockBegins,
        blockEnds, maxBlockSpan) or None; `pool` = Pool or None (V-tails written in place)."""
        indexQk, wK = _u16(indexQk), _u16(wK)
        cosSin = np.ascontiguousarray(cosSin, dtype=np.float32)
        ctx = _i32(ctx)
        B, S, W = indexQk.shape
        assert W == 640 and ctx.shape == (B,)
        out = np.zeros((B, numBlocks, 128), np.uint16) if kbar is None else _u16(kbar).copy()
        assert out.shape == (B, numBlocks, 128)
        pl, bb, be, ms = _ranges(ranges)
        ps = pool.c_struct() if pool is not None else None
        dbg = None
        if debug:
            dbg = {"mT": np.zeros((B, numBlocks, 128), np.uint16),
                   "meanSq": np.zeros((B, numBlocks), np.float32),
                   "invRms": np.zeros((B, numBlocks), np.float32),
                   "preCast": np.zeros((B, numBlocks, 128), np.float32)}
        d = dbg or {}
        mp = cosSin.shape[0] if maxPositions is None else int(maxPositions)
        self.L.ref_k_compress(_p(out), _p(indexQk), _p(cosSin), mp, _p(ctx), _p(wK), float(eps),
                              B, S, numBlocks, blockBegin, blockEnd, pastLen, _p(pl), _p(bb),
                              _p(be), ms, ctypes.byref(ps) if ps is not None else None,
                              _dt(dt), _p(d.get("mT")), _p(d.get("meanSq")),
                              _p(d.get("invRms")), _p(d.get("preCast")))
        return (out, dbg) if debug else out

    def persist(self, pool, indexQk, kbar, ctx, numBlocks, blockBegin, blockEnd, pastLen,
                ranges=None):
        """Raw-K tails and (kbar given) V-tails into `pool` (in place).  A bit copy: the
        element type does not enter."""
        indexQk = _u16(indexQk)
        kbar = None if kbar is None else _u16(kbar)
        ctx = _i32(ctx)
        B, S, _ = indexQk.shape
        pl, bb, be, ms = _ranges(ranges)
        ps = pool.c_struct()
        self.L.ref_persist(ctypes.byref(ps), _p(indexQk), _p(kbar), _p(ctx), B, S, numBlocks,
                           blockBegin, blockEnd, pastLen, _p(pl), _p(bb), _p(be), ms)


    def pre_decode(self, indexQk, cosSin, ctx, newLens, wQ, wK, eps, pool, dt,
                   maxPositions=None):
        """Decode pre-pass.  indexQk uint16 [B,S,640] holds each sequence's new tokens in rows
        0..n-1; ctx = TOTAL lengths; newLens int32 [B] or None (one new token).  Returns
        qNormed uint16 [B,S,4,128]; K-tails and V-tails go to `pool` in place."""
        indexQk, wQ, wK = _u16(indexQk), _u16(wQ), _u16(wK)
        cosSin = np.ascontiguousarray(cosSin, dtype=np.float32)
        ctx = _i32(ctx)
        nl = None if newLens is None else _i32(newLens)
        B, S, W = indexQk.shape
        assert W == 640 and ctx.shape == (B,)
        q = np.empty((B, S, 4, 128), np.uint16)
        ps = pool.c_struct()
        mp = cosSin.shape[0] if maxPositions is None else int(maxPositions)
        self.L.ref_pre_decode(_p(q), _p(indexQk), _p(cosSin), mp, _p(ctx), _p(nl), _p(wQ),
                              _p(wK), float(eps), ctypes.byref(ps), B, S, _dt(dt))
        return q


    def scores(self, qNormed, kbar, ctx, rowStart, numRows, dt):
        """Block scores.  qNormed uint16 [B,S,4,128], kbar uint16 [B,numBlocks,128] ->
        logits float32 [numRows, numBlocks] for global rows [rowStart, rowStart+numRows)."""
        qNormed, kbar = _u16(qNormed), _u16(kbar)
        ctx = _i32(ctx)
        B, S = qNormed.shape[:2]
        nb = kbar.shape[1]
        out = np.empty((numRows, nb), np.float32)
        self.L.ref_scores(_p(out), _p(qNormed), _p(kbar), _p(ctx), B, S, nb, rowStart, numRows,
                          _dt(dt))
        return out

    def scores_decode(self, qNormed, ctx, pool, maxBlocks, dt, logits=None):
        """Decode block scores from V-tails.  qNormed uint16 [B,1,4,128] (or [B,4,128]);
        returns logits float32 [B, maxBlocks]; entries past each row's prefix keep `logits`'s
        content (NaN when None)."""
        qNormed = _u16(qNormed)
        ctx = _i32(ctx)
        B = qNormed.shape[0]
        out = np.full((B, maxBlocks), np.nan, np.float32) if logits is None else \
            np.ascontiguousarray(logits, np.float32).copy()
        ps = pool.c_struct()
        self.L.ref_scores_decode(_p(out), _p(qNormed), _p(ctx), ctypes.byref(ps), B, maxBlocks,
                                 _dt(dt))
        return out

    def ids_fill(self, numRows, numBlocks):
        ids = np.empty((numRows, numBlocks), np.int32)
        self.L.ref_ids_fill(_p(ids), numRows, numBlocks)
        return ids

    def expand(self, sortedIds, ctx, B, S, rowStart, numRows, outIdx=None):
        """K4: outIdx int32 [B*S, 2051]; rows outside the chunk keep `outIdx` (zeros)."""
        sortedIds = _i32(sortedIds)
        ctx = _i32(ctx)
        out = np.zeros((B * S, 2051), np.int32) if outIdx is None else _i32(outIdx).copy()
        self.L.ref_expand(_p(out), _p(sortedIds), _p(ctx), B, S, sortedIds.shape[1], rowStart,
                          numRows)
        return out

    def topk_expand(self, logits, ctx, B, S, rowStart, numRows, outIdx=None):
        """Prefill selection: full stable descending sort of each row, then K4.  Returns
        (outIdx [B*S, 2051], sortedIds [numRows, numBlocks])."""
        logits = np.ascontiguousarray(logits, np.float32)
        ctx = _i32(ctx)
        nb = logits.shape[1]
        out = np.zeros((B * S, 2051), np.int32) if outIdx is None else _i32(outIdx).copy()
        srt = np.empty((numRows, nb), np.int32)
        self.L.ref_topk_expand(_p(out), _p(srt), _p(logits), _p(ctx), B, S, nb, rowStart,
                               numRows)
        return out, srt

    def topk_expand_decode(self, logits, ctx, splitCounters=None):
        """Decode selection: logits float32 [B, maxBlocks] -> outIdx int32 [B, 2051]; with
        splitCounters int32 [B, numKVHeads] given, returns (outIdx, the counters after)."""
        logits = np.ascontiguousarray(logits, np.float32)
        ctx = _i32(ctx)
        B, mb = logits.shape
        out = np.empty((B, 2051), np.int32)
        sc = None if splitCounters is None else _i32(splitCounters).copy()
        self.L.ref_topk_expand_decode(_p(out), _p(logits), _p(ctx),
                                      None if sc is None else _p(sc),
                                      0 if sc is None else sc.shape[1], B, mb)
        return out if sc is None else (out, sc)

    def score_scale(self):
        return self.L.ref_score_scale()


_default = None


def default():
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def __getattr__(name):
    # module-level q_prep / k_compress / persist / widen / narrow / ... use the default build
    if name in ("q_prep", "k_compress", "persist", "widen", "narrow", "set_threads",
                "max_threads", "pre_decode", "scores", "scores_decode", "score_scale", "ids_fill",
                "expand", "topk_expand", "topk_expand_decode"):
        return getattr(default(), name)
    raise AttributeError(name)
