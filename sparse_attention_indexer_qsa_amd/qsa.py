"""Python binding of libqsa.so (the C ABI of include/qsa.h).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
Each function has the name of the C entry point it calls and takes torch tensors where the C
function takes device pointers.  Before calling, the binding checks what C cannot see: that
every tensor is a contiguous tensor on the current GPU, with the dtype and at least the size
that the sizes passed to the kernel imply.  A non-OK status raises ``QsaError`` carrying the
library's error text.  T tensors may be torch.float16 / torch.bfloat16, or int16 bit patterns
when ``dt`` is given.

If libqsa.so is missing, importing this module raises ImportError: there is no fallback.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_F16, QSA_BF16 = 0, 1
QSA_OK, QSA_E_INVALID, QSA_E_ALIGN, QSA_E_DTYPE, QSA_E_LAUNCH, QSA_E_NO_DEVICE = \
    0, -1, -2, -3, -4, -5
ROW_WIDTH, HEAD_DIM, HEADS = 640, 128, 4
TOPK, INDEX_WIDTH = 512, 2051

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                      f"python -m sparse_attention_indexer_qsa_amd.build")


class qsa_pool_state_t(ctypes.Structure):
    _fields_ = [("poolPtr", ctypes.c_void_p), ("pageTable", ctypes.c_void_p),
                ("maxPagesPerSeq", ctypes.c_int32), ("numPages", ctypes.c_int32),
                ("numKVHeads", ctypes.c_int32), ("poolHeadDim", ctypes.c_int32),
                ("headSize", ctypes.c_int32)]


class qsa_seq_ranges_t(ctypes.Structure):
    _fields_ = [("pastLens", ctypes.c_void_p), ("blockBegins", ctypes.c_void_p),
                ("blockEnds", ctypes.c_void_p), ("maxBlockSpan", ctypes.c_int32)]


def _declare(lib):
    P, I, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    sig = {
        "qsa_index_q_prep": [P, P, P, I, P, P, F, I, I, ctypes.c_int, P],
        "qsa_debug_q_prep": [P, P, P, I, P, P, F, I, I, ctypes.c_int, P, P, P, P],
        "qsa_index_k_compress": [P, P, P, I, P, P, F, I, I, I, I, I, I, P, P, ctypes.c_int, P],
        "qsa_debug_k_compress": [P, P, P, I, P, P, F, I, I, I, I, I, I, P, P, ctypes.c_int, P,
                                 P, P, P, P],
        "qsa_index_persist": [P, P, P, P, I, I, I, I, I, I, P, ctypes.c_int, P],
        "qsa_index_prefill": [P, P, P, P, I, P, P, P, F, P, I, I, I, ctypes.c_int, P],
        "qsa_index_pre_decode": [P, P, P, I, P, P, P, P, F, P, I, I, ctypes.c_int, P],
        "qsa_index_scores": [P, P, P, P, I, I, I, I, I, ctypes.c_int, P],
        "qsa_index_scores_decode": [P, P, P, P, I, I, ctypes.c_int, P],
        "qsa_index_ids_fill": [P, I, I, P],
        "qsa_index_expand": [P, P, P, I, I, I, I, I, P],
        "qsa_index_topk_expand": [P, P, P, I, I, I, I, I, P],
        "qsa_index_topk_expand_decode": [P, P, P, P, I, I, I, P],
        "qsa_stream_copy": [P, P, ctypes.c_int64, P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.qsa_last_error.argtypes = []
    lib.qsa_last_error.restype = ctypes.c_char_p
    lib.qsa_abi_version.argtypes = []
    lib.qsa_abi_version.restype = ctypes.c_int
    return lib


lib = _declare(ctypes.CDLL(LIB_PATH))


class QsaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"qsa status {code}: {msg}")
        self.code = code


def _check(rc):
    if rc != QSA_OK:
        raise QsaError(rc, lib.qsa_last_error().decode())


def _dt_of(t, dt):
    if dt is not None:
        return {"f16": QSA_F16, "fp16": QSA_F16, "bf16": QSA_BF16}.get(dt, dt)
    if t.dtype == torch.bfloat16:
        return QSA_BF16
    if t.dtype == torch.float16:
        return QSA_F16
    raise TypeError(f"cannot infer T from {t.dtype}; pass dt='bf16' or dt='f16'")


def _dev(t, name, min_numel, dtypes):
    """Pointer of a contiguous tensor on the current GPU holding >= min_numel elements."""
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} must live on the current GPU (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_numel}")
    return t.data_ptr()


_T = (torch.float16, torch.bfloat16, torch.int16)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


class PoolState:
    """qsa_pool_state_t over a pool tensor [2*numPages, 128, numKVHeads, poolHeadDim] and a
    page table int32 [B, 2, maxPagesPerSeq]."""

    def __init__(self, pool, pageTable, numPages, numKVHeads, poolHeadDim, headSize):
        self.pool, self.pageTable = pool, pageTable
        self.numPages, self.numKVHeads = int(numPages), int(numKVHeads)
        self.poolHeadDim, self.headSize = int(poolHeadDim), int(headSize)

    def c_struct(self, batchSize):
        if self.pageTable.dim() != 3 or self.pageTable.shape[1] != 2:
            raise ValueError("pageTable must be [B, 2, maxPagesPerSeq]")
        m = self.pageTable.shape[2]
        pt = _dev(self.pageTable, "pageTable", batchSize * 2 * m, _I32)
        pp = _dev(self.pool, "pool", 2 * self.numPages * 128 * self.numKVHeads * self.poolHeadDim,
                  _T)
        return qsa_pool_state_t(pp, pt, m, self.numPages, self.numKVHeads, self.poolHeadDim,
                                self.headSize)


class SeqRanges:
    """qsa_seq_ranges_t: per-sequence pastLens / blockBegins / blockEnds (int32 [B])."""

    def __init__(self, pastLens, blockBegins, blockEnds, maxBlockSpan):
        self.pastLens, self.blockBegins, self.blockEnds = pastLens, blockBegins, blockEnds
        self.maxBlockSpan = int(maxBlockSpan)

    def c_struct(self, batchSize):
        return qsa_seq_ranges_t(_dev(self.pastLens, "pastLens", batchSize, _I32),
                                _dev(self.blockBegins, "blockBegins", batchSize, _I32),
                                _dev(self.blockEnds, "blockEnds", batchSize, _I32),
                                self.maxBlockSpan)


def _ref(s):
    return None if s is None else ctypes.byref(s)


def qsa_index_q_prep(qNormed, indexQk, cosSin, contextLengths, wQ, rmsEps, batchSize=None,
                     seqLen=None, dt=None, stream=None, debug=None):
    """K1a.  indexQk [B,S,640] -> qNormed [B,S,4,128].  `debug` = dict of FP32 tensors
    meanSq [B,S,4], invRms [B,S,4], preCast [B,S,4,128] selects qsa_debug_q_prep."""
    B = indexQk.shape[0] if batchSize is None else batchSize
    S = indexQk.shape[1] if seqLen is None else seqLen
    if B == 0 or S == 0:
        return
    P = cosSin.shape[0]
    args = [_dev(qNormed, "qNormed", B * S * HEADS * HEAD_DIM, _T),
            _dev(indexQk, "indexQk", B * S * ROW_WIDTH, _T),
            _dev(cosSin, "cosSin", P * 64, _F32), P,
            _dev(contextLengths, "contextLengths", B, _I32), _dev(wQ, "wQ", HEAD_DIM, _T),
            float(rmsEps), B, S, _dt_of(indexQk, dt), _stream(stream)]
    if debug is None:
        _check(lib.qsa_index_q_prep(*args))
    else:
        _check(lib.qsa_debug_q_prep(*args, _dev(debug["meanSq"], "meanSq", B * S * 4, _F32),
                                    _dev(debug["invRms"], "invRms", B * S * 4, _F32),
                                    _dev(debug["preCast"], "preCast", B * S * 512, _F32)))


def qsa_index_k_compress(kbar, indexQk, cosSin, contextLengths, wK, rmsEps, numBlocks,
                         blockBegin, blockEnd, pastLen, ranges=None, pool=None, batchSize=None,
                         seqLen=None, dt=None, stream=None, debug=None):
    """K1b (and with `pool`, the V-tail write).  kbar [B,numBlocks,128]; `ranges` = SeqRanges;
    `debug` = dict mT (T) [B,nb,128], meanSq [B,nb], invRms [B,nb], preCast [B,nb,128]."""
    B = indexQk.shape[0] if batchSize is None else batchSize
    S = indexQk.shape[1] if seqLen is None else seqLen
    span = (blockEnd - blockBegin) if ranges is None else ranges.maxBlockSpan
    if B == 0 or span <= 0:
        if ranges is None:  # nothing to launch; the library still validates the scalars
            _check(lib.qsa_index_k_compress(None, None, None, cosSin.shape[0], None, None,
                                            float(rmsEps), B, S, numBlocks, blockBegin,
                                            blockEnd, pastLen, None, None, _dt_of(indexQk, dt),
                                            None))
        return
    P = cosSin.shape[0]
    rs = None if ranges is None else ranges.c_struct(B)
    ps = None if pool is None else pool.c_struct(B)
    args = [_dev(kbar, "kbar", B * numBlocks * HEAD_DIM, _T),
            _dev(indexQk, "indexQk", B * S * ROW_WIDTH, _T), _dev(cosSin, "cosSin", P * 64, _F32),
            P, _dev(contextLengths, "contextLengths", B, _I32), _dev(wK, "wK", HEAD_DIM, _T),
            float(rmsEps), B, S, numBlocks, blockBegin, blockEnd, pastLen, _ref(rs), _ref(ps),
            _dt_of(indexQk, dt), _stream(stream)]
    if debug is None:
        _check(lib.qsa_index_k_compress(*args))
    else:
        n = B * numBlocks
        _check(lib.qsa_debug_k_compress(*args, _dev(debug["mT"], "mT", n * HEAD_DIM, _T),
                                        _dev(debug["meanSq"], "meanSq", n, _F32),
                                        _dev(debug["invRms"], "invRms", n, _F32),
                                        _dev(debug["preCast"], "preCast", n * HEAD_DIM, _F32)))


def qsa_index_persist(pool, indexQk, kbar, contextLengths, numBlocks, blockBegin, blockEnd,
                      pastLen, ranges=None, batchSize=None, seqLen=None, dt=None, stream=None):
    """Raw-K tails, and with `kbar` the V-tails, into `pool` (a PoolState)."""
    B = indexQk.shape[0] if batchSize is None else batchSize
    S = indexQk.shape[1] if seqLen is None else seqLen
    if B == 0 or S == 0:
        return
    rs = None if ranges is None else ranges.c_struct(B)
    kb = None if kbar is None else _dev(kbar, "kbar", B * numBlocks * HEAD_DIM, _T)
    _check(lib.qsa_index_persist(ctypes.byref(pool.c_struct(B)),
                                 _dev(indexQk, "indexQk", B * S * ROW_WIDTH, _T), kb,
                                 _dev(contextLengths, "contextLengths", B, _I32), B, S, numBlocks,
                                 blockBegin, blockEnd, pastLen, _ref(rs), _dt_of(indexQk, dt),
                                 _stream(stream)))


def qsa_index_prefill(qNormed, kbar, indexQk, cosSin, contextLengths, wQ, wK, rmsEps,
                      numBlocks, pool=None, batchSize=None, seqLen=None, dt=None, stream=None):
    """K1a + K1b(0, ceilDiv(S,4), 0) + V-tails + raw-K tails in one launch."""
    B = indexQk.shape[0] if batchSize is None else batchSize
    S = indexQk.shape[1] if seqLen is None else seqLen
    if B == 0 or S == 0:
        return
    P = cosSin.shape[0]
    ps = None if pool is None else pool.c_struct(B)
    _check(lib.qsa_index_prefill(_dev(qNormed, "qNormed", B * S * HEADS * HEAD_DIM, _T),
                                 _dev(kbar, "kbar", B * numBlocks * HEAD_DIM, _T),
                                 _dev(indexQk, "indexQk", B * S * ROW_WIDTH, _T),
                                 _dev(cosSin, "cosSin", P * 64, _F32), P,
                                 _dev(contextLengths, "contextLengths", B, _I32),
                                 _dev(wQ, "wQ", HEAD_DIM, _T), _dev(wK, "wK", HEAD_DIM, _T),
                                 float(rmsEps), _ref(ps), B, S, numBlocks, _dt_of(indexQk, dt),
                                 _stream(stream)))


def qsa_index_pre_decode(qNormed, indexQk, cosSin, contextLengths, wQ, wK, rmsEps, pool,
                         newLens=None, batchSize=None, seqLen=None, dt=None, stream=None):
    """Decode pre-pass: K1a of the new tokens (rows 0..n-1 of each sequence), raw-K tails, and
    the kbar V-tails of blocks the new tokens complete.  `newLens` int32 [B] or None (one)."""
    B = indexQk.shape[0] if batchSize is None else batchSize
    S = indexQk.shape[1] if seqLen is None else seqLen
    if B == 0:
        return
    P = cosSin.shape[0]
    nl = None if newLens is None else _dev(newLens, "newLens", B, _I32)
    _check(lib.qsa_index_pre_decode(_dev(qNormed, "qNormed", B * S * HEADS * HEAD_DIM, _T),
                                    _dev(indexQk, "indexQk", B * S * ROW_WIDTH, _T),
                                    _dev(cosSin, "cosSin", P * 64, _F32), P,
                                    _dev(contextLengths, "contextLengths", B, _I32), nl,
                                    _dev(wQ, "wQ", HEAD_DIM, _T), _dev(wK, "wK", HEAD_DIM, _T),
                                    float(rmsEps), ctypes.byref(pool.c_struct(B)), B, S,
                                    _dt_of(indexQk, dt), _stream(stream)))


def qsa_index_scores(logits, qNormed, kbar, contextLengths, numBlocks, rowStart, numRows,
                     batchSize=None, seqLen=None, dt=None, stream=None):
    """Block scores of global rows [rowStart, rowStart+numRows): logits FP32 [numRows,
    numBlocks] from qNormed [B,S,4,128] and kbar [B,numBlocks,128]."""
    B = qNormed.shape[0] if batchSize is None else batchSize
    S = qNormed.shape[1] if seqLen is None else seqLen
    if numRows == 0 or numBlocks == 0:
        return
    _check(lib.qsa_index_scores(_dev(logits, "logits", numRows * numBlocks, _F32),
                                _dev(qNormed, "qNormed", B * S * HEADS * HEAD_DIM, _T),
                                _dev(kbar, "kbar", B * numBlocks * HEAD_DIM, _T),
                                _dev(contextLengths, "contextLengths", B, _I32), B, S, numBlocks,
                                rowStart, numRows, _dt_of(qNormed, dt), _stream(stream)))


def qsa_index_scores_decode(logits, qNormed, contextLengths, pool, maxBlocks, batchSize=None,
                            dt=None, stream=None):
    """Decode block scores against the V-tails: logits FP32 [B, maxBlocks], prefix
    [0, ctx/4) of each row written."""
    B = qNormed.shape[0] if batchSize is None else batchSize
    if B == 0 or maxBlocks == 0:
        return
    _check(lib.qsa_index_scores_decode(_dev(logits, "logits", B * maxBlocks, _F32),
                                       _dev(qNormed, "qNormed", B * HEADS * HEAD_DIM, _T),
                                       _dev(contextLengths, "contextLengths", B, _I32),
                                       ctypes.byref(pool.c_struct(B)), B, maxBlocks,
                                       _dt_of(qNormed, dt), _stream(stream)))


def qsa_stream_copy(dst, src, stream=None):
    """Measurement helper: copy all bytes of src into dst (same byte size, a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError(f"dst holds {dst.numel() * dst.element_size()} bytes, src {nbytes}")
    if nbytes == 0:
        return
    _check(lib.qsa_stream_copy(_dev(dst, "dst", 0, (dst.dtype,)), _dev(src, "src", 0, (src.dtype,)),
                               nbytes, _stream(stream)))


def qsa_index_ids_fill(ids, numRows, numBlocks, stream=None):
    """ids int32 [numRows, numBlocks]: ids[r][c] = c."""
    if numRows == 0 or numBlocks == 0:
        return
    _check(lib.qsa_index_ids_fill(_dev(ids, "ids", numRows * numBlocks, _I32), numRows,
                                  numBlocks, _stream(stream)))


def qsa_index_expand(outIdx, sortedIds, contextLengths, batchSize, seqLen, numBlocks, rowStart,
                     numRows, stream=None):
    """K4: rows [rowStart, rowStart+numRows) of outIdx int32 [B*S, 2051] from sortedIds int32
    [numRows, numBlocks]."""
    if numRows == 0:
        return
    _check(lib.qsa_index_expand(
        _dev(outIdx, "outIdx", batchSize * seqLen * INDEX_WIDTH, _I32),
        _dev(sortedIds, "sortedIds", numRows * numBlocks, _I32) if numBlocks else None,
        _dev(contextLengths, "contextLengths", batchSize, _I32), batchSize, seqLen, numBlocks,
        rowStart, numRows, _stream(stream)))


def qsa_index_topk_expand(outIdx, logits, contextLengths, batchSize, seqLen, numBlocks,
                          rowStart, numRows, stream=None):
    """Prefill top-512 selection + K4: rows [rowStart, rowStart+numRows) of outIdx int32
    [B*S, 2051] from logits FP32 [numRows, numBlocks]."""
    if numRows == 0:
        return
    _check(lib.qsa_index_topk_expand(
        _dev(outIdx, "outIdx", batchSize * seqLen * INDEX_WIDTH, _I32),
        _dev(logits, "logits", numRows * numBlocks, _F32) if numBlocks else None,
        _dev(contextLengths, "contextLengths", batchSize, _I32), batchSize, seqLen, numBlocks,
        rowStart, numRows, _stream(stream)))


def qsa_index_topk_expand_decode(outIdx, logits, contextLengths, maxBlocks, splitCounters=None,
                                 numKVHeads=0, batchSize=None, stream=None):
    """Decode top-512 selection + expand: outIdx int32 [B, 2051] from logits FP32
    [B, maxBlocks]; splitCounters int32 [B, numKVHeads] zeroed when given."""
    B = contextLengths.shape[0] if batchSize is None else batchSize
    if B == 0:
        return
    _check(lib.qsa_index_topk_expand_decode(
        _dev(outIdx, "outIdx", B * INDEX_WIDTH, _I32),
        _dev(logits, "logits", B * maxBlocks, _F32) if maxBlocks > TOPK else None,
        _dev(contextLengths, "contextLengths", B, _I32),
        None if splitCounters is None else _dev(splitCounters, "splitCounters",
                                                B * numKVHeads, _I32),
        numKVHeads, B, maxBlocks, _stream(stream)))


def qsa_last_error():
    return lib.qsa_last_error().decode()


def qsa_abi_version():
    return lib.qsa_abi_version()
