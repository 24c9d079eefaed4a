// qsa_api.cpp — the C ABI of include/qsa.h: host-side argument validation, error reporting,
// and the hand-off to the kernel launchers.  No device memory is read here and nothing is
// synchronised or allocated; a non-OK return has launched nothing (except QSA_E_LAUNCH).

#include "qsa.h"

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "qsa_internal.h"

#define QSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() { return QSA_OK; }

#define TRY(expr)                 \
  do {                            \
    const int rc_ = (expr);       \
    if (rc_ != QSA_OK) return rc_; \
  } while (0)

int need(const void* p, const char* name, std::uintptr_t align) {
  if (p == nullptr) return fail(QSA_E_INVALID, "%s is NULL", name);
  if (reinterpret_cast<std::uintptr_t>(p) % align != 0)
    return fail(QSA_E_ALIGN, "%s (%p) is not %u-byte aligned", name, p, (unsigned)align);
  return QSA_OK;
}

int check_dt(qsa_dtype dt, qsa::Dt* out) {
  if (dt == QSA_F16) *out = qsa::Dt::F16;
  else if (dt == QSA_BF16) *out = qsa::Dt::BF16;
  else return fail(QSA_E_DTYPE, "dt = %d is neither QSA_F16 (0) nor QSA_BF16 (1)", (int)dt);
  return QSA_OK;
}

int check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.0f)
    return fail(QSA_E_INVALID, "rmsEps = %g must be finite and >= 0", (double)eps);
  return QSA_OK;
}

// A launch's x extent counts work-items in 32 bits, so it holds at most UINT32_MAX threads;
// `threads` is the workgroup size of the kernel (256 unless stated at the call).
int check_grid(int64_t workgroups, int64_t threads = 256) {
  if (workgroups > (int64_t)UINT32_MAX / threads)
    return fail(QSA_E_INVALID, "problem needs %lld workgroups, more than one launch can hold",
                (long long)workgroups);
  return QSA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_pool(const qsa_pool_state_t* p, qsa::PoolArgs* out) {
  if (p == nullptr) return fail(QSA_E_INVALID, "pool state is NULL");
  TRY(need(p->poolPtr, "pool->poolPtr", 16));
  TRY(need(p->pageTable, "pool->pageTable", 4));
  if (p->maxPagesPerSeq <= 0 || p->numPages <= 0 || p->numPages > INT32_MAX / 2)
    return fail(QSA_E_INVALID, "pool: maxPagesPerSeq = %d, numPages = %d out of range",
                p->maxPagesPerSeq, p->numPages);
  if (p->numKVHeads < 1 || p->headSize < 0 || p->poolHeadDim < 128 ||
      (int64_t)p->headSize + 128 > p->poolHeadDim)
    return fail(QSA_E_INVALID,
                "pool: numKVHeads = %d, poolHeadDim = %d, headSize = %d (need numKVHeads >= 1, "
                "0 <= headSize, headSize + 128 <= poolHeadDim)",
                p->numKVHeads, p->poolHeadDim, p->headSize);
  const int64_t rowElems = (int64_t)p->numKVHeads * p->poolHeadDim;
  if (p->headSize % 8 != 0 || rowElems % 8 != 0)
    return fail(QSA_E_ALIGN, "pool: headSize = %d and numKVHeads*poolHeadDim = %lld must be "
                "multiples of 8 elements", p->headSize, (long long)rowElems);
  out->base = p->poolPtr;
  out->pageTable = p->pageTable;
  out->maxPagesPerSeq = p->maxPagesPerSeq;
  out->numIds = 2 * p->numPages;
  out->rowElems = rowElems;
  out->headSize = p->headSize;
  return QSA_OK;
}

// Block triplet: scalars (ranges == NULL) or per-sequence arrays.  Sets out->span.
int check_range(int32_t numBlocks, int32_t blockBegin, int32_t blockEnd, int32_t pastLen,
                const qsa_seq_ranges_t* ranges, qsa::Ranges* out) {
  *out = qsa::Ranges{};
  if (numBlocks < 0) return fail(QSA_E_INVALID, "numBlocks = %d < 0", numBlocks);
  if (ranges == nullptr) {
    if (!(0 <= blockBegin && blockBegin <= blockEnd && blockEnd <= numBlocks))
      return fail(QSA_E_INVALID, "need 0 <= blockBegin (%d) <= blockEnd (%d) <= numBlocks (%d)",
                  blockBegin, blockEnd, numBlocks);
    if (pastLen < 0) return fail(QSA_E_INVALID, "pastLen = %d < 0", pastLen);
    out->blockBegin = blockBegin;
    out->blockEnd = blockEnd;
    out->pastLen = pastLen;
    out->span = blockEnd - blockBegin;
    return QSA_OK;
  }
  TRY(need(ranges->pastLens, "ranges->pastLens", 4));
  TRY(need(ranges->blockBegins, "ranges->blockBegins", 4));
  TRY(need(ranges->blockEnds, "ranges->blockEnds", 4));
  if (ranges->maxBlockSpan < 0)
    return fail(QSA_E_INVALID, "ranges->maxBlockSpan = %d < 0", ranges->maxBlockSpan);
  out->pastLens = ranges->pastLens;
  out->blockBegins = ranges->blockBegins;
  out->blockEnds = ranges->blockEnds;
  out->span = ranges->maxBlockSpan;
  return QSA_OK;
}

// A call that is about to launch needs a current HIP device: with no device (or no usable
// driver) hipGetDevice reports an error, and the call returns QSA_E_NO_DEVICE having launched
// nothing.  Runs after validation, so invalid arguments are reported as such on any machine.
int device_ready() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(QSA_E_NO_DEVICE, "no usable HIP device: %s", hipGetErrorString(e));
  return QSA_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(QSA_E_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

int q_prep_impl(void* qNormed, const void* indexQk, const float* cosSin, int32_t maxPositions,
                const int32_t* ctx, const void* wQ, float eps, int32_t B, int32_t S,
                qsa_dtype dt, void* stream, bool debug, float* meanSq, float* inv,
                float* preCast) {
  qsa::Dt t;
  TRY(check_dt(dt, &t));
  if (B < 0 || S < 0) return fail(QSA_E_INVALID, "batchSize = %d, seqLen = %d", B, S);
  if (B == 0 || S == 0) return ok();
  TRY(need(qNormed, "qNormed", 16));
  TRY(need(indexQk, "indexQk", 16));
  TRY(need(cosSin, "cosSin", 16));
  TRY(need(ctx, "contextLengths", 4));
  TRY(need(wQ, "wQ", 16));
  if (maxPositions < S)
    return fail(QSA_E_INVALID, "maxPositions = %d < seqLen = %d", maxPositions, S);
  TRY(check_eps(eps));
  if (debug) {
    TRY(need(meanSq, "meanSq", 4));
    TRY(need(inv, "invRms", 4));
    TRY(need(preCast, "preCast", 16));
  }
  TRY(check_grid((int64_t)B * ceil_div(ceil_div(S, 4), 4)));
  const qsa::QPrepArgs a{qNormed, indexQk, cosSin, ctx, wQ, eps, B, S, meanSq, inv, preCast};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_q_prep(a, t, debug, static_cast<hipStream_t>(stream)),
                  "qsa_index_q_prep");
}

int k_compress_impl(void* kbar, const void* indexQk, const float* cosSin, int32_t maxPositions,
                    const int32_t* ctx, const void* wK, float eps, int32_t B, int32_t S,
                    int32_t numBlocks, int32_t blockBegin, int32_t blockEnd, int32_t pastLen,
                    const qsa_seq_ranges_t* ranges, const qsa_pool_state_t* pool, qsa_dtype dt,
                    void* stream, bool debug, void* mT, float* meanSq, float* inv,
                    float* preCast) {
  qsa::Dt t;
  TRY(check_dt(dt, &t));
  if (B < 0 || S < 0) return fail(QSA_E_INVALID, "batchSize = %d, seqLen = %d", B, S);
  qsa::Ranges r;
  TRY(check_range(numBlocks, blockBegin, blockEnd, pastLen, ranges, &r));
  if (ranges == nullptr && blockEnd > blockBegin && (int64_t)maxPositions < 4LL * blockEnd - 3)
    return fail(QSA_E_INVALID, "maxPositions = %d < 4*blockEnd - 3 = %lld", maxPositions,
                4LL * blockEnd - 3);
  if (maxPositions < 0) return fail(QSA_E_INVALID, "maxPositions = %d < 0", maxPositions);
  if (B == 0 || r.span == 0) return ok();
  TRY(need(kbar, "kbar", 16));
  TRY(need(indexQk, "indexQk", 16));
  TRY(need(cosSin, "cosSin", 16));
  TRY(need(ctx, "contextLengths", 4));
  TRY(need(wK, "wK", 16));
  TRY(check_eps(eps));
  qsa::PoolArgs p{};
  if (pool != nullptr) TRY(check_pool(pool, &p));
  if (debug) {
    TRY(need(mT, "mT", 16));
    TRY(need(meanSq, "meanSq", 4));
    TRY(need(inv, "invRms", 4));
    TRY(need(preCast, "preCast", 16));
  }
  TRY(check_grid((int64_t)B * ceil_div(r.span, 16)));
  const qsa::KCompressArgs a{kbar, indexQk, cosSin, maxPositions, ctx, wK, eps, B, S, numBlocks,
                             r, p, mT, meanSq, inv, preCast};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_k_compress(a, t, debug, static_cast<hipStream_t>(stream)),
                  "qsa_index_k_compress");
}

}  // namespace

QSA_EXPORT int qsa_index_q_prep(void* qNormed, const void* indexQk, const float* cosSin,
                                int32_t maxPositions, const int32_t* contextLengths,
                                const void* wQ, float rmsEps, int32_t batchSize, int32_t seqLen,
                                qsa_dtype dt, void* stream) {
  return q_prep_impl(qNormed, indexQk, cosSin, maxPositions, contextLengths, wQ, rmsEps,
                     batchSize, seqLen, dt, stream, false, nullptr, nullptr, nullptr);
}

QSA_EXPORT int qsa_debug_q_prep(void* qNormed, const void* indexQk, const float* cosSin,
                                int32_t maxPositions, const int32_t* contextLengths,
                                const void* wQ, float rmsEps, int32_t batchSize, int32_t seqLen,
                                qsa_dtype dt, void* stream, float* meanSq, float* invRms,
                                float* preCast) {
  return q_prep_impl(qNormed, indexQk, cosSin, maxPositions, contextLengths, wQ, rmsEps,
                     batchSize, seqLen, dt, stream, true, meanSq, invRms, preCast);
}

QSA_EXPORT int qsa_index_k_compress(void* kbar, const void* indexQk, const float* cosSin,
                                    int32_t maxPositions, const int32_t* contextLengths,
                                    const void* wK, float rmsEps, int32_t batchSize,
                                    int32_t seqLen, int32_t numBlocks, int32_t blockBegin,
                                    int32_t blockEnd, int32_t pastLen,
                                    const qsa_seq_ranges_t* ranges,
                                    const qsa_pool_state_t* pool, qsa_dtype dt, void* stream) {
  return k_compress_impl(kbar, indexQk, cosSin, maxPositions, contextLengths, wK, rmsEps,
                         batchSize, seqLen, numBlocks, blockBegin, blockEnd, pastLen, ranges,
                         pool, dt, stream, false, nullptr, nullptr, nullptr, nullptr);
}

QSA_EXPORT int qsa_debug_k_compress(void* kbar, const void* indexQk, const float* cosSin,
                                    int32_t maxPositions, const int32_t* contextLengths,
                                    const void* wK, float rmsEps, int32_t batchSize,
                                    int32_t seqLen, int32_t numBlocks, int32_t blockBegin,
                                    int32_t blockEnd, int32_t pastLen,
                                    const qsa_seq_ranges_t* ranges,
                                    const qsa_pool_state_t* pool, qsa_dtype dt, void* stream,
                                    void* mT, float* meanSq, float* invRms, float* preCast) {
  return k_compress_impl(kbar, indexQk, cosSin, maxPositions, contextLengths, wK, rmsEps,
                         batchSize, seqLen, numBlocks, blockBegin, blockEnd, pastLen, ranges,
                         pool, dt, stream, true, mT, meanSq, invRms, preCast);
}

QSA_EXPORT int qsa_index_persist(const qsa_pool_state_t* pool, const void* indexQk,
                                 const void* kbar, const int32_t* contextLengths,
                                 int32_t batchSize, int32_t seqLen, int32_t numBlocks,
                                 int32_t blockBegin, int32_t blockEnd, int32_t pastLen,
                                 const qsa_seq_ranges_t* ranges, qsa_dtype dt, void* stream) {
  qsa::Dt t;
  TRY(check_dt(dt, &t));
  if (batchSize < 0 || seqLen < 0)
    return fail(QSA_E_INVALID, "batchSize = %d, seqLen = %d", batchSize, seqLen);
  qsa::Ranges r;
  TRY(check_range(numBlocks, blockBegin, blockEnd, pastLen, ranges, &r));
  if (batchSize == 0 || seqLen == 0) return ok();
  qsa::PoolArgs p{};
  TRY(check_pool(pool, &p));
  TRY(need(indexQk, "indexQk", 16));
  if (kbar != nullptr) TRY(need(kbar, "kbar", 16));
  TRY(need(contextLengths, "contextLengths", 4));
  const int64_t items = 3 + (kbar != nullptr ? (int64_t)r.span : 0);
  TRY(check_grid((int64_t)batchSize * ceil_div(items, 16)));
  const qsa::PersistArgs a{p, indexQk, kbar, contextLengths, batchSize, seqLen, numBlocks, r};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_persist(a, static_cast<hipStream_t>(stream)), "qsa_index_persist");
}

QSA_EXPORT int qsa_index_prefill(void* qNormed, void* kbar, const void* indexQk,
                                 const float* cosSin, int32_t maxPositions,
                                 const int32_t* contextLengths, const void* wQ, const void* wK,
                                 float rmsEps, const qsa_pool_state_t* pool, int32_t batchSize,
                                 int32_t seqLen, int32_t numBlocks, qsa_dtype dt, void* stream) {
  qsa::Dt t;
  TRY(check_dt(dt, &t));
  if (batchSize < 0 || seqLen < 0 || numBlocks < 0)
    return fail(QSA_E_INVALID, "batchSize = %d, seqLen = %d, numBlocks = %d", batchSize,
                seqLen, numBlocks);
  if (numBlocks < ceil_div(seqLen, 4))
    return fail(QSA_E_INVALID, "numBlocks = %d < ceilDiv(seqLen, 4) = %lld", numBlocks,
                (long long)ceil_div(seqLen, 4));
  if (batchSize == 0 || seqLen == 0) return ok();
  TRY(need(qNormed, "qNormed", 16));
  TRY(need(kbar, "kbar", 16));
  TRY(need(indexQk, "indexQk", 16));
  TRY(need(cosSin, "cosSin", 16));
  TRY(need(contextLengths, "contextLengths", 4));
  TRY(need(wQ, "wQ", 16));
  TRY(need(wK, "wK", 16));
  if (maxPositions < seqLen)
    return fail(QSA_E_INVALID, "maxPositions = %d < seqLen = %d", maxPositions, seqLen);
  TRY(check_eps(rmsEps));
  qsa::PoolArgs p{};
  if (pool != nullptr) TRY(check_pool(pool, &p));
  TRY(check_grid((int64_t)batchSize * ceil_div(ceil_div(seqLen, 4), 4)));
  const qsa::PrefillArgs a{qNormed, kbar, indexQk, cosSin, contextLengths, wQ, wK, rmsEps,
                           batchSize, seqLen, numBlocks, p};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_prefill(a, t, static_cast<hipStream_t>(stream)),
                  "qsa_index_prefill");
}

QSA_EXPORT int qsa_index_pre_decode(void* qNormed, const void* indexQk, const float* cosSin,
                                    int32_t maxPositions, const int32_t* contextLengths,
                                    const int32_t* newLens, const void* wQ, const void* wK,
                                    float rmsEps, const qsa_pool_state_t* pool,
                                    int32_t batchSize, int32_t seqLen, qsa_dtype dt,
                                    void* stream) {
  qsa::Dt t;
  TRY(check_dt(dt, &t));
  if (batchSize < 0 || seqLen < 1)
    return fail(QSA_E_INVALID, "batchSize = %d, seqLen = %d (need seqLen >= 1)", batchSize,
                seqLen);
  if (maxPositions < 0) return fail(QSA_E_INVALID, "maxPositions = %d < 0", maxPositions);
  if (batchSize == 0) return ok();
  TRY(need(qNormed, "qNormed", 16));
  TRY(need(indexQk, "indexQk", 16));
  TRY(need(cosSin, "cosSin", 16));
  TRY(need(contextLengths, "contextLengths", 4));
  if (newLens != nullptr) TRY(need(newLens, "newLens", 4));
  TRY(need(wQ, "wQ", 16));
  TRY(need(wK, "wK", 16));
  TRY(check_eps(rmsEps));
  qsa::PoolArgs p{};
  TRY(check_pool(pool, &p));
  TRY(check_grid(batchSize));  // one workgroup per sequence
  const qsa::PreDecodeArgs a{qNormed, indexQk, cosSin, maxPositions, contextLengths, newLens,
                             wQ, wK, rmsEps, batchSize, seqLen, p};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_pre_decode(a, t, static_cast<hipStream_t>(stream)),
                  "qsa_index_pre_decode");
}

QSA_EXPORT int qsa_index_scores(float* logits, const void* qNormed, const void* kbar,
                                const int32_t* contextLengths, int32_t batchSize, int32_t seqLen,
                                int32_t numBlocks, int32_t rowStart, int32_t numRows, qsa_dtype dt,
                                void* stream) {
  qsa::Dt t;
  TRY(check_dt(dt, &t));
  if (batchSize < 0 || seqLen < 0 || numBlocks < 0 || rowStart < 0 || numRows < 0)
    return fail(QSA_E_INVALID, "batchSize = %d, seqLen = %d, numBlocks = %d, rowStart = %d, "
                "numRows = %d must be >= 0", batchSize, seqLen, numBlocks, rowStart, numRows);
  const int64_t rows = (int64_t)batchSize * seqLen;
  if ((int64_t)rowStart + numRows > rows)
    return fail(QSA_E_INVALID, "rowStart + numRows = %lld > batchSize * seqLen = %lld",
                (long long)rowStart + numRows, (long long)rows);
  if (numRows == 0 || numBlocks == 0) return ok();
  if (numBlocks > (1 << 26))  // the kernel addresses 16 logits rows with 32-bit byte offsets
    return fail(QSA_E_INVALID, "numBlocks = %d exceeds the supported %d", numBlocks, 1 << 26);
  TRY(need(logits, "logits", 4));
  TRY(need(qNormed, "qNormed", 16));
  TRY(need(kbar, "kbar", 16));
  TRY(need(contextLengths, "contextLengths", 4));
  qsa::ScoresArgs a{};
  a.logits = logits;
  a.qNormed = qNormed;
  a.kbar = kbar;
  a.ctx = contextLengths;
  a.B = batchSize;
  a.S = seqLen;
  a.numBlocks = numBlocks;
  a.rowStart = rowStart;
  a.numRows = numRows;
  qsa::ScoresArgs probe = a;  // the launcher fills the tile fields the same way
  TRY(check_grid(qsa::scores_workgroups(probe), qsa::kScoresThreads));
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_scores(a, t, static_cast<hipStream_t>(stream)), "qsa_index_scores");
}

QSA_EXPORT int qsa_index_scores_decode(float* logits, const void* qNormed,
                                       const int32_t* contextLengths,
                                       const qsa_pool_state_t* pool, int32_t batchSize,
                                       int32_t maxBlocks, qsa_dtype dt, void* stream) {
  qsa::Dt t;
  TRY(check_dt(dt, &t));
  if (batchSize < 0 || maxBlocks < 0)
    return fail(QSA_E_INVALID, "batchSize = %d, maxBlocks = %d", batchSize, maxBlocks);
  if (batchSize == 0 || maxBlocks == 0) return ok();
  TRY(need(logits, "logits", 4));
  TRY(need(qNormed, "qNormed", 16));
  TRY(need(contextLengths, "contextLengths", 4));
  qsa::PoolArgs p{};
  TRY(check_pool(pool, &p));
  TRY(check_grid(qsa::scores_decode_workgroups(batchSize, maxBlocks), 64));
  const qsa::ScoresDecodeArgs a{logits, qNormed, contextLengths, p, batchSize, maxBlocks};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_scores_decode(a, t, static_cast<hipStream_t>(stream)),
                  "qsa_index_scores_decode");
}

namespace {

// Row chunk [rowStart, rowStart + numRows) of a [B*S, ...] problem.
int check_rows(int32_t B, int32_t S, int32_t numBlocks, int32_t rowStart, int32_t numRows) {
  if (B < 0 || S < 0 || numBlocks < 0 || rowStart < 0 || numRows < 0)
    return fail(QSA_E_INVALID, "batchSize = %d, seqLen = %d, numBlocks = %d, rowStart = %d, "
                "numRows = %d must be >= 0", B, S, numBlocks, rowStart, numRows);
  if ((int64_t)rowStart + numRows > (int64_t)B * S)
    return fail(QSA_E_INVALID, "rowStart + numRows = %lld > batchSize * seqLen = %lld",
                (long long)rowStart + numRows, (long long)B * S);
  return QSA_OK;
}

}  // namespace

QSA_EXPORT int qsa_index_ids_fill(int32_t* ids, int32_t numRows, int32_t numBlocks,
                                  void* stream) {
  if (numRows < 0 || numBlocks < 0)
    return fail(QSA_E_INVALID, "numRows = %d, numBlocks = %d must be >= 0", numRows, numBlocks);
  if (numRows == 0 || numBlocks == 0) return ok();
  TRY(need(ids, "ids", 4));
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_ids_fill(ids, (int64_t)numRows * numBlocks, numBlocks,
                                       static_cast<hipStream_t>(stream)),
                  "qsa_index_ids_fill");
}

QSA_EXPORT int qsa_index_expand(int32_t* outIdx, const int32_t* sortedIds,
                                const int32_t* contextLengths, int32_t batchSize, int32_t seqLen,
                                int32_t numBlocks, int32_t rowStart, int32_t numRows,
                                void* stream) {
  TRY(check_rows(batchSize, seqLen, numBlocks, rowStart, numRows));
  if (numRows == 0) return ok();
  const int32_t maxSel = seqLen / 4 < QSA_TOPK ? seqLen / 4 : QSA_TOPK;
  if (numBlocks < maxSel)
    return fail(QSA_E_INVALID, "numBlocks = %d < min(%d, seqLen/4) = %d: a row would need "
                "more sorted ids than it holds", numBlocks, QSA_TOPK, maxSel);
  TRY(need(outIdx, "outIdx", 4));
  if (maxSel > 0) TRY(need(sortedIds, "sortedIds", 4));
  TRY(need(contextLengths, "contextLengths", 4));
  TRY(check_grid(numRows));
  const qsa::ExpandArgs a{outIdx, sortedIds, contextLengths, seqLen, numBlocks, rowStart, numRows};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_expand(a, static_cast<hipStream_t>(stream)), "qsa_index_expand");
}

QSA_EXPORT int qsa_index_topk_expand(int32_t* outIdx, const float* logits,
                                     const int32_t* contextLengths, int32_t batchSize,
                                     int32_t seqLen, int32_t numBlocks, int32_t rowStart,
                                     int32_t numRows, void* stream) {
  TRY(check_rows(batchSize, seqLen, numBlocks, rowStart, numRows));
  if (numRows == 0) return ok();
  TRY(need(outIdx, "outIdx", 4));
  if (numBlocks > 0) TRY(need(logits, "logits", 4));
  TRY(need(contextLengths, "contextLengths", 4));
  TRY(check_grid(numRows));
  const qsa::TopkArgs a{outIdx, logits, contextLengths, seqLen, numBlocks, rowStart, numRows};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_topk_expand(a, static_cast<hipStream_t>(stream)),
                  "qsa_index_topk_expand");
}

QSA_EXPORT int qsa_index_topk_expand_decode(int32_t* outIdx, const float* logits,
                                            const int32_t* contextLengths,
                                            int32_t* splitCounters, int32_t numKVHeads,
                                            int32_t batchSize, int32_t maxBlocks, void* stream) {
  if (batchSize < 0 || maxBlocks < 0)
    return fail(QSA_E_INVALID, "batchSize = %d, maxBlocks = %d must be >= 0", batchSize,
                maxBlocks);
  if (splitCounters != nullptr && numKVHeads < 0)
    return fail(QSA_E_INVALID, "numKVHeads = %d must be >= 0", numKVHeads);
  if (batchSize == 0) return ok();
  TRY(need(outIdx, "outIdx", 4));
  if (splitCounters != nullptr) TRY(need(splitCounters, "splitCounters", 4));
  if (maxBlocks > QSA_TOPK) TRY(need(logits, "logits", 4));
  TRY(need(contextLengths, "contextLengths", 4));
  const int64_t wgs = qsa::topk_decode_workgroups(batchSize, maxBlocks);
  TRY(check_grid(wgs, 512));
  if (wgs > batchSize) {
    // rows cut into chunks stage candidates in outIdx while logits are still being read
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(outIdx), l0 = reinterpret_cast<uintptr_t>(logits);
    const uintptr_t o1 = o0 + (uintptr_t)batchSize * QSA_INDEX_WIDTH * 4;
    const uintptr_t l1 = l0 + (uintptr_t)batchSize * (uintptr_t)maxBlocks * 4;
    if (o0 < l1 && l0 < o1)
      return fail(QSA_E_INVALID, "outIdx overlaps logits (rows of %d blocks are selected in "
                  "chunks that stage candidates in outIdx)", maxBlocks);
  }
  const qsa::TopkDecodeArgs a{outIdx, logits, contextLengths, splitCounters,
                              splitCounters != nullptr ? numKVHeads : 0, batchSize, maxBlocks};
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_topk_expand_decode(a, static_cast<hipStream_t>(stream)),
                  "qsa_index_topk_expand_decode");
}

QSA_EXPORT int qsa_stream_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0)
    return fail(QSA_E_INVALID, "bytes = %lld must be >= 0 and a multiple of 16",
                (long long)bytes);
  if (bytes == 0) return ok();
  TRY(need(dst, "dst", 16));
  TRY(need(src, "src", 16));
  TRY(check_grid((bytes / 16 + 255) / 256));
  TRY(device_ready());
  (void)hipGetLastError();
  return launched(qsa::launch_stream_copy(dst, src, bytes, static_cast<hipStream_t>(stream)),
                  "qsa_stream_copy");
}

QSA_EXPORT const char* qsa_last_error(void) { return g_err; }

QSA_EXPORT int qsa_abi_version(void) { return QSA_ABI_VERSION; }
