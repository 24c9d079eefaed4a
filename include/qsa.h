/*
 * qsa.h — C ABI of the QSA indexer hot path for AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the "Qsa Indexer Kernels" page of the TensorRT-Edge-LLM C++ API
 * documentation.  Each entry point below names the section of that page that defines the
 * operation it performs.  Notation follows the page: T is the activation type (fp16 or bf16),
 * B = batchSize, S = seqLen, ctx[b] = contextLengths[b], g = 4-token block index.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Memory.  Every tensor pointer is DEVICE memory owned by the caller, except the two structs
 *    (qsa_pool_state_t, qsa_seq_ranges_t), which are HOST structs whose pointer members are
 *    device memory.  The library allocates nothing, keeps no per-call state and holds no
 *    pointer after a call returns.
 *  - Layout.  All tensors are dense, row-major, contiguous.  Tensors of T and FP32 tensors must
 *    be 16-byte aligned; int32 tensors 4-byte aligned.
 *  - Asynchrony.  A call validates its arguments on the host (it reads no device memory), then
 *    enqueues its kernel(s) on `stream` (a hipStream_t; NULL is the null stream of the current
 *    device) and returns.  It never synchronises, never allocates and is safe to capture in a
 *    HIP graph.  The current HIP device must be the one that owns the pointers.
 *  - Errors.  A non-zero return is one of the QSA_E_* codes; qsa_last_error() then returns a
 *    thread-local text describing it.  Validation failures are reported before any launch, so a
 *    call that returns QSA_E_INVALID / QSA_E_ALIGN / QSA_E_DTYPE has written nothing.
 *    A call with valid arguments and work to do then checks for a current HIP device and
 *    returns QSA_E_NO_DEVICE, having launched nothing, when there is none (no GPU visible or no
 *    usable driver).  QSA_E_LAUNCH means the HIP runtime refused the launch (for instance a
 *    device without gfx950 code objects).  These map the page's launchers, which throw on
 *    invalid arguments or launch failure ("Qsa Indexer Kernels", each launcher's Throws).
 *  - Empty work.  batchSize == 0, an empty block range, or seqLen == 0 for q-prep returns
 *    QSA_OK without launching anything.
 *  - Device values outside the contract never fault: context lengths are clamped or treated as
 *    in the rules below, blocks that would read rows or cosSin positions that are not there are
 *    invalid, and page-table entries that are -1 or out of range skip the pool write.
 */
#ifndef QSA_H
#define QSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QSA_ABI_VERSION 1

/* Activation type T ("Qsa Indexer Kernels": template parameter T, half or __nv_bfloat16). */
typedef enum { QSA_F16 = 0, QSA_BF16 = 1 } qsa_dtype;

/* Return codes. */
enum {
  QSA_OK = 0,
  QSA_E_INVALID = -1, /* a null required pointer, a negative size, an inconsistent range    */
  QSA_E_ALIGN = -2,   /* a pointer or pool geometry that breaks the alignment rules above   */
  QSA_E_DTYPE = -3,   /* dt is not QSA_F16 or QSA_BF16                                        */
  QSA_E_LAUNCH = -4,  /* the HIP runtime rejected a kernel launch                             */
  QSA_E_NO_DEVICE = -5 /* no usable current HIP device (no GPU or no driver); nothing launched */
};

/* Fixed geometry of the method ("Qsa Indexer Kernels": launchQsaIndexQPrep and
 * launchQsaIndexKCompress parameter lists, QsaIndexerPoolState). */
#define QSA_INDEX_HEADS 4      /* index-Q heads per token row                           */
#define QSA_HEAD_DIM 128       /* dims per index-Q head, per raw index-K, per kbar row    */
#define QSA_ROW_WIDTH 640      /* indexQk row: 4 q-heads x 128, then raw k x 128          */
#define QSA_ROTARY_DIMS 64     /* neox rope on dims [0, 64); cosSin row = 32 cos, 32 sin   */
#define QSA_COMPRESS_RATIO 4   /* tokens per compressed block                             */
#define QSA_PAGE_TOKENS 128    /* tokens per pool page                                    */
#define QSA_UNUSED_PAGE_ENTRY (-1)
#define QSA_TOPK 512           /* blocks a query selects at most                          */
#define QSA_INDEX_WIDTH 2051   /* token indices per query row: 4 * QSA_TOPK + 3 tail slots  */

/*
 * Where the indexer state lives ("Qsa Indexer Kernels": struct QsaIndexerPoolState).
 *
 * The pool is T [2*numPages, 128, numKVHeads, poolHeadDim]; element (page, row, head, col) is
 * at element offset ((page*128 + row)*numKVHeads + head)*poolHeadDim + col, computed in 64 bits.
 * Only head 0, columns [headSize, headSize + 128) are ever written:
 *   - K-tail of token t of sequence b: page pageTable[b][0][t >> 7], row t & 127;
 *   - V-tail (kbar) of block g of sequence b: page pageTable[b][1][(4g) >> 7], row (4g) & 127
 *     (the V ids already include the +numPages offset; the library does not add it).
 * pageTable is int32 [B, 2, maxPagesPerSeq] on the device.  A slot outside
 * [0, maxPagesPerSeq), an entry equal to QSA_UNUSED_PAGE_ENTRY, or an entry outside
 * [0, 2*numPages) is "nothing persistable here": the write is skipped, nothing else changes.
 * The pool element type must be dt of the call.
 * Host-side checks: poolPtr 16-byte aligned and non-null, pageTable non-null, numPages > 0,
 * maxPagesPerSeq > 0, numKVHeads >= 1, 0 <= headSize, headSize + 128 <= poolHeadDim,
 * headSize % 8 == 0 and (numKVHeads*poolHeadDim) % 8 == 0 (QSA_E_ALIGN otherwise).
 */
typedef struct {
  void* poolPtr;
  const int32_t* pageTable;
  int32_t maxPagesPerSeq;
  int32_t numPages;   /* K-plane page count                      */
  int32_t numKVHeads; /* 2 in the documented model               */
  int32_t poolHeadDim;/* 384 in the documented model             */
  int32_t headSize;   /* 256 in the documented model = tail column offset */
} qsa_pool_state_t;

/*
 * Per-sequence block sub-range (an extension: the page defines one scalar triplet
 * (blockBegin, blockEnd, pastLen) per call in launchQsaIndexKCompress; a batch of decoding
 * sequences needs one triplet per sequence).  Three device int32 [B] arrays; entry b replaces
 * the scalar triplet for sequence b, and the block validity rule applies to it verbatim.
 * maxBlockSpan is a host bound on blockEnds[b] - blockBegins[b]; it sizes the grid, and
 * blocks g >= blockBegins[b] + maxBlockSpan are not processed.  Blocks g outside
 * [0, numBlocks) are skipped (nothing written).
 */
typedef struct {
  const int32_t* pastLens;
  const int32_t* blockBegins;
  const int32_t* blockEnds;
  int32_t maxBlockSpan;
} qsa_seq_ranges_t;

/*
 * K1a — index-Q norm and rope ("Qsa Indexer Kernels": launchQsaIndexQPrep).
 *
 * qNormed  [out] T [B, S, 4, 128].
 * indexQk  [in]  T [B, S, 640]; columns [128h, 128h+128) are q-head h.
 * cosSin   [in]  FP32 [maxPositions, 64]: cos in [0, 32), sin in [32, 64); row t is used for
 *                token t.  maxPositions >= S (QSA_E_INVALID otherwise).
 * contextLengths [in] device int32 [B]; valid length, clamped to [0, S] on the device.
 * wQ       [in]  T [128], raw checkpoint gamma (the kernel applies 1 + wQ).
 * rmsEps   finite and >= 0.
 * For t < ctx[b] and each head h, in FP32: meanSq = sum_d x_d^2 / 128;
 * y_d = x_d * rsqrt(meanSq + rmsEps) * (1 + wQ_d); neox rope on pairs (i, i+32), i < 32,
 * o_i = y_i cos_i - y_{i+32} sin_i, o_{i+32} = y_{i+32} cos_i + y_i sin_i; o_d = y_d for
 * d >= 64; one round-to-nearest-even cast to T.  Rows t >= ctx[b] are written as +0 and their
 * indexQk row is never read.
 */
int qsa_index_q_prep(void* qNormed, const void* indexQk, const float* cosSin, int32_t maxPositions,
                     const int32_t* contextLengths, const void* wQ, float rmsEps, int32_t batchSize,
                     int32_t seqLen, qsa_dtype dt, void* stream);

/*
 * K1b — index-K block compression ("Qsa Indexer Kernels": launchQsaIndexKCompress, and with a
 * pool, launchQsaIndexKCompressPaged).
 *
 * kbar     [out] T [B, numBlocks, 128]; only rows g in [blockBegin, blockEnd) are written.
 * indexQk  [in]  T [B, S, 640]; the raw key of token 4g+j is row 4g+j-pastLen, cols [512, 640).
 * cosSin   [in]  FP32 [maxPositions, 64]; block g uses row 4g.  Scalar mode requires
 *                maxPositions >= 4*blockEnd - 3.
 * contextLengths [in] device int32 [B]: TOTAL length (past + new) of each sequence.
 * wK       [in]  T [128] raw gamma.
 * numBlocks      kbar row stride, ceilDiv(maxTotalLen, 4); 0 <= blockBegin <= blockEnd <= numBlocks,
 *                pastLen >= 0 (scalar mode).
 * ranges   NULL: the scalar triplet applies to every sequence.  Otherwise the per-sequence
 *                triplets of qsa_seq_ranges_t are used and the scalars are ignored.
 * pool     NULL: no pool write.  Otherwise every VALID block's kbar row is also written, bit
 *                for bit, to its V-tail (page guard as in qsa_pool_state_t).  Invalid blocks
 *                never touch the pool.  The dense kbar is identical with and without a pool.
 * Block g of sequence b is valid iff 4g+3 < ctx[b], 4g >= pastLen, 4g+3-pastLen < S and
 * 4g < maxPositions.  A valid block computes, per dim d, in FP32 and in this order,
 * mean_d = (((k0+k1)+k2)+k3) * 0.25, casts it to T (round to nearest even) and widens it back,
 * then applies the K1a norm with wK and the rope at position 4g, and casts to T.  An invalid
 * block writes 128 zeros (+0) and reads no indexQk row.
 */
int qsa_index_k_compress(void* kbar, const void* indexQk, const float* cosSin, int32_t maxPositions,
                         const int32_t* contextLengths, const void* wK, float rmsEps,
                         int32_t batchSize, int32_t seqLen, int32_t numBlocks, int32_t blockBegin,
                         int32_t blockEnd, int32_t pastLen, const qsa_seq_ranges_t* ranges,
                         const qsa_pool_state_t* pool, qsa_dtype dt, void* stream);

/*
 * Persist — raw-K tails and (optionally) kbar V-tails into the pool ("Qsa Indexer Kernels":
 * launchQsaRawKTailWritePrefill for the tails, launchQsaIndexKCompressPaged and
 * QsaIndexerPoolState for the V-tails).
 *
 * pool     [in/out] required.
 * indexQk  [in]  T [B, S, 640].
 * kbar     [in]  T [B, numBlocks, 128] from qsa_index_k_compress with the same triplet(s), or
 *                NULL when the V-tails were already written by qsa_index_k_compress(pool).
 * Tails: for each b, tokens t in [max(pastLen, ctx - ctx%4), ctx) with 0 <= t-pastLen < S
 *        (at most 3; none when ctx % 4 == 0) copy indexQk row t-pastLen, columns [512, 640),
 *        bit-unmodified to their K-tail.
 * V-tails: for each valid block g in the range (validity as in qsa_index_k_compress without
 *        the maxPositions clause), kbar[b, g, :] is copied bit for bit to its V-tail.
 * No other pool cell is touched.
 */
int qsa_index_persist(const qsa_pool_state_t* pool, const void* indexQk, const void* kbar,
                      const int32_t* contextLengths, int32_t batchSize, int32_t seqLen,
                      int32_t numBlocks, int32_t blockBegin, int32_t blockEnd, int32_t pastLen,
                      const qsa_seq_ranges_t* ranges, qsa_dtype dt, void* stream);

/*
 * Fused prefill — the three steps above in ONE kernel launch, with output identical bit for bit
 * to qsa_index_q_prep, then qsa_index_k_compress(0, ceilDiv(S, 4), 0, ranges = NULL, pool),
 * then (if pool != NULL) qsa_index_persist(kbar = NULL) ("Qsa Indexer Kernels": the prefill
 * sequence of launchQsaIndexQPrep, launchQsaIndexKCompressPaged, launchQsaRawKTailWritePrefill).
 * Each indexQk row and each cosSin row is read once.  numBlocks >= ceilDiv(S, 4);
 * maxPositions >= S; contextLengths are valid lengths in [0, S] (clamped as in K1a).
 */
int qsa_index_prefill(void* qNormed, void* kbar, const void* indexQk, const float* cosSin,
                      int32_t maxPositions, const int32_t* contextLengths, const void* wQ,
                      const void* wK, float rmsEps, const qsa_pool_state_t* pool,
                      int32_t batchSize, int32_t seqLen, int32_t numBlocks, qsa_dtype dt,
                      void* stream);

/*
 * Decode pre-pass ("Qsa Indexer Kernels": launchQsaIndexerPreDecode), with n new tokens per
 * sequence (the page's form has exactly one: pass newLens = NULL).
 *
 * qNormed  [out] T [B, S, 4, 128]: row j of sequence b is the K1a output of its new token j.
 * indexQk  [in]  T [B, S, 640]: rows 0 .. n-1 of each sequence are its new tokens.
 * cosSin   [in]  FP32 [maxPositions, 64]; must cover max(contextLengths).
 * contextLengths [in] device int32 [B]: TOTAL lengths including the new tokens.
 * newLens  [in]  device int32 [B] (n per sequence, capped at S and at the length) or NULL (1).
 * wQ, wK   [in]  T [128] raw gammas.   pool: required.   seqLen = S >= 1 rows per sequence.
 * With p = ctx - n (the past length), per sequence:
 *  1. K1a numerics of each new token at its position p + j; rows j >= n are +0.
 *     ctx <= 0 writes zeros and skips steps 2 and 3.
 *  2. Tokens whose block stays incomplete, [max(p, ctx - ctx%4), ctx), copy their raw key
 *     bit-unmodified to their K-tail.
 *  3. Each block the new tokens complete, g in [floor(p/4), floor(ctx/4)): keys of tokens below
 *     p are read from their pool K-tails, keys of new tokens from indexQk; K1b numerics at 4g;
 *     the kbar row is written to the V-tail of token 4g (no dense kbar).  A block whose earlier
 *     keys are not in the pool (page guard fails) is skipped.
 * Positions at or past maxPositions produce +0 q rows and skipped blocks.  Because raw keys are
 * persisted bit-unmodified, decode-time kbar rows equal those of a prefill over the history.
 * One 256-thread workgroup per sequence; a batch larger than one launch holds is rejected
 * (QSA_E_INVALID).
 */
int qsa_index_pre_decode(void* qNormed, const void* indexQk, const float* cosSin,
                         int32_t maxPositions, const int32_t* contextLengths,
                         const int32_t* newLens, const void* wQ, const void* wK, float rmsEps,
                         const qsa_pool_state_t* pool, int32_t batchSize, int32_t seqLen,
                         qsa_dtype dt, void* stream);

/*
 * Block-relevance scores, prefill ("Qsa Indexer Kernels": launchQsaIndexScores).
 *
 * logits   [out] FP32 [numRows, numBlocks]: row i is global row r = rowStart + i = b*S + t.
 * qNormed  [in]  T [B, S, 4, 128] (qsa_index_q_prep);  kbar [in] T [B, numBlocks, 128].
 * contextLengths [in] device int32 [B].   0 <= rowStart, rowStart + numRows <= B*S.
 * logits[i][g] = (1/sqrtf(128)) * sum_{h<4, ascending} relu(q[r][h] . kbar[b][g]), FP32 dots,
 * ReLU per head, the scale after the sum; g >= (t+1)/4 (not a complete block up to t) gives
 * -FLT_MAX; a padded row (t >= ctx[b], or ctx[b] <= 0) is -FLT_MAX throughout and its q row is
 * not read.  The dot products run on MFMA; their summation order is the hardware's.
 * numBlocks <= 2^26.  One launch of (128-token tiles of the rows) * ceil(numBlocks/4096)
 * workgroups of 512 threads; a call needing more than 2^23 - 1 of them is rejected
 * (QSA_E_INVALID).
 */
int qsa_index_scores(float* logits, const void* qNormed, const void* kbar,
                     const int32_t* contextLengths, int32_t batchSize, int32_t seqLen,
                     int32_t numBlocks, int32_t rowStart, int32_t numRows, qsa_dtype dt,
                     void* stream);

/*
 * Block-relevance scores, decode ("Qsa Indexer Kernels": launchQsaIndexScoresDecode).
 *
 * logits   [out] FP32 [B, maxBlocks]; only [0, min(ctx/4, maxBlocks)) of each row is written.
 * qNormed  [in]  T [B, 1, 4, 128] (one query token per sequence).
 * contextLengths [in] device int32 [B]: TOTAL lengths.   pool: required (kbar is read from the
 * V-tail of token 4g).  Same score as qsa_index_scores; a block whose V page entry is unused
 * or out of range scores -FLT_MAX.  B * ceil(maxBlocks / 128) workgroups of 64 threads; a
 * batch larger than one launch holds (more than 2^26 - 1 of them) is rejected (QSA_E_INVALID).
 */
int qsa_index_scores_decode(float* logits, const void* qNormed, const int32_t* contextLengths,
                            const qsa_pool_state_t* pool, int32_t batchSize, int32_t maxBlocks,
                            qsa_dtype dt, void* stream);

/*
 * Block selection and expansion to token indices ("Qsa Indexer Kernels": launchQsaIndexIdsFill,
 * launchQsaIndexExpand, launchQsaTopKExpandDecode).  All integer; results are exact.
 *
 * Keys: a logit's FP32 bits mapped monotonically to u = bits >= 0 ? bits | 0x80000000 : ~bits;
 * a row is ordered by descending u, equal u by ascending block id (the order of a stable
 * descending sort over ascending ids).  For a query row with t = its position and
 * nVis = (t+1)/4 complete blocks, kSel = min(512, nVis): out[4i + j] = id_i * 4 + j for i < kSel,
 * j < 4, then the tail tokens out[4*kSel + j] = 4*nVis + j for j < (t+1) % 4, then -1 up to
 * QSA_INDEX_WIDTH.  A padded row (t >= ctx[b], or ctx[b] <= 0) is -1 throughout.
 */

/* ids [out] device int32 [numRows, numBlocks]: ids[r][c] = c. */
int qsa_index_ids_fill(int32_t* ids, int32_t numRows, int32_t numBlocks, void* stream);

/*
 * K4 over global rows r = rowStart + i = b*S + t, i < numRows.
 * outIdx    [out] device int32 [B*S, QSA_INDEX_WIDTH]; only the chunk's rows are written.
 * sortedIds [in]  device int32 [numRows, numBlocks]: each row's block ids in selection order;
 *                 only the first kSel entries are read.  numBlocks >= min(512, seqLen/4).
 */
int qsa_index_expand(int32_t* outIdx, const int32_t* sortedIds, const int32_t* contextLengths,
                     int32_t batchSize, int32_t seqLen, int32_t numBlocks, int32_t rowStart,
                     int32_t numRows, void* stream);

/*
 * Prefill selection + K4 in one pass (the page's ids fill, per-row descending sort and expand,
 * without materialising the sorted rows).
 * logits [in] device FP32 [numRows, numBlocks] (the layout qsa_index_scores writes).
 * Row i selects the kSel largest keys among its complete blocks [0, min(nVis, numBlocks)) and
 * emits them in descending key order, equal keys by ascending id.  This is the page's full-row
 * sort whenever no logit past a row's complete blocks outranks a selected one, which holds for
 * logits from qsa_index_scores (complete blocks >= 0, the rest -FLT_MAX); entries past the
 * complete blocks are not read.
 */
int qsa_index_topk_expand(int32_t* outIdx, const float* logits, const int32_t* contextLengths,
                          int32_t batchSize, int32_t seqLen, int32_t numBlocks, int32_t rowStart,
                          int32_t numRows, void* stream);

/*
 * Decode selection + expand, one query per sequence (launchQsaTopKExpandDecode).
 * outIdx [out] device int32 [B, QSA_INDEX_WIDTH];  logits [in] device FP32 [B, maxBlocks]
 * (qsa_index_scores_decode);  splitCounters [out, nullable] device int32 [B, numKVHeads]: the
 * split-merge counters of the decode attention that follows, zeroed here when non-NULL.
 * nVis = ctx/4, which maxBlocks must cover (a larger ctx is capped: nVis = maxBlocks, the tail
 * tokens then start at 4*maxBlocks); tail = ctx % 4.  nVis <= 512 takes every block 0..nVis-1
 * and reads no logits.  Otherwise the kSel = 512 largest keys of [0, nVis), equal keys at the
 * threshold in ascending id, emitted in ascending block id.  ctx <= 0 gives an all -1 row.
 * One 512-thread workgroup per sequence; for maxBlocks in (32768, 262144] each row is cut
 * into c = ceil(maxBlocks / chunk) <= 8 chunks (chunk a power of two from 8192 to 32768),
 * selected by one workgroup each, and a second launch merges them: the chunk pass stages
 * 16-bit candidate ids in the sequence's own outIdx row, which the merge then overwrites, so
 * outIdx must not overlap logits (QSA_E_INVALID).  batchSize * c <= 2^23 - 1 (c = 1 for
 * shorter rows), else QSA_E_INVALID.  Rows above 262144 blocks take a kernel that re-reads
 * the row.
 */
int qsa_index_topk_expand_decode(int32_t* outIdx, const float* logits,
                                 const int32_t* contextLengths, int32_t* splitCounters,
                                 int32_t numKVHeads, int32_t batchSize, int32_t maxBlocks,
                                 void* stream);

/*
 * Measurement helper, not a step of the indexer: a plain device-to-device copy of `bytes`
 * (>= 0, a multiple of 16; dst and src 16-byte aligned device buffers that do not overlap),
 * one 16-byte chunk per thread with non-temporal loads and stores.  The benchmark times it on
 * the fused launch's traffic to state the rate at which this machine streams bytes at all.
 * Errors as for every entry point: QSA_E_INVALID / QSA_E_ALIGN before any launch.
 */
int qsa_stream_copy(void* dst, const void* src, int64_t bytes, void* stream);

/*
 * Debug forms: the same kernels with their FP32 intermediates written out.  Arguments as the
 * entry point of the same name, plus (all device FP32 unless noted, all required):
 *   qsa_debug_q_prep:     meanSq [B,S,4], invRms [B,S,4], preCast [B,S,4,128];
 *   qsa_debug_k_compress: mT (T) [B,numBlocks,128] = the cast block mean, meanSq [B,numBlocks],
 *                         invRms [B,numBlocks], preCast [B,numBlocks,128].
 * invRms is rsqrt(meanSq + rmsEps); preCast is the roped value before the final cast to T.
 * Padding rows and invalid blocks write zeros to every debug output.
 */
int qsa_debug_q_prep(void* qNormed, const void* indexQk, const float* cosSin, int32_t maxPositions,
                     const int32_t* contextLengths, const void* wQ, float rmsEps, int32_t batchSize,
                     int32_t seqLen, qsa_dtype dt, void* stream, float* meanSq, float* invRms,
                     float* preCast);
int qsa_debug_k_compress(void* kbar, const void* indexQk, const float* cosSin, int32_t maxPositions,
                         const int32_t* contextLengths, const void* wK, float rmsEps,
                         int32_t batchSize, int32_t seqLen, int32_t numBlocks, int32_t blockBegin,
                         int32_t blockEnd, int32_t pastLen, const qsa_seq_ranges_t* ranges,
                         const qsa_pool_state_t* pool, qsa_dtype dt, void* stream, void* mT,
                         float* meanSq, float* invRms, float* preCast);

/* Thread-local text for the last non-QSA_OK return on this thread ("" if none). */
const char* qsa_last_error(void);

/* QSA_ABI_VERSION of the built library. */
int qsa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QSA_H */
