/*
 * qsa_ref.c — CPU oracle of the QSA indexer hot path.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the reference the GPU library is checked against.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it; the product path never
 * does.  It shares no code, header or constant with the GPU library.
 *
 * It is the plain definition of what the "Qsa Indexer Kernels" page (TensorRT-Edge-LLM C++ API
 * documentation) says the kernels compute, written as slow straight-line C:
 *   - ref_q_prep        launchQsaIndexQPrep (K1a),
 *   - ref_k_compress    launchQsaIndexKCompress (K1b), and with a pool
 *                       launchQsaIndexKCompressPaged,
 *   - ref_persist       launchQsaRawKTailWritePrefill (raw-K tails) and the kbar V-tail write,
 *   with the pool addressing of struct QsaIndexerPoolState.
 *
 * Numerics (the page: "FP32 unless stated"; readings where it is open are listed beside each
 * step):
 *   - Build with -ffp-contract=off -fno-fast-math on x86-64 (SSE): every float operation below
 *     is one IEEE binary32 operation rounded to nearest even; no FMA, no reassociation.
 *   - The sum of squares (reduction order left open by the page) is accumulated in binary64
 *     and then rounded to binary32.  Each product of two widened T values is exact in
 *     binary64; the running sum is exact too while the squares span less than 2^24 in
 *     magnitude (2^30 for bf16, whose products have fewer bits), and otherwise within 127 * 2^-53 relative of the exact sum (positive terms),
 *     so the binary32 result is the exact sum correctly rounded except within that distance of
 *     a binary32 rounding midpoint.
 *   - rsqrtf (an approximate intrinsic on the page's hardware) is taken as 1/sqrt(v) evaluated
 *     in binary64 and then narrowed: three roundings (the binary64 square root, the binary64
 *     division, the conversion to binary32).  The two binary64 steps leave a relative error
 *     below 2^-52, so the result is the correctly rounded binary32 value except where the
 *     exact 1/sqrt(v) lies within that distance of a binary32 rounding midpoint; either way it
 *     is within 0.5 ulp + 2^-29 ulp of the exact value.
 *   - Conversions between binary32 and T are written below from the IEEE 754 definitions:
 *     widening is exact; narrowing rounds to nearest, ties to even, keeps subnormals, and maps
 *     NaN to a quiet NaN.
 * OpenMP splits rows and blocks over threads; every output element is written by exactly one
 * iteration, so results do not depend on the thread count.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define REF_F16 0
#define REF_BF16 1

enum { HEADS = 4, DIM = 128, ROW = 640, KCOL = 512, HALF_ROPE = 32, CS_W = 64, RATIO = 4,
       PAGE = 128 };

/* Mirror of the page's QsaIndexerPoolState (declared here on its own, not shared). */
typedef struct {
  void* poolPtr;
  const int32_t* pageTable;
  int32_t maxPagesPerSeq;
  int32_t numPages;
  int32_t numKVHeads;
  int32_t poolHeadDim;
  int32_t headSize;
} ref_pool_t;

/* ---------------------------------------------------------------- IEEE conversions ---- */

static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bfloat16 is the top half of a binary32: widening appends 16 zero bits. */
static float bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static float f16_to_f32(uint16_t h) {
  uint32_t sign = (uint32_t)(h >> 15) << 31;
  uint32_t e = (h >> 10) & 0x1f, m = h & 0x3ff;
  if (e == 0x1f) /* inf or NaN: keep the payload, quiet the NaN */
    return bits_f32(sign | 0x7f800000u | (m << 13) | (m ? 0x00400000u : 0u));
  /* zero, subnormal (m * 2^-24) or normal ((1024 + m) * 2^(e-25)); all exact in binary32 */
  double mag = (e == 0) ? ldexp((double)m, -24) : ldexp((double)(0x400 | m), (int)e - 25);
  float f = (float)mag;
  return bits_f32(sign | f32_bits(f));
}

/* binary32 -> bfloat16, round to nearest, ties to even. */
static uint16_t f32_to_bf16(float f) {
  uint32_t u = f32_bits(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u); /* quiet NaN */
  uint32_t keep = u >> 16, rest = u & 0xffffu;
  if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u; /* carries into exp */
  return (uint16_t)keep;
}

/* binary32 -> binary16, round to nearest, ties to even, with subnormals and overflow to inf. */
static uint16_t f32_to_f16(float f) {
  uint32_t u = f32_bits(f);
  uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u | ((a >> 13) & 0x3ffu)); /* NaN */
  if (a == 0x7f800000u) return (uint16_t)(sign | 0x7c00u);                       /* inf */
  if (a < 0x00800000u) return sign; /* |f| < 2^-126: far below half the smallest subnormal */
  int e = (int)(a >> 23) - 127;               /* |f| = sig * 2^(e-23), sig in [2^23, 2^24) */
  uint32_t sig = (a & 0x7fffffu) | 0x800000u;
  /* binary16 keeps 11 significant bits for a normal result (e >= -14); below that the
   * quantum is fixed at 2^-24, so the number of dropped bits grows by one per binade. */
  int drop = (e >= -14) ? 13 : 13 + (-14 - e);
  if (drop > 24) return sign; /* |f| < 2^-25 = half the smallest subnormal: rounds to 0 */
  uint32_t q = sig >> drop, rem = sig & ((1u << drop) - 1u), half = 1u << (drop - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1u;
  if (e >= -14) {
    uint32_t E = (uint32_t)(e + 15);
    if (q == 0x800u) { q = 0x400u; E += 1u; } /* rounding carried into the next binade */
    if (E >= 31u) return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (E << 10) | (q & 0x3ffu));
  }
  return (uint16_t)(sign | q); /* subnormal; q == 0x400 is exactly the smallest normal */
}

static float widen(uint16_t h, int dt) { return dt == REF_BF16 ? bf16_to_f32(h) : f16_to_f32(h); }
static uint16_t narrow(float f, int dt) { return dt == REF_BF16 ? f32_to_bf16(f) : f32_to_f16(f); }

/* ------------------------------------------------------ norm + rope of one 128-vector ---- */

/*
 * Gemma-style RMSNorm with (1 + w) gamma, then partial neox rope, then one cast to T
 * ("Qsa Indexer Kernels": launchQsaIndexQPrep, "Exact numerics"; reused verbatim by
 * launchQsaIndexKCompress on the cast block mean).
 *   meanSq = sum_d x_d^2 / 128; inv = rsqrt(meanSq + eps); y_d = (x_d * inv) * (1 + w_d)
 *   o_i = y_i*cos_i - y_{i+32}*sin_i, o_{i+32} = y_{i+32}*cos_i + y_i*sin_i (i < 32)
 *   o_d = y_d (d >= 64); out_d = T(o_d).
 * cs is the 64-float cosSin row of the rope position: cos in [0,32), sin in [32,64).
 * dbg (nullable): meanSq, inv, and the 128 pre-cast values.
 */
static void norm_rope(const float* x, const uint16_t* w, const float* cs, float eps, int dt,
                      uint16_t* out, float* dbgMeanSq, float* dbgInv, float* dbgPre) {
  double acc = 0.0;
  for (int d = 0; d < DIM; ++d) acc += (double)x[d] * (double)x[d];
  float sumSq = (float)acc;
  float meanSq = sumSq / 128.0f;
  float v = meanSq + eps;
  float inv = (float)(1.0 / sqrt((double)v));
  float y[DIM], o[DIM];
  for (int d = 0; d < DIM; ++d) {
    float w1 = 1.0f + widen(w[d], dt);
    float xs = x[d] * inv;
    y[d] = xs * w1;
  }
  for (int i = 0; i < HALF_ROPE; ++i) {
    float c = cs[i], s = cs[HALF_ROPE + i];
    float a0 = y[i] * c, b0 = y[i + HALF_ROPE] * s;
    float a1 = y[i + HALF_ROPE] * c, b1 = y[i] * s;
    o[i] = a0 - b0;
    o[i + HALF_ROPE] = a1 + b1;
  }
  for (int d = 2 * HALF_ROPE; d < DIM; ++d) o[d] = y[d];
  for (int d = 0; d < DIM; ++d) out[d] = narrow(o[d], dt);
  if (dbgMeanSq) *dbgMeanSq = meanSq;
  if (dbgInv) *dbgInv = inv;
  if (dbgPre) memcpy(dbgPre, o, sizeof o);
}

/* ----------------------------------------------------------------------------- K1a ---- */

/*
 * launchQsaIndexQPrep: for each (b, t), rows t >= clamp(ctx[b], 0, S) are written as +0 and
 * their input is not read; otherwise each of the 4 heads (columns [128h, 128h+128)) goes
 * through norm_rope with wQ and the cosSin row of position t.
 * Debug outputs (each nullable): meanSq/inv [B,S,4], preCast [B,S,4,128]; zeros on padding.
 */
void ref_q_prep(uint16_t* qNormed, const uint16_t* indexQk, const float* cosSin,
                int32_t maxPositions, const int32_t* ctx, const uint16_t* wQ, float eps,
                int32_t B, int32_t S, int dt, float* dbgMeanSq, float* dbgInv, float* dbgPre) {
  (void)maxPositions;
  int64_t rows = (int64_t)B * S;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    int64_t b = r / S, t = r % S;
    int64_t L = ctx[b] < 0 ? 0 : (ctx[b] > S ? S : ctx[b]);
    uint16_t* out = qNormed + r * (HEADS * DIM);
    if (t >= L) {
      memset(out, 0, sizeof(uint16_t) * HEADS * DIM);
      if (dbgMeanSq) memset(dbgMeanSq + r * HEADS, 0, sizeof(float) * HEADS);
      if (dbgInv) memset(dbgInv + r * HEADS, 0, sizeof(float) * HEADS);
      if (dbgPre) memset(dbgPre + r * HEADS * DIM, 0, sizeof(float) * HEADS * DIM);
      continue;
    }
    for (int h = 0; h < HEADS; ++h) {
      float x[DIM];
      for (int d = 0; d < DIM; ++d) x[d] = widen(indexQk[r * ROW + h * DIM + d], dt);
      norm_rope(x, wQ, cosSin + t * CS_W, eps, dt, out + h * DIM,
                dbgMeanSq ? dbgMeanSq + r * HEADS + h : 0, dbgInv ? dbgInv + r * HEADS + h : 0,
                dbgPre ? dbgPre + (r * HEADS + h) * DIM : 0);
    }
  }
}

/* ------------------------------------------------------------------- pool addressing ---- */

/*
 * QsaIndexerPoolState addressing: element (page, row, head, col) of the
 * [2*numPages, 128, numKVHeads, poolHeadDim] pool is at
 * page*128*H*D + row*H*D + head*D + col; the indexer state is head 0, columns
 * [headSize, headSize+128).  Returns the element offset of column headSize of the tail row of
 * position pos in plane `plane`, or -1 when the page-table slot is out of range or the entry is
 * unused (-1) or outside [0, 2*numPages): nothing is persisted then.
 */
static int64_t pool_tail_offset(const ref_pool_t* p, int64_t b, int plane, int64_t pos) {
  int64_t slot = pos / PAGE; /* pos >= 0 here, so this is pos >> 7 */
  if (slot < 0 || slot >= p->maxPagesPerSeq) return -1;
  int32_t id = p->pageTable[(b * 2 + plane) * p->maxPagesPerSeq + slot];
  if (id == -1 || id < 0 || (int64_t)id >= 2 * (int64_t)p->numPages) return -1;
  int64_t HD = (int64_t)p->numKVHeads * p->poolHeadDim;
  int64_t row = pos % PAGE;
  return ((int64_t)id * PAGE + row) * HD + 0 * p->poolHeadDim + p->headSize;
}

/* ----------------------------------------------------------------------------- K1b ---- */

/* The block triplet of sequence b: the scalars, or entry b of the per-sequence arrays. */
static void triplet(int64_t b, int32_t bB, int32_t bE, int32_t pl, const int32_t* pastLens,
                    const int32_t* blockBegins, const int32_t* blockEnds, int32_t maxSpan,
                    int64_t* gB, int64_t* gE, int64_t* p) {
  if (pastLens) {
    *gB = blockBegins[b];
    *gE = blockEnds[b];
    if (*gE > *gB + maxSpan) *gE = *gB + maxSpan;
    *p = pastLens[b];
  } else {
    *gB = bB; *gE = bE; *p = pl;
  }
}

/*
 * K1b numerics of one block from its four raw keys ("Qsa Indexer Kernels",
 * launchQsaIndexKCompress; reused verbatim by launchQsaIndexerPreDecode): per dim d,
 * s = ((k0+k1)+k2)+k3 in binary32 in that order, mean = s * 0.25, m_T = T(mean),
 * m = f32(m_T); then norm_rope(m) with wK and the cosSin row `cs` of the block's position.
 */
static void compress_block(const uint16_t* const k[RATIO], const uint16_t* wK, const float* cs,
                           float eps, int dt, uint16_t* out, uint16_t* dbgMT, float* dbgMeanSq,
                           float* dbgInv, float* dbgPre) {
  float m[DIM];
  for (int d = 0; d < DIM; ++d) {
    float k0 = widen(k[0][d], dt), k1 = widen(k[1][d], dt);
    float k2 = widen(k[2][d], dt), k3 = widen(k[3][d], dt);
    float s = k0 + k1;
    s = s + k2;
    s = s + k3;
    float mean = s * 0.25f;
    uint16_t mT = narrow(mean, dt);
    if (dbgMT) dbgMT[d] = mT;
    m[d] = widen(mT, dt);
  }
  norm_rope(m, wK, cs, eps, dt, out, dbgMeanSq, dbgInv, dbgPre);
}

/*
 * launchQsaIndexKCompress validity: the block is complete and fully inside the provided rows,
 * 4g+3 < ctx and 4g >= pastLen; "inside the provided rows" also bounds the last row,
 * 4g+3-pastLen < S; and the rope row 4g must exist in cosSin (checkMaxPos).
 */
static int block_valid(int64_t g, int64_t ctx, int64_t p, int64_t S, int64_t maxPos,
                       int checkMaxPos) {
  int64_t t0 = 4 * g;
  if (!(t0 + 3 < ctx)) return 0;
  if (!(t0 >= p)) return 0;
  if (!(t0 + 3 - p < S)) return 0;
  if (checkMaxPos && !(t0 < maxPos)) return 0;
  return 1;
}

/*
 * launchQsaIndexKCompress / launchQsaIndexKCompressPaged: for each b and each g in the block
 * range (skipping g outside [0, numBlocks)), an invalid block writes 128 zeros and reads
 * nothing; a valid block forms, per dim d, s = ((k0+k1)+k2)+k3 in binary32 in that order,
 * mean = s * 0.25, m_T = T(mean), m = f32(m_T), then norm_rope(m) with wK at position 4g.
 * With a pool, each valid block's kbar row is also copied bit for bit to its V-tail (plane 1,
 * position 4g) when the page guard passes.
 * Debug outputs (nullable): mT [B,nb,128] (T), meanSq/inv [B,nb], preCast [B,nb,128].
 */
void ref_k_compress(uint16_t* kbar, const uint16_t* indexQk, const float* cosSin,
                    int32_t maxPositions, const int32_t* ctx, const uint16_t* wK, float eps,
                    int32_t B, int32_t S, int32_t numBlocks, int32_t blockBegin, int32_t blockEnd,
                    int32_t pastLen, const int32_t* pastLens, const int32_t* blockBegins,
                    const int32_t* blockEnds, int32_t maxBlockSpan, const ref_pool_t* pool,
                    int dt, uint16_t* dbgMT, float* dbgMeanSq, float* dbgInv, float* dbgPre) {
  int64_t span = pastLens ? maxBlockSpan : (int64_t)blockEnd - blockBegin;
  if (span <= 0) return;
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < (int64_t)B * span; ++u) {
    int64_t b = u / span, gB, gE, p;
    triplet(b, blockBegin, blockEnd, pastLen, pastLens, blockBegins, blockEnds, maxBlockSpan,
            &gB, &gE, &p);
    int64_t g = gB + u % span;
    if (g >= gE || g < 0 || g >= numBlocks) continue;
    int64_t o = b * numBlocks + g;
    uint16_t* out = kbar + o * DIM;
    if (!block_valid(g, ctx[b], p, S, maxPositions, 1)) {
      memset(out, 0, sizeof(uint16_t) * DIM);
      if (dbgMT) memset(dbgMT + o * DIM, 0, sizeof(uint16_t) * DIM);
      if (dbgMeanSq) dbgMeanSq[o] = 0.0f;
      if (dbgInv) dbgInv[o] = 0.0f;
      if (dbgPre) memset(dbgPre + o * DIM, 0, sizeof(float) * DIM);
      continue;
    }
    const uint16_t* k[RATIO];
    for (int j = 0; j < RATIO; ++j) k[j] = indexQk + ((b * S) + (4 * g + j - p)) * ROW + KCOL;
    compress_block(k, wK, cosSin + 4 * g * CS_W, eps, dt, out, dbgMT ? dbgMT + o * DIM : 0,
                   dbgMeanSq ? dbgMeanSq + o : 0, dbgInv ? dbgInv + o : 0,
                   dbgPre ? dbgPre + o * DIM : 0);
    if (pool) {
      int64_t off = pool_tail_offset(pool, b, 1, 4 * g);
      if (off >= 0) memcpy((uint16_t*)pool->poolPtr + off, out, sizeof(uint16_t) * DIM);
    }
  }
}

/* --------------------------------------------------------------------------- persist ---- */

/*
 * launchQsaRawKTailWritePrefill, generalised to a past length: tokens
 * t in [max(p, ctx - ctx%4), ctx) with 0 <= t-p < S copy indexQk row t-p, columns
 * [512, 640), bit-unmodified to their K-tail (plane 0, position t).
 * With kbar: every valid block of the range (validity without the cosSin clause) copies its
 * dense kbar row bit for bit to its V-tail (plane 1, position 4g).  Guards as
 * pool_tail_offset; no other cell changes.
 */
void ref_persist(const ref_pool_t* pool, const uint16_t* indexQk, const uint16_t* kbar,
                 const int32_t* ctx, int32_t B, int32_t S, int32_t numBlocks, int32_t blockBegin,
                 int32_t blockEnd, int32_t pastLen, const int32_t* pastLens,
                 const int32_t* blockBegins, const int32_t* blockEnds, int32_t maxBlockSpan) {
  uint16_t* base = (uint16_t*)pool->poolPtr;
  for (int64_t b = 0; b < B; ++b) {
    int64_t gB, gE, p;
    triplet(b, blockBegin, blockEnd, pastLen, pastLens, blockBegins, blockEnds, maxBlockSpan,
            &gB, &gE, &p);
    int64_t c = ctx[b];
    if (c > 0) {
      int64_t t0 = c - c % 4;
      if (t0 < p) t0 = p;
      for (int64_t t = t0; t < c; ++t) {
        int64_t r = t - p;
        if (r < 0 || r >= S) continue;
        int64_t off = pool_tail_offset(pool, b, 0, t);
        if (off >= 0)
          memcpy(base + off, indexQk + (b * S + r) * ROW + KCOL, sizeof(uint16_t) * DIM);
      }
    }
    if (!kbar) continue;
    for (int64_t g = gB; g < gE; ++g) {
      if (g < 0 || g >= numBlocks) continue;
      if (!block_valid(g, c, p, S, 0, 0)) continue;
      int64_t off = pool_tail_offset(pool, b, 1, 4 * g);
      if (off >= 0) memcpy(base + off, kbar + (b * numBlocks + g) * DIM, sizeof(uint16_t) * DIM);
    }
  }
}

/* ----------------------------------------------------------------- decode pre-pass ---- */

/*
 * launchQsaIndexerPreDecode, with n new tokens per sequence (newLens[b]; NULL means the page's
 * single token).  ctx[b] is the TOTAL length including the new tokens, so they are positions
 * p .. ctx-1 with p = ctx - n, held in indexQk rows 0 .. n-1 of [B, S, 640] (n <= S; n is also
 * capped at ctx).
 *  1. K1a numerics at each new token's position -> qNormed[b, j] ([B, S, 4, 128]); rows j >= n
 *     are +0.  ctx <= 0 or n <= 0 writes zeros and skips steps 2 and 3.
 *  2. Tokens whose block stays incomplete, [max(p, ctx - ctx%4), ctx), store their raw key
 *     bit-unmodified to their K-tail.
 *  3. Each block completed by the new tokens, g in [floor(p/4), floor(ctx/4)): keys of tokens
 *     below p are read from their pool K-tails, keys of new tokens from indexQk; the K1b numerics
 *     of compress_block at position 4g; the kbar row is written to the V-tail of token 4g.  A block
 *     whose earlier keys are not in the pool (page guard fails) is skipped.
 * Positions at or past maxPositions are outside the cosSin table: their q rows stay +0 and their
 * blocks are skipped.
 */
void ref_pre_decode(uint16_t* qNormed, const uint16_t* indexQk, const float* cosSin,
                    int32_t maxPositions, const int32_t* ctx, const int32_t* newLens,
                    const uint16_t* wQ, const uint16_t* wK, float eps, const ref_pool_t* pool,
                    int32_t B, int32_t S, int dt) {
  uint16_t* base = (uint16_t*)pool->poolPtr;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    int64_t c = ctx[b];
    int64_t n = newLens ? newLens[b] : 1;
    if (n > S) n = S;
    if (n > c) n = c;
    uint16_t* qb = qNormed + b * S * HEADS * DIM;
    memset(qb, 0, sizeof(uint16_t) * S * HEADS * DIM);
    if (c <= 0 || n <= 0) continue;
    int64_t p = c - n;
    for (int64_t j = 0; j < n; ++j) {
      int64_t t = p + j;
      if (t >= maxPositions) continue;
      for (int h = 0; h < HEADS; ++h) {
        float x[DIM];
        for (int d = 0; d < DIM; ++d) x[d] = widen(indexQk[(b * S + j) * ROW + h * DIM + d], dt);
        norm_rope(x, wQ, cosSin + t * CS_W, eps, dt, qb + (j * HEADS + h) * DIM, 0, 0, 0);
      }
    }
    int64_t t0 = c - c % 4;
    if (t0 < p) t0 = p;
    for (int64_t t = t0; t < c; ++t) {
      int64_t off = pool_tail_offset(pool, b, 0, t);
      if (off >= 0) memcpy(base + off, indexQk + (b * S + (t - p)) * ROW + KCOL, sizeof(uint16_t) * DIM);
    }
    for (int64_t g = p / 4; 4 * g + 3 < c; ++g) {
      if (4 * g >= maxPositions) continue;
      const uint16_t* k[RATIO];
      int ok = 1;
      for (int j = 0; j < RATIO && ok; ++j) {
        int64_t t = 4 * g + j;
        if (t >= p) {
          k[j] = indexQk + (b * S + (t - p)) * ROW + KCOL;
        } else {
          int64_t off = pool_tail_offset(pool, b, 0, t);
          if (off < 0) ok = 0;
          else k[j] = base + off;
        }
      }
      if (!ok) continue;
      uint16_t out[DIM];
      compress_block(k, wK, cosSin + 4 * g * CS_W, eps, dt, out, 0, 0, 0, 0);
      int64_t off = pool_tail_offset(pool, b, 1, 4 * g);
      if (off >= 0) memcpy(base + off, out, sizeof(uint16_t) * DIM);
    }
  }
}

/* ------------------------------------------------------------------- block scores ---- */

/* The score scale 1/sqrtf(128), evaluated in binary32: sqrt then divide, each rounded. */
static float score_scale(void) {
  float r = sqrtf(128.0f);
  return 1.0f / r;
}

/*
 * Block relevance of one query token against one kbar row ("Qsa Indexer Kernels",
 * launchQsaIndexScores): per head h the FP32 dot q_h . kbar (products of T values are exact
 * in binary64; the sum, whose order the page leaves open, is accumulated in binary64, exact
 * while the products span less than 2^24 (2^30 for bf16) in magnitude and otherwise within
 * 127 * 2^-53 of the sum of their magnitudes, then rounded to binary32), ReLU per head, the
 * four heads summed in ascending h in binary32, then scaled by 1/sqrtf(128) after the sum.
 */
static float block_score(const uint16_t* q, const uint16_t* kb, int dt) {
  float sum = 0.0f;
  for (int h = 0; h < HEADS; ++h) {
    double acc = 0.0;
    for (int d = 0; d < DIM; ++d) acc += (double)widen(q[h * DIM + d], dt) * (double)widen(kb[d], dt);
    float dot = (float)acc;
    float relu = dot > 0.0f ? dot : 0.0f;
    sum = sum + relu;
  }
  return score_scale() * sum;
}

/*
 * launchQsaIndexScores: logits [numRows, numBlocks] for the global rows r = b*S + t in
 * [rowStart, rowStart + numRows).  A padded row (t >= ctx[b], or ctx[b] <= 0) is -FLT_MAX
 * throughout and reads nothing; otherwise block g is visible iff g < nVis(t) = (t+1)/4 (complete
 * blocks up to t) and gets block_score, and invisible blocks get -FLT_MAX.
 */
void ref_scores(float* logits, const uint16_t* qNormed, const uint16_t* kbar, const int32_t* ctx,
                int32_t B, int32_t S, int32_t numBlocks, int32_t rowStart, int32_t numRows,
                int dt) {
  (void)B;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < numRows; ++i) {
    int64_t r = rowStart + i, b = r / S, t = r % S;
    float* out = logits + i * (int64_t)numBlocks;
    int64_t c = ctx[b];
    if (c <= 0 || t >= c) {
      for (int64_t g = 0; g < numBlocks; ++g) out[g] = -FLT_MAX;
      continue;
    }
    int64_t nVis = (t + 1) / 4;
    const uint16_t* q = qNormed + r * HEADS * DIM;
    for (int64_t g = 0; g < numBlocks; ++g)
      out[g] = g < nVis ? block_score(q, kbar + (b * numBlocks + g) * DIM, dt) : -FLT_MAX;
  }
}

/*
 * launchQsaIndexScoresDecode: one query token per sequence (qNormed [B, 1, 4, 128]) against the
 * kbar rows held in the V-tails: for g < nVis = ctx/4 (and g < maxBlocks), logits[b][g] =
 * block_score(q_b, V-tail of token 4g).  Only that prefix is written.  A block whose V-tail
 * page entry is unused or out of range has no kbar: it scores -FLT_MAX.
 */
void ref_scores_decode(float* logits, const uint16_t* qNormed, const int32_t* ctx,
                       const ref_pool_t* pool, int32_t B, int32_t maxBlocks, int dt) {
  const uint16_t* base = (const uint16_t*)pool->poolPtr;
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < B; ++b) {
    int64_t c = ctx[b];
    int64_t nVis = c > 0 ? c / 4 : 0;
    if (nVis > maxBlocks) nVis = maxBlocks;
    for (int64_t g = 0; g < nVis; ++g) {
      int64_t off = pool_tail_offset(pool, b, 1, 4 * g);
      logits[b * maxBlocks + g] =
          off < 0 ? -FLT_MAX : block_score(qNormed + b * HEADS * DIM, base + off, dt);
    }
  }
}

float ref_score_scale(void) { return score_scale(); }

/* --------------------------------------------------------------- selection + expand ---- */

enum { TOPK = 512, INDEX_WIDTH = 2051 };

/* launchQsaIndexIdsFill: ids[r * numBlocks + c] = c. */
void ref_ids_fill(int32_t* ids, int32_t numRows, int32_t numBlocks) {
  for (int64_t r = 0; r < numRows; ++r)
    for (int64_t c = 0; c < numBlocks; ++c) ids[r * numBlocks + c] = (int32_t)c;
}

/*
 * The monotone map of binary32 bit patterns to unsigned integers used for the selection
 * ("Qsa Indexer Kernels", launchQsaTopKExpandDecode): u = bits >= 0 ? bits | 0x80000000 : ~bits
 * (bits read as a signed integer).  Larger floats map to larger u; -0 maps just below +0.
 */
static uint32_t orderable(float f) {
  uint32_t b = f32_bits(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

/*
 * launchQsaIndexExpand for one row (also the expand step e. of launchQsaTopKExpandDecode):
 * out[4i+j] = sel[i]*4 + j for i < kSel, then the tail tokens out[4*kSel + j] = 4*nVis + j for
 * j < tail (always appended), then -1 up to 2051 slots.  `sel` is read only for i < kSel.
 */
static void expand_row(int32_t* out, const int32_t* sel, int64_t kSel, int64_t nVis,
                       int64_t tail) {
  int64_t n = 0;
  for (int64_t i = 0; i < kSel; ++i)
    for (int j = 0; j < 4; ++j) out[n++] = sel[i] * 4 + j;
  for (int64_t j = 0; j < tail; ++j) out[n++] = (int32_t)(4 * nVis + j);
  while (n < INDEX_WIDTH) out[n++] = -1;
}

static int64_t k_sel(int64_t nVis) { return nVis < TOPK ? nVis : TOPK; }

/*
 * launchQsaIndexExpand: rows r = b*S + t in [rowStart, rowStart + numRows) of outIdx
 * [B*S, 2051]; a padded row (t >= ctx[b], or ctx[b] <= 0) is all -1 and reads nothing.
 */
void ref_expand(int32_t* outIdx, const int32_t* sortedIds, const int32_t* ctx, int32_t B,
                int32_t S, int32_t numBlocks, int32_t rowStart, int32_t numRows) {
  (void)B;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < numRows; ++i) {
    int64_t r = rowStart + i, b = r / S, t = r % S;
    int32_t* out = outIdx + r * INDEX_WIDTH;
    if (ctx[b] <= 0 || t >= ctx[b]) {
      for (int k = 0; k < INDEX_WIDTH; ++k) out[k] = -1;
      continue;
    }
    int64_t nVis = (t + 1) / 4;
    expand_row(out, sortedIds + i * numBlocks, k_sel(nVis), nVis, (t + 1) % 4);
  }
}

/* Descending by orderable key; equal keys in ascending id (a stable sort over ascending ids). */
typedef struct { uint32_t key; int32_t id; } keyed_t;
static int by_key_desc_id_asc(const void* x, const void* y) {
  const keyed_t *a = (const keyed_t*)x, *b = (const keyed_t*)y;
  if (a->key != b->key) return a->key > b->key ? -1 : 1;
  return a->id < b->id ? -1 : (a->id > b->id);
}

/*
 * The prefill selection of the page's pipeline: ids filled per row (launchQsaIndexIdsFill),
 * sorted by descending logit with a stable radix sort over ascending ids (equal logits keep
 * ascending id order), then launchQsaIndexExpand.  Written here as exactly that: a full sort of
 * each row's numBlocks (key, id) pairs, then expand_row.  Also returns the sorted ids.
 */
void ref_topk_expand(int32_t* outIdx, int32_t* sortedIds /*nullable*/, const float* logits,
                     const int32_t* ctx, int32_t B, int32_t S, int32_t numBlocks,
                     int32_t rowStart, int32_t numRows) {
  (void)B;
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t i = 0; i < numRows; ++i) {
    int64_t r = rowStart + i, b = r / S, t = r % S;
    int32_t* out = outIdx + r * INDEX_WIDTH;
    keyed_t* kv = (keyed_t*)malloc(sizeof(keyed_t) * (numBlocks > 0 ? numBlocks : 1));
    int32_t* sorted = (int32_t*)malloc(sizeof(int32_t) * (numBlocks > 0 ? numBlocks : 1));
    for (int64_t g = 0; g < numBlocks; ++g) {
      kv[g].key = orderable(logits[i * numBlocks + g]);
      kv[g].id = (int32_t)g;
    }
    qsort(kv, (size_t)numBlocks, sizeof(keyed_t), by_key_desc_id_asc);
    for (int64_t g = 0; g < numBlocks; ++g) sorted[g] = kv[g].id;
    if (sortedIds) memcpy(sortedIds + i * numBlocks, sorted, sizeof(int32_t) * numBlocks);
    if (ctx[b] <= 0 || t >= ctx[b]) {
      for (int k = 0; k < INDEX_WIDTH; ++k) out[k] = -1;
    } else {
      int64_t nVis = (t + 1) / 4;
      expand_row(out, sorted, k_sel(nVis < numBlocks ? nVis : numBlocks), nVis, (t + 1) % 4);
    }
    free(kv);
    free(sorted);
  }
}

/*
 * launchQsaTopKExpandDecode: per sequence, the split counters splitCounters[b][0, numKVHeads)
 * of the attention that follows are zeroed when the pointer is non-null (step a.); then
 * nVis = ctx/4 (capped at maxBlocks), kSel = min(512, nVis),
 * tail = ctx%4.  nVis <= 512 selects every block.  Otherwise the selected set is the kSel
 * largest orderable keys of logits[b][0, nVis), equal keys at the threshold taken in ascending
 * block id; the selection is emitted in ascending block id order (a fixed-order scan), expanded
 * to 4 tokens each, followed by the tail tokens [4*nVis, ctx) and -1 padding to 2051.
 * ctx <= 0 gives an all -1 row.
 */
void ref_topk_expand_decode(int32_t* outIdx, const float* logits, const int32_t* ctx,
                            int32_t* splitCounters, int32_t numKVHeads, int32_t B,
                            int32_t maxBlocks) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < B; ++b) {
    int32_t* out = outIdx + b * INDEX_WIDTH;
    if (splitCounters)
      for (int64_t h = 0; h < numKVHeads; ++h) splitCounters[b * numKVHeads + h] = 0;
    int64_t c = ctx[b];
    if (c <= 0) {
      for (int k = 0; k < INDEX_WIDTH; ++k) out[k] = -1;
      continue;
    }
    int64_t nVis = c / 4;
    if (nVis > maxBlocks) nVis = maxBlocks;
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * (nVis > 0 ? nVis : 1));
    int64_t kSel = k_sel(nVis);
    if (nVis <= TOPK) {
      for (int64_t g = 0; g < nVis; ++g) sel[g] = (int32_t)g;
    } else {
      keyed_t* kv = (keyed_t*)malloc(sizeof(keyed_t) * nVis);
      for (int64_t g = 0; g < nVis; ++g) {
        kv[g].key = orderable(logits[b * maxBlocks + g]);
        kv[g].id = (int32_t)g;
      }
      qsort(kv, (size_t)nVis, sizeof(keyed_t), by_key_desc_id_asc);
      /* the first kSel of this order are the selected set; emit them by ascending id */
      char* pick = (char*)calloc((size_t)nVis, 1);
      for (int64_t i = 0; i < kSel; ++i) pick[kv[i].id] = 1;
      int64_t n = 0;
      for (int64_t g = 0; g < nVis; ++g)
        if (pick[g]) sel[n++] = (int32_t)g;
      free(pick);
      free(kv);
    }
    expand_row(out, sel, kSel, nVis, c % 4);
    free(sel);
  }
}

/* ------------------------------------------------------------------------- utilities ---- */

/* Element-wise conversions, exported so the tests can pin them against library routines. */
void ref_widen(const uint16_t* in, float* out, int64_t n, int dt) {
  for (int64_t i = 0; i < n; ++i) out[i] = widen(in[i], dt);
}
void ref_narrow(const float* in, uint16_t* out, int64_t n, int dt) {
  for (int64_t i = 0; i < n; ++i) out[i] = narrow(in[i], dt);
}

void ref_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
