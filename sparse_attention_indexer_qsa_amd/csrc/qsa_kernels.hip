// qsa_kernels.hip — gfx950 kernels of the QSA indexer hot path.
//
// What is computed is defined on the "Qsa Indexer Kernels" page (TensorRT-Edge-LLM C++ API
// documentation): launchQsaIndexQPrep (K1a), launchQsaIndexKCompress / ...Paged (K1b and the
// kbar V-tail) and launchQsaRawKTailWritePrefill (raw-K tails), with the pool addressing of
// QsaIndexerPoolState.  How it is computed here is our own wave64 design:
//
//  * The unit of work is a 128-element vector (an index-Q head, a raw key, a block mean) held by
//    one 16-lane DPP row: lane c of the row owns elements [8c, 8c+8), loaded and stored with one
//    16-byte access.  A wave therefore carries four such vectors side by side: the four q heads
//    of one token in K1a, four blocks in the stand-alone K1b.
//  * Sum of squares: eight in-lane terms, then a four-step DPP butterfly (quad_perm [1,0,3,2],
//    quad_perm [2,3,0,1], row_half_mirror, row_mirror).  Each step adds a lane's value to its
//    mirror's, and IEEE addition is commutative, so all 16 lanes end with the same bits.
//  * Rope partner (dims i and i+32 live in lanes c and c^4): two DPP moves (row_shl:4 into
//    bank 0, row_shr:4 into bank 1).
//  * cosSin: the 64-float row of a position is staged once in LDS per wave, together with the
//    negated sines, and read by the rope lanes of all four rows.  With -sin stored,
//    o = y*cos + partner*(+-sin) covers both halves of each pair with one add (a - b and
//    a + (-b) are the same IEEE operation).
//  * FP32 arithmetic, no FMA contraction (-ffp-contract=off), one rounding per operation.  The
//    sum of squares and the reciprocal square root are carried in FP64 and rounded once to
//    FP32, which is where FP32 evaluation orders differ least from the exact value.
//  * Casts to T use the gfx950 packed converts (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32), which
//    round to nearest even with subnormals kept.
//  * Rows past the context length and invalid blocks are stored as zeros without loading
//    their inputs; page-table entries are checked before any pool address is formed.
//  * No MFMA: nothing here is a contraction; the path is bound by HBM bandwidth.

#include "qsa_internal.h"

namespace qsa {
namespace {

constexpr int kDim = 128;        // elements per head / key / kbar row
constexpr int kRow = 640;        // indexQk row: 4 q heads x 128, raw key x 128
constexpr int kKCol = 512;       // raw key columns [512, 640)
constexpr int kQElems = 512;     // qNormed elements per token
constexpr int kCsW = 64;         // cosSin row: cos[32] | sin[32]
constexpr int kCsLds = 96;       // LDS copy: cos[32] | sin[32] | -sin[32]
constexpr int kPageTokens = 128;
constexpr int kWaves = 4;        // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTailSlots = 3;    // at most 3 raw-K tail tokens per sequence

struct Bf16 {};
struct F16 {};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ element conversions ---

__device__ __forceinline__ void widen8(Bf16, const uint4& r, float (&f)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ void widen8(F16, const uint4& r, float (&f)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = __builtin_bit_cast(f16x2, w[i]);
    f[2 * i] = (float)h.x;
    f[2 * i + 1] = (float)h.y;
  }
}

__device__ __forceinline__ uint32_t pack2(Bf16, float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint32_t pack2(F16, float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

template <class T>
__device__ __forceinline__ uint4 narrow8(const float (&o)[8]) {
  return make_uint4(pack2(T{}, o[0], o[1]), pack2(T{}, o[2], o[3]), pack2(T{}, o[4], o[5]),
                    pack2(T{}, o[6], o[7]));
}

// ---------------------------------------------------------------------- cross-lane ops ---

template <int kCtrl>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}

template <int kCtrl>
__device__ __forceinline__ double dpp_d(double v) {
  const int2 p = __builtin_bit_cast(int2, v);
  return __builtin_bit_cast(double, make_int2(dpp_i<kCtrl>(p.x), dpp_i<kCtrl>(p.y)));
}

// Sum over the 16 lanes of a DPP row; every lane of the row returns the same bits.
__device__ __forceinline__ double row_sum16(double s) {
  s = s + dpp_d<0xB1>(s);   // quad_perm [1,0,3,2]
  s = s + dpp_d<0x4E>(s);   // quad_perm [2,3,0,1]
  s = s + dpp_d<0x141>(s);  // row_half_mirror
  s = s + dpp_d<0x140>(s);  // row_mirror
  return s;
}

// Value of lane c^4 for lanes c < 8 of each row (the rope partner); lanes c >= 8 keep v.
__device__ __forceinline__ float partner4(float v) {
  const int x = __builtin_bit_cast(int, v);
  int r = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0x1, false);  // bank 0 <- lane + 4
  r = __builtin_amdgcn_update_dpp(r, x, 0x114, 0xF, 0x2, false);      // bank 1 <- lane - 4
  return __builtin_bit_cast(float, r);
}

// LDS written by a wave and read back by other lanes of the same wave: LDS executes a wave's
// operations in order, so only the compiler must be kept from reordering them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Stage the 16-byte piece c of a cosSin row into an LDS row of kCsLds floats (and the
// negated sines next to it).
__device__ __forceinline__ void stage_cos_sin(float* lds_row, const float* cs_row, int c) {
  const float4 v = *reinterpret_cast<const float4*>(cs_row + 4 * c);
  *reinterpret_cast<float4*>(lds_row + 4 * c) = v;
  if (c >= 8)
    *reinterpret_cast<float4*>(lds_row + 64 + 4 * (c - 8)) = make_float4(-v.x, -v.y, -v.z, -v.w);
}

// ------------------------------------------------------------------- norm + rope + cast ---

struct RowDbg {  // debug destinations of one vector (null when not requested)
  float* meanSq;
  float* inv;
  float* pre;    // the lane's 8 pre-cast values
};

// Gemma RMSNorm with (1 + w), neox rope on dims [0, 64), cast to T, for the 128-vector held
// by this lane's DPP row ("Qsa Indexer Kernels", launchQsaIndexQPrep "Exact numerics").
// x: the lane's 8 values; w1 = 1 + w for them; cs: LDS cosSin row of the rope position.
template <class T, bool kDbg>
__device__ __forceinline__ uint4 norm_rope(const float (&x)[8], const float (&w1)[8], float eps,
                                           const float* cs, int c, RowDbg dbg) {
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < 8; ++k) ss += (double)x[k] * (double)x[k];  // products exact in FP64
  ss = row_sum16(ss);
  const float meanSq = (float)ss * (1.0f / 128.0f);
  const float v = meanSq + eps;
  const float inv = (float)(1.0 / __builtin_sqrt((double)v));
  float y[8], o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y[k] = (x[k] * inv) * w1[k];
    o[k] = y[k];
  }
  float yp[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) yp[k] = partner4(y[k]);
  if (c < 8) {
    // lanes 0..3 hold dims i < 32 (use -sin); lanes 4..7 hold dims i + 32 (use +sin)
    const float* cp = cs + 8 * (c & 3);
    const float* sp = cs + (c < 4 ? 64 : 32) + 8 * (c & 3);
    const float4 c0 = *reinterpret_cast<const float4*>(cp);
    const float4 c1 = *reinterpret_cast<const float4*>(cp + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(sp);
    const float4 s1 = *reinterpret_cast<const float4*>(sp + 4);
    const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float a = y[k] * cv[k];
      const float b = yp[k] * sv[k];
      o[k] = a + b;
    }
  }
  if constexpr (kDbg) {
    if (c == 0) {
      *dbg.meanSq = meanSq;
      *dbg.inv = inv;
    }
    *reinterpret_cast<float4*>(dbg.pre) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(dbg.pre + 4) = make_float4(o[4], o[5], o[6], o[7]);
  }
  return narrow8<T>(o);
}

template <bool kDbg>
__device__ __forceinline__ void zero_dbg(RowDbg dbg, int c) {
  if constexpr (kDbg) {
    if (c == 0) {
      *dbg.meanSq = 0.0f;
      *dbg.inv = 0.0f;
    }
    *reinterpret_cast<float4*>(dbg.pre) = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dbg.pre + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

template <class T>
__device__ __forceinline__ void load_w1(const void* w, int c, float (&w1)[8]) {
  const uint4 r = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(w) + 8 * c);
  widen8(T{}, r, w1);
#pragma unroll
  for (int k = 0; k < 8; ++k) w1[k] = 1.0f + w1[k];
}

// Fixed-order block mean ("Qsa Indexer Kernels", launchQsaIndexKCompress):
// s = ((k0 + k1) + k2) + k3, mean = s * 0.25, cast to T (returned packed) and widened back.
template <class T>
__device__ __forceinline__ uint4 block_mean(const uint4& r0, const uint4& r1, const uint4& r2,
                                            const uint4& r3, float (&m)[8]) {
  float k0[8], k1[8], k2[8], k3[8], mean[8];
  widen8(T{}, r0, k0);
  widen8(T{}, r1, k1);
  widen8(T{}, r2, k2);
  widen8(T{}, r3, k3);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    float s = k0[k] + k1[k];
    s = s + k2[k];
    s = s + k3[k];
    mean[k] = s * 0.25f;
  }
  const uint4 mT = narrow8<T>(mean);
  widen8(T{}, mT, m);
  return mT;
}

// ---------------------------------------------------------------------- pool addressing ---

// Element offset of column headSize + 8c of the tail row of `pos` in `plane` for sequence b,
// or -1 when the slot is outside [0, maxPagesPerSeq) or the entry is -1 or outside
// [0, 2*numPages) (QsaIndexerPoolState: guarded before any dereference).
__device__ __forceinline__ int64_t tail_offset(const PoolArgs& p, int64_t b, int plane,
                                               int64_t pos, int c) {
  const int64_t slot = pos >> 7;
  if (slot < 0 || slot >= p.maxPagesPerSeq) return -1;
  const int32_t id = p.pageTable[(b * 2 + plane) * p.maxPagesPerSeq + slot];
  if (id < 0 || id >= p.numIds) return -1;
  return ((int64_t)id * kPageTokens + (pos & (kPageTokens - 1))) * p.rowElems + p.headSize +
         8 * c;
}

__device__ __forceinline__ void store16(void* base, int64_t elem_off, const uint4& v) {
  *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + elem_off) = v;
}

__device__ __forceinline__ uint4 load16(const void* base, int64_t elem_off) {
  return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
}

__device__ __forceinline__ int32_t clamp_len(int32_t ctx, int32_t S) {
  return ctx < 0 ? 0 : (ctx > S ? S : ctx);
}

// --------------------------------------------------------------------------- K1a kernel ---
// One wave per 4 consecutive tokens of one sequence; row h of the wave is q head h.

template <class T, bool kDbg>
__global__ __launch_bounds__(kThreads) void q_prep_kernel(QPrepArgs a, int32_t wgPerSeq) {
  __shared__ float cs_lds[kWaves][4][kCsLds];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 4, c = lane & 15;
  const int32_t b = blockIdx.x / wgPerSeq;
  const int64_t t0 = ((int64_t)(blockIdx.x - b * wgPerSeq) * kWaves + wave) * 4;
  if (t0 >= a.S) return;
  const int32_t L = clamp_len(a.ctx[b], a.S);
  const int64_t row0 = (int64_t)b * a.S + t0;

  uint4 raw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (t0 + j < L) raw[j] = load16(a.indexQk, (row0 + j) * kRow + h * kDim + 8 * c);
  if (t0 + h < L) stage_cos_sin(cs_lds[wave][h], a.cosSin + (t0 + h) * kCsW, c);
  float w1[8];
  load_w1<T>(a.wQ, c, w1);
  wave_lds_sync();

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (t0 + j >= a.S) break;
    const int64_t qoff = (row0 + j) * kQElems + h * kDim + 8 * c;
    RowDbg dbg{};
    if constexpr (kDbg) {
      dbg.meanSq = a.dMeanSq + (row0 + j) * 4 + h;
      dbg.inv = a.dInv + (row0 + j) * 4 + h;
      dbg.pre = a.dPre + qoff;
    }
    if (t0 + j < L) {
      float x[8];
      widen8(T{}, raw[j], x);
      store16(a.qNormed, qoff, norm_rope<T, kDbg>(x, w1, a.eps, cs_lds[wave][j], c, dbg));
    } else {
      store16(a.qNormed, qoff, make_uint4(0, 0, 0, 0));
      zero_dbg<kDbg>(dbg, c);
    }
  }
}

// --------------------------------------------------------------------------- K1b kernel ---
// Row r of a wave handles one block; a workgroup covers 16 consecutive blocks of a sequence.

template <class T, bool kRanges, bool kPool, bool kDbg>
__global__ __launch_bounds__(kThreads) void k_compress_kernel(KCompressArgs a,
                                                              int32_t wgPerSeq) {
  __shared__ float cs_lds[kWaves][4][kCsLds];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int32_t b = blockIdx.x / wgPerSeq;
  const int64_t i = ((int64_t)(blockIdx.x - b * wgPerSeq) * kWaves + wave) * 4 + r;
  int64_t bB, bE, p;
  if constexpr (kRanges) {
    bB = a.r.blockBegins[b];
    bE = a.r.blockEnds[b];
    p = a.r.pastLens[b];
  } else {
    bB = a.r.blockBegin;
    bE = a.r.blockEnd;
    p = a.r.pastLen;
  }
  const int64_t g = bB + i;
  const bool inRange = i < a.r.span && g < bE && g >= 0 && g < a.numBlocks;
  const int64_t t0 = 4 * g;
  const int64_t ctx = a.ctx[b];
  const bool valid = inRange && t0 + 3 < ctx && t0 >= p && t0 + 3 - p < a.S &&
                     t0 < a.maxPositions;

  uint4 kr[4];
  if (valid) {
    const int64_t src = ((int64_t)b * a.S + (t0 - p)) * kRow + kKCol + 8 * c;
#pragma unroll
    for (int j = 0; j < 4; ++j) kr[j] = load16(a.indexQk, src + j * kRow);
    stage_cos_sin(cs_lds[wave][r], a.cosSin + t0 * kCsW, c);
  }
  float w1[8];
  load_w1<T>(a.wK, c, w1);
  wave_lds_sync();
  if (!inRange) return;

  const int64_t o = (int64_t)b * a.numBlocks + g;
  RowDbg dbg{};
  if constexpr (kDbg) {
    dbg.meanSq = a.dMeanSq + o;
    dbg.inv = a.dInv + o;
    dbg.pre = a.dPre + o * kDim + 8 * c;
  }
  if (valid) {
    float m[8];
    const uint4 mT = block_mean<T>(kr[0], kr[1], kr[2], kr[3], m);
    if constexpr (kDbg) store16(a.dMT, o * kDim + 8 * c, mT);
    const uint4 out = norm_rope<T, kDbg>(m, w1, a.eps, cs_lds[wave][r], c, dbg);
    store16(a.kbar, o * kDim + 8 * c, out);
    if constexpr (kPool) {
      const int64_t off = tail_offset(a.pool, b, 1, t0, c);
      if (off >= 0) store16(a.pool.base, off, out);
    }
  } else {
    store16(a.kbar, o * kDim + 8 * c, make_uint4(0, 0, 0, 0));
    if constexpr (kDbg) store16(a.dMT, o * kDim + 8 * c, make_uint4(0, 0, 0, 0));
    zero_dbg<kDbg>(dbg, c);
  }
}

// ----------------------------------------------------------------------- persist kernel ---
// Each row of a wave copies one 256-byte vector: items 0..2 of a sequence are its raw-K tail
// slots, items 3.. are the blocks of its range (when kbar is given).

template <bool kRanges, bool kKbar>
__global__ __launch_bounds__(kThreads) void persist_kernel(PersistArgs a, int32_t wgPerSeq) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int32_t b = blockIdx.x / wgPerSeq;
  const int64_t item = ((int64_t)(blockIdx.x - b * wgPerSeq) * kWaves + wave) * 4 + r;
  int64_t bB, bE, p;
  if constexpr (kRanges) {
    bB = a.r.blockBegins[b];
    bE = a.r.blockEnds[b];
    p = a.r.pastLens[b];
  } else {
    bB = a.r.blockBegin;
    bE = a.r.blockEnd;
    p = a.r.pastLen;
  }
  const int64_t ctx = a.ctx[b];
  if (item < kTailSlots) {
    if (ctx <= 0) return;
    int64_t t = ctx - (ctx & 3);
    if (t < p) t = p;
    t += item;
    if (t >= ctx || t - p < 0 || t - p >= a.S) return;
    const int64_t off = tail_offset(a.pool, b, 0, t, c);
    if (off < 0) return;
    store16(a.pool.base, off,
            load16(a.indexQk, ((int64_t)b * a.S + (t - p)) * kRow + kKCol + 8 * c));
  } else if constexpr (kKbar) {
    const int64_t i = item - kTailSlots, g = bB + i, t0 = 4 * g;
    if (!(i < a.r.span && g < bE && g >= 0 && g < a.numBlocks)) return;
    if (!(t0 + 3 < ctx && t0 >= p && t0 + 3 - p < a.S)) return;
    const int64_t off = tail_offset(a.pool, b, 1, t0, c);
    if (off < 0) return;
    store16(a.pool.base, off, load16(a.kbar, ((int64_t)b * a.numBlocks + g) * kDim + 8 * c));
  }
}

// ----------------------------------------------------------------- fused prefill kernel ---
// One wave per 4-token block g of one sequence: K1a for its 4 tokens (row h = q head h),
// K1b for the block, the kbar V-tail, and the raw-K tails of an incomplete last block.  Every
// indexQk row and cosSin row is read once.

template <class T, bool kPool>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a, int32_t wgPerSeq) {
  __shared__ float cs_lds[kWaves][4][kCsLds];
  __shared__ uint4 k_lds[kWaves][4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 4, c = lane & 15;
  const int32_t b = blockIdx.x / wgPerSeq;
  const int64_t g = (int64_t)(blockIdx.x - b * wgPerSeq) * kWaves + wave;
  const int64_t t0 = 4 * g;
  if (t0 >= a.S) return;
  const int32_t L = clamp_len(a.ctx[b], a.S);
  const int64_t row0 = (int64_t)b * a.S + t0;

  uint4 raw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (t0 + j < L) raw[j] = load16(a.indexQk, (row0 + j) * kRow + h * kDim + 8 * c);
  // row h also fetches the raw key of token t0 + h and stages the cosSin row of t0 + h
  const bool tokValid = t0 + h < L;
  uint4 key;
  if (tokValid) {
    key = load16(a.indexQk, (row0 + h) * kRow + kKCol + 8 * c);
    stage_cos_sin(cs_lds[wave][h], a.cosSin + (t0 + h) * kCsW, c);
  }
  float w1q[8], w1k[8];
  load_w1<T>(a.wQ, c, w1q);
  load_w1<T>(a.wK, c, w1k);
  const bool blockValid = t0 + 3 < L;
  if (blockValid) k_lds[wave][h][c] = key;
  wave_lds_sync();

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (t0 + j >= a.S) break;
    const int64_t qoff = (row0 + j) * kQElems + h * kDim + 8 * c;
    if (t0 + j < L) {
      float x[8];
      widen8(T{}, raw[j], x);
      store16(a.qNormed, qoff, norm_rope<T, false>(x, w1q, a.eps, cs_lds[wave][j], c, RowDbg{}));
    } else {
      store16(a.qNormed, qoff, make_uint4(0, 0, 0, 0));
    }
  }

  const int64_t kout = ((int64_t)b * a.numBlocks + g) * kDim + 8 * c;
  if (blockValid) {
    // every row computes the block (identical bits); row 0 stores it
    float m[8];
    block_mean<T>(k_lds[wave][0][c], k_lds[wave][1][c], k_lds[wave][2][c], k_lds[wave][3][c], m);
    const uint4 out = norm_rope<T, false>(m, w1k, a.eps, cs_lds[wave][0], c, RowDbg{});
    if (h == 0) {
      store16(a.kbar, kout, out);
      if constexpr (kPool) {
        const int64_t off = tail_offset(a.pool, b, 1, t0, c);
        if (off >= 0) store16(a.pool.base, off, out);
      }
    }
  } else {
    if (h == 0) store16(a.kbar, kout, make_uint4(0, 0, 0, 0));
    if constexpr (kPool) {
      // tokens of an incomplete block below L are the raw-K tail: copy them bit-unmodified
      if (tokValid) {
        const int64_t off = tail_offset(a.pool, b, 0, t0 + h, c);
        if (off >= 0) store16(a.pool.base, off, key);
      }
    }
  }
}

inline int32_t ceil_div(int64_t a, int64_t b) { return (int32_t)((a + b - 1) / b); }

}  // namespace

// ------------------------------------------------------------------------------ launchers ---

hipError_t launch_q_prep(const QPrepArgs& a, Dt dt, bool debug, hipStream_t stream) {
  const int32_t wgPerSeq = ceil_div(ceil_div(a.S, 4), kWaves);
  const dim3 grid((unsigned)((int64_t)a.B * wgPerSeq)), block(kThreads);
  if (dt == Dt::BF16) {
    if (debug) hipLaunchKernelGGL((q_prep_kernel<Bf16, true>), grid, block, 0, stream, a, wgPerSeq);
    else hipLaunchKernelGGL((q_prep_kernel<Bf16, false>), grid, block, 0, stream, a, wgPerSeq);
  } else {
    if (debug) hipLaunchKernelGGL((q_prep_kernel<F16, true>), grid, block, 0, stream, a, wgPerSeq);
    else hipLaunchKernelGGL((q_prep_kernel<F16, false>), grid, block, 0, stream, a, wgPerSeq);
  }
  return hipGetLastError();
}

template <class T, bool kRanges, bool kPool>
static void k_compress_dispatch_dbg(const KCompressArgs& a, bool debug, dim3 grid,
                                    int32_t wgPerSeq, hipStream_t stream) {
  if (debug)
    hipLaunchKernelGGL((k_compress_kernel<T, kRanges, kPool, true>), grid, dim3(kThreads), 0,
                       stream, a, wgPerSeq);
  else
    hipLaunchKernelGGL((k_compress_kernel<T, kRanges, kPool, false>), grid, dim3(kThreads), 0,
                       stream, a, wgPerSeq);
}

template <class T>
static void k_compress_dispatch(const KCompressArgs& a, bool debug, dim3 grid, int32_t wgPerSeq,
                                hipStream_t stream) {
  const bool ranges = a.r.pastLens != nullptr, pool = a.pool.base != nullptr;
  if (ranges && pool) k_compress_dispatch_dbg<T, true, true>(a, debug, grid, wgPerSeq, stream);
  else if (ranges) k_compress_dispatch_dbg<T, true, false>(a, debug, grid, wgPerSeq, stream);
  else if (pool) k_compress_dispatch_dbg<T, false, true>(a, debug, grid, wgPerSeq, stream);
  else k_compress_dispatch_dbg<T, false, false>(a, debug, grid, wgPerSeq, stream);
}

hipError_t launch_k_compress(const KCompressArgs& a, Dt dt, bool debug, hipStream_t stream) {
  const int32_t wgPerSeq = ceil_div(a.r.span, 4 * kWaves);
  const dim3 grid((unsigned)((int64_t)a.B * wgPerSeq));
  if (dt == Dt::BF16) k_compress_dispatch<Bf16>(a, debug, grid, wgPerSeq, stream);
  else k_compress_dispatch<F16>(a, debug, grid, wgPerSeq, stream);
  return hipGetLastError();
}

hipError_t launch_persist(const PersistArgs& a, hipStream_t stream) {
  const bool ranges = a.r.pastLens != nullptr, kbar = a.kbar != nullptr;
  const int64_t items = kTailSlots + (kbar ? (int64_t)a.r.span : 0);
  const int32_t wgPerSeq = ceil_div(items, 4 * kWaves);
  const dim3 grid((unsigned)((int64_t)a.B * wgPerSeq)), block(kThreads);
  if (ranges && kbar) hipLaunchKernelGGL((persist_kernel<true, true>), grid, block, 0, stream, a, wgPerSeq);
  else if (ranges) hipLaunchKernelGGL((persist_kernel<true, false>), grid, block, 0, stream, a, wgPerSeq);
  else if (kbar) hipLaunchKernelGGL((persist_kernel<false, true>), grid, block, 0, stream, a, wgPerSeq);
  else hipLaunchKernelGGL((persist_kernel<false, false>), grid, block, 0, stream, a, wgPerSeq);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, Dt dt, hipStream_t stream) {
  const int32_t wgPerSeq = ceil_div(ceil_div(a.S, 4), kWaves);
  const dim3 grid((unsigned)((int64_t)a.B * wgPerSeq)), block(kThreads);
  const bool pool = a.pool.base != nullptr;
  if (dt == Dt::BF16) {
    if (pool) hipLaunchKernelGGL((prefill_kernel<Bf16, true>), grid, block, 0, stream, a, wgPerSeq);
    else hipLaunchKernelGGL((prefill_kernel<Bf16, false>), grid, block, 0, stream, a, wgPerSeq);
  } else {
    if (pool) hipLaunchKernelGGL((prefill_kernel<F16, true>), grid, block, 0, stream, a, wgPerSeq);
    else hipLaunchKernelGGL((prefill_kernel<F16, false>), grid, block, 0, stream, a, wgPerSeq);
  }
  return hipGetLastError();
}

}  // namespace qsa
