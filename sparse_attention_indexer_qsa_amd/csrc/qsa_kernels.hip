// qsa_kernels.hip — gfx950 kernels of the QSA indexer hot path.
//
// What is computed is defined on the "Qsa Indexer Kernels" page (TensorRT-Edge-LLM C++ API
// documentation): launchQsaIndexQPrep (K1a), launchQsaIndexKCompress / ...Paged (K1b and the
// kbar V-tail) and launchQsaRawKTailWritePrefill (raw-K tails), with the pool addressing of
// QsaIndexerPoolState.  How it is computed here is our own wave64 design:
//
//  * The unit of work is a 128-element vector (an index-Q head, a raw key, a block mean) held by
//    one 16-lane DPP row.  Lane c of the row owns elements [4c, 4c+4) and [64+4c, 64+4c+4),
//    each moved with one 8-byte access (a row moves two full 128-byte lines per instruction).
//    With this split every lane holds four rope elements: lanes 0..7 hold dims i < 32 and
//    lanes 8..15 their partners i + 32, so the rope partner is lane c ^ 8, one symmetric DPP
//    move (row_ror:8), and all 16 lanes share the rope arithmetic.  A wave carries four such
//    vectors side by side: the four q heads of one token in K1a, four blocks in the
//    stand-alone K1b.
//  * Sum of squares in FP32: eight in-lane terms, then a four-step DPP butterfly (quad_perm
//    [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror).  Each step adds a lane's
//    value to its mirror's, and IEEE addition is commutative, so all 16 lanes end with the same
//    bits.  The reciprocal square root is v_rsq_f32.  (The method fixes FP32 and a warp-level
//    reduction but not its order, nor how rsqrt is rounded.)
//  * cosSin: the 64-float row of a position is staged once in LDS per wave, together with the
//    negated sines, and read by all four rows.  With -sin stored,
//    o = y*cos + partner*(+-sin) covers both halves of each pair with one add (a - b and
//    a + (-b) are the same IEEE operation).
//  * FP32 arithmetic, no FMA contraction (-ffp-contract=off), one rounding per operation.
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

// The lane's share of a 128-element vector: elements [4c, 4c+4) in `a`, [64+4c, 64+4c+4) in `b`.
struct Piece {
  uint2 a, b;
};

__device__ __forceinline__ Piece load_piece(const void* base, int64_t vec, int c) {
  const uint16_t* p = static_cast<const uint16_t*>(base) + vec + 4 * c;
  return Piece{*reinterpret_cast<const uint2*>(p), *reinterpret_cast<const uint2*>(p + 64)};
}

// Bulk inputs streamed once (indexQk rows and keys, kbar rows being persisted): non-temporal
// loads, measured ~10 % faster for this path on gfx950 than cached ones.  The cosSin row stays
// a cached load: it is the first value a wave waits for, so its latency matters more.
__device__ __forceinline__ Piece stream_piece(const void* base, int64_t vec, int c) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  const u32x2* p = reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + vec + 4 * c);
  const u32x2 x = __builtin_nontemporal_load(p), y = __builtin_nontemporal_load(p + 16);
  return Piece{make_uint2(x.x, x.y), make_uint2(y.x, y.y)};
}

__device__ __forceinline__ float4 load_cs(const float* row, int c) {
  return *reinterpret_cast<const float4*>(row + 4 * c);
}

// Outputs are written once and not read again by this path: non-temporal stores keep them from
// displacing the input stream in the caches.
__device__ __forceinline__ void store_piece(void* base, int64_t vec, int c, const Piece& v) {
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  uint16_t* p = static_cast<uint16_t*>(base) + vec + 4 * c;
  __builtin_nontemporal_store(u32x2{v.a.x, v.a.y}, reinterpret_cast<u32x2*>(p));
  __builtin_nontemporal_store(u32x2{v.b.x, v.b.y}, reinterpret_cast<u32x2*>(p + 64));
}

__device__ __forceinline__ Piece zero_piece() { return Piece{make_uint2(0, 0), make_uint2(0, 0)}; }

__device__ __forceinline__ void widen4(Bf16, const uint2& r, float (&f)[4]) {
  f[0] = __uint_as_float(r.x << 16);
  f[1] = __uint_as_float(r.x & 0xffff0000u);
  f[2] = __uint_as_float(r.y << 16);
  f[3] = __uint_as_float(r.y & 0xffff0000u);
}

__device__ __forceinline__ void widen4(F16, const uint2& r, float (&f)[4]) {
  const f16x2 lo = __builtin_bit_cast(f16x2, r.x), hi = __builtin_bit_cast(f16x2, r.y);
  f[0] = (float)lo.x;
  f[1] = (float)lo.y;
  f[2] = (float)hi.x;
  f[3] = (float)hi.y;
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
__device__ __forceinline__ uint2 narrow4(const float (&o)[4]) {
  return make_uint2(pack2(T{}, o[0], o[1]), pack2(T{}, o[2], o[3]));
}

// ---------------------------------------------------------------------- cross-lane ops ---

template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row returns the same bits.
__device__ __forceinline__ float row_sum16(float s) {
  s = s + dpp_f<0xB1>(s);   // quad_perm [1,0,3,2]
  s = s + dpp_f<0x4E>(s);   // quad_perm [2,3,0,1]
  s = s + dpp_f<0x141>(s);  // row_half_mirror
  s = s + dpp_f<0x140>(s);  // row_mirror
  return s;
}

// Value held by lane c ^ 8 of the same row (row_ror:8): the rope partner.
__device__ __forceinline__ float partner8(float v) { return dpp_f<0x128>(v); }

// LDS written by a wave and read back by other lanes of the same wave: LDS executes a wave's
// operations in order, so only the compiler must be kept from reordering them.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Stage the 16-byte piece c of a cosSin row (floats [4c, 4c+4)) into an LDS row of kCsLds
// floats, and the negated sines next to it.
__device__ __forceinline__ void stage_cos_sin(float* lds_row, const float4& v, int c) {
  *reinterpret_cast<float4*>(lds_row + 4 * c) = v;
  if (c >= 8)
    *reinterpret_cast<float4*>(lds_row + 64 + 4 * (c - 8)) = make_float4(-v.x, -v.y, -v.z, -v.w);
}

// ------------------------------------------------------------------- norm + rope + cast ---

struct RowDbg {  // debug destinations of one vector (null when not requested)
  float* meanSq;
  float* inv;
  float* pre;    // the vector's 128 pre-cast values
};

struct Gamma {   // 1 + w for the lane's 8 elements
  float a[4], b[4];
};

template <class T>
__device__ __forceinline__ Gamma load_gamma(const void* w, int c) {
  const Piece r = load_piece(w, 0, c);
  Gamma g;
  widen4(T{}, r.a, g.a);
  widen4(T{}, r.b, g.b);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    g.a[k] = 1.0f + g.a[k];
    g.b[k] = 1.0f + g.b[k];
  }
  return g;
}

// Gemma RMSNorm with (1 + w), neox rope on dims [0, 64), cast to T, for the 128-vector held
// by this lane's DPP row ("Qsa Indexer Kernels", launchQsaIndexQPrep "Exact numerics").
// xa/xb: the lane's values of dims [4c, 4c+4) and [64+4c, 64+4c+4); cs: LDS cosSin row of the
// rope position.
template <class T, bool kDbg>
__device__ __forceinline__ Piece norm_rope(const float (&xa)[4], const float (&xb)[4],
                                           const Gamma& w1, float eps, const float* cs, int c,
                                           RowDbg dbg) {
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) ss = __builtin_fmaf(xa[k], xa[k], ss);
#pragma unroll
  for (int k = 0; k < 4; ++k) ss = __builtin_fmaf(xb[k], xb[k], ss);
  ss = row_sum16(ss);
  const float meanSq = ss * (1.0f / 128.0f);
  const float inv = __builtin_amdgcn_rsqf(meanSq + eps);
  float ya[4], oa[4], ob[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    ya[k] = (xa[k] * inv) * w1.a[k];
    ob[k] = (xb[k] * inv) * w1.b[k];
  }
  // lanes 0..7 hold dims i < 32 and use -sin; lanes 8..15 hold dims i + 32 and use +sin
  const float4 cv = *reinterpret_cast<const float4*>(cs + 4 * (c & 7));
  const float4 sv = *reinterpret_cast<const float4*>(cs + (c < 8 ? 64 : 32) + 4 * (c & 7));
  const float cc[4] = {cv.x, cv.y, cv.z, cv.w}, sn[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = ya[k] * cc[k];
    const float b = partner8(ya[k]) * sn[k];
    oa[k] = a + b;
  }
  if constexpr (kDbg) {
    if (c == 0) {
      *dbg.meanSq = meanSq;
      *dbg.inv = inv;
    }
    *reinterpret_cast<float4*>(dbg.pre + 4 * c) = make_float4(oa[0], oa[1], oa[2], oa[3]);
    *reinterpret_cast<float4*>(dbg.pre + 64 + 4 * c) = make_float4(ob[0], ob[1], ob[2], ob[3]);
  }
  return Piece{narrow4<T>(oa), narrow4<T>(ob)};
}

template <bool kDbg>
__device__ __forceinline__ void zero_dbg(RowDbg dbg, int c) {
  if constexpr (kDbg) {
    if (c == 0) {
      *dbg.meanSq = 0.0f;
      *dbg.inv = 0.0f;
    }
    *reinterpret_cast<float4*>(dbg.pre + 4 * c) = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dbg.pre + 64 + 4 * c) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// Fixed-order block mean ("Qsa Indexer Kernels", launchQsaIndexKCompress) of four raw keys:
// s = ((k0 + k1) + k2) + k3, mean = s * 0.25, cast to T (returned) and widened back (ma, mb).
template <class T>
__device__ __forceinline__ Piece block_mean(const Piece (&k)[4], float (&ma)[4],
                                            float (&mb)[4]) {
  float ka[4][4], kb[4][4], sa[4], sb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    widen4(T{}, k[j].a, ka[j]);
    widen4(T{}, k[j].b, kb[j]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float s = ka[0][e] + ka[1][e];
    s = s + ka[2][e];
    s = s + ka[3][e];
    sa[e] = s * 0.25f;
    float t = kb[0][e] + kb[1][e];
    t = t + kb[2][e];
    t = t + kb[3][e];
    sb[e] = t * 0.25f;
  }
  const Piece mT{narrow4<T>(sa), narrow4<T>(sb)};
  widen4(T{}, mT.a, ma);
  widen4(T{}, mT.b, mb);
  return mT;
}

// ---------------------------------------------------------------------- pool addressing ---

// Element offset of column headSize of the tail row of `pos` in `plane` for sequence b, or -1
// when the slot is outside [0, maxPagesPerSeq) or the entry is -1 or outside [0, 2*numPages)
// (QsaIndexerPoolState: guarded before any dereference).
__device__ __forceinline__ int64_t tail_offset(const PoolArgs& p, int64_t b, int plane,
                                               int64_t pos) {
  const int64_t slot = pos >> 7;
  if (slot < 0 || slot >= p.maxPagesPerSeq) return -1;
  const int32_t id = p.pageTable[(b * 2 + plane) * p.maxPagesPerSeq + slot];
  if (id < 0 || id >= p.numIds) return -1;
  return ((int64_t)id * kPageTokens + (pos & (kPageTokens - 1))) * p.rowElems + p.headSize;
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
  const Gamma w1 = load_gamma<T>(a.wQ, c);
  const int32_t L = clamp_len(a.ctx[b], a.S);
  const int64_t row0 = (int64_t)b * a.S + t0;

  float4 csv;
  if (t0 + h < L) csv = load_cs(a.cosSin + (t0 + h) * kCsW, c);
  Piece raw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (t0 + j < L) raw[j] = stream_piece(a.indexQk, (row0 + j) * kRow + h * kDim, c);
  if (t0 + h < L) stage_cos_sin(cs_lds[wave][h], csv, c);
  wave_lds_sync();

#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (t0 + j >= a.S) break;
    const int64_t qvec = (row0 + j) * kQElems + h * kDim;
    RowDbg dbg{};
    if constexpr (kDbg) {
      dbg.meanSq = a.dMeanSq + (row0 + j) * 4 + h;
      dbg.inv = a.dInv + (row0 + j) * 4 + h;
      dbg.pre = a.dPre + qvec;
    }
    if (t0 + j < L) {
      float xa[4], xb[4];
      widen4(T{}, raw[j].a, xa);
      widen4(T{}, raw[j].b, xb);
      store_piece(a.qNormed, qvec, c, norm_rope<T, kDbg>(xa, xb, w1, a.eps, cs_lds[wave][j], c, dbg));
    } else {
      store_piece(a.qNormed, qvec, c, zero_piece());
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
  const Gamma w1 = load_gamma<T>(a.wK, c);
  const int64_t g = bB + i;
  const bool inRange = i < a.r.span && g < bE && g >= 0 && g < a.numBlocks;
  const int64_t t0 = 4 * g;
  const int64_t ctx = a.ctx[b];
  const bool valid = inRange && t0 + 3 < ctx && t0 >= p && t0 + 3 - p < a.S &&
                     t0 < a.maxPositions;

  Piece kr[4];
  if (valid) {
    const int64_t src = ((int64_t)b * a.S + (t0 - p)) * kRow + kKCol;
#pragma unroll
    for (int j = 0; j < 4; ++j) kr[j] = stream_piece(a.indexQk, src + j * kRow, c);
    stage_cos_sin(cs_lds[wave][r], load_cs(a.cosSin + t0 * kCsW, c),
                  c);
  }
  wave_lds_sync();
  if (!inRange) return;

  const int64_t o = (int64_t)b * a.numBlocks + g;
  RowDbg dbg{};
  if constexpr (kDbg) {
    dbg.meanSq = a.dMeanSq + o;
    dbg.inv = a.dInv + o;
    dbg.pre = a.dPre + o * kDim;
  }
  if (valid) {
    float ma[4], mb[4];
    const Piece mT = block_mean<T>(kr, ma, mb);
    if constexpr (kDbg) store_piece(a.dMT, o * kDim, c, mT);
    const Piece out = norm_rope<T, kDbg>(ma, mb, w1, a.eps, cs_lds[wave][r], c, dbg);
    store_piece(a.kbar, o * kDim, c, out);
    if constexpr (kPool) {
      const int64_t off = tail_offset(a.pool, b, 1, t0);
      if (off >= 0) store_piece(a.pool.base, off, c, out);
    }
  } else {
    store_piece(a.kbar, o * kDim, c, zero_piece());
    if constexpr (kDbg) store_piece(a.dMT, o * kDim, c, zero_piece());
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
    const int64_t off = tail_offset(a.pool, b, 0, t);
    if (off < 0) return;
    store_piece(a.pool.base, off, c,
                stream_piece(a.indexQk, ((int64_t)b * a.S + (t - p)) * kRow + kKCol, c));
  } else if constexpr (kKbar) {
    const int64_t i = item - kTailSlots, g = bB + i, t0 = 4 * g;
    if (!(i < a.r.span && g < bE && g >= 0 && g < a.numBlocks)) return;
    if (!(t0 + 3 < ctx && t0 >= p && t0 + 3 - p < a.S)) return;
    const int64_t off = tail_offset(a.pool, b, 1, t0);
    if (off < 0) return;
    store_piece(a.pool.base, off, c, stream_piece(a.kbar, ((int64_t)b * a.numBlocks + g) * kDim, c));
  }
}

// ----------------------------------------------------------------- fused prefill kernel ---
// One wave per 4-token block g of one sequence: K1a for its 4 tokens (row h = q head h),
// K1b for the block, the kbar V-tail, and the raw-K tails of an incomplete last block.  Every
// indexQk row and cosSin row is read once.
//
// A block whose four tokens are all inside the context takes a straight-line path: every load
// is issued up front in the order the data is consumed (gammas, the cosSin row and raw key of
// token t0 + h in row h, then the four q rows), so each wait covers only what is needed next.
// Boundary and padding blocks take a per-token path that reads only valid rows.

template <class T>
__device__ __forceinline__ Piece q_token(const Piece& raw, const Gamma& w1, float eps,
                                         const float* cs, int c) {
  float xa[4], xb[4];
  widen4(T{}, raw.a, xa);
  widen4(T{}, raw.b, xb);
  return norm_rope<T, false>(xa, xb, w1, eps, cs, c, RowDbg{});
}

// Block g of sequence b; cs/ks are the wave's LDS staging areas.
template <class T, bool kPool>
__device__ __forceinline__ void prefill_block(const PrefillArgs& a, int32_t b, int64_t g,
                                              int32_t L, const Gamma& w1q, const Gamma& w1k,
                                              float (*cs)[kCsLds], Piece (*ks)[16], int h,
                                              int c) {
  const int64_t t0 = 4 * g;
  const int64_t row0 = (int64_t)b * a.S + t0;
  const int64_t kvec = ((int64_t)b * a.numBlocks + g) * kDim;

  if (t0 + 3 < L) {
    // ---- full block
    const float4 csv = load_cs(a.cosSin + (t0 + h) * kCsW, c);
    const Piece key = stream_piece(a.indexQk, (row0 + h) * kRow + kKCol, c);
    Piece raw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = stream_piece(a.indexQk, (row0 + j) * kRow + h * kDim, c);
    stage_cos_sin(cs[h], csv, c);
    ks[h][c] = key;
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_piece(a.qNormed, (row0 + j) * kQElems + h * kDim, c,
                  q_token<T>(raw[j], w1q, a.eps, cs[j], c));
    // every row computes the block (identical bits); row 0 stores it
    const Piece kk[4] = {ks[0][c], ks[1][c], ks[2][c], ks[3][c]};
    float ma[4], mb[4];
    block_mean<T>(kk, ma, mb);
    const Piece out = norm_rope<T, false>(ma, mb, w1k, a.eps, cs[0], c, RowDbg{});
    if (h == 0) {
      store_piece(a.kbar, kvec, c, out);
      if constexpr (kPool) {
        const int64_t off = tail_offset(a.pool, b, 1, t0);
        if (off >= 0) store_piece(a.pool.base, off, c, out);
      }
    }
    return;
  }

  // ---- boundary or padding block: the kbar row is zero; tokens below L are K1a rows and,
  // since their block is incomplete, raw-K tails
  const bool tokValid = t0 + h < L;
  Piece raw[4], key;
  if (tokValid) {
    const float4 csv = load_cs(a.cosSin + (t0 + h) * kCsW, c);
    key = stream_piece(a.indexQk, (row0 + h) * kRow + kKCol, c);
    stage_cos_sin(cs[h], csv, c);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (t0 + j < L) raw[j] = stream_piece(a.indexQk, (row0 + j) * kRow + h * kDim, c);
  wave_lds_sync();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (t0 + j >= a.S) break;
    const int64_t qvec = (row0 + j) * kQElems + h * kDim;
    if (t0 + j < L)
      store_piece(a.qNormed, qvec, c, q_token<T>(raw[j], w1q, a.eps, cs[j], c));
    else
      store_piece(a.qNormed, qvec, c, zero_piece());
  }
  if (h == 0) store_piece(a.kbar, kvec, c, zero_piece());
  if constexpr (kPool) {
    if (tokValid) {
      const int64_t off = tail_offset(a.pool, b, 0, t0 + h);
      if (off >= 0) store_piece(a.pool.base, off, c, key);
    }
  }
}

template <class T, bool kPool>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a, int32_t wgPerSeq) {
  __shared__ float cs_lds[kWaves][4][kCsLds];
  __shared__ Piece k_lds[kWaves][4][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane >> 4, c = lane & 15;
  const int32_t b = blockIdx.x / wgPerSeq;
  const int64_t g = (int64_t)(blockIdx.x - b * wgPerSeq) * kWaves + wave;
  if (4 * g >= a.S) return;
  const Gamma w1q = load_gamma<T>(a.wQ, c);
  const Gamma w1k = load_gamma<T>(a.wK, c);
  const int32_t L = clamp_len(a.ctx[b], a.S);
  prefill_block<T, kPool>(a, b, g, L, w1q, w1k, cs_lds[wave], k_lds[wave], h, c);
}

// ------------------------------------------------------------------ decode pre-pass ---
// "Qsa Indexer Kernels", launchQsaIndexerPreDecode, with n new tokens per sequence (newLens;
// the page's form is one).  One workgroup per sequence; ctx is the TOTAL length, the new
// tokens are positions p .. ctx-1 (p = ctx - n) held in rows 0 .. n-1 of the sequence.
//  * K1a: wave w takes rows w, w+4, ... (row h of the wave = q head h) at position p + j.
//  * Raw-K tails: tokens [max(p, ctx - ctx%4), ctx) (their block stays incomplete), one DPP
//    row each, bit copies.
//  * Blocks completed by the new tokens, g in [p/4, ctx/4): DPP row R = 4*wave + r takes
//    g = p/4 + R, + 16, ...; keys of tokens below p come from their pool K-tails (written by
//    earlier calls), keys of new tokens from indexQk; K1b numerics; kbar to the V-tail of 4g.
//    Tails written by this call are all at positions >= p, so no read depends on them.

template <class T, bool kNewLens>
__global__ __launch_bounds__(kThreads) void pre_decode_kernel(PreDecodeArgs a) {
  __shared__ float cs_lds[kWaves][4][kCsLds];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int64_t b = blockIdx.x;
  const Gamma w1q = load_gamma<T>(a.wQ, c);
  const Gamma w1k = load_gamma<T>(a.wK, c);
  const int64_t ctx = a.ctx[b];
  int64_t n = kNewLens ? a.newLens[b] : 1;
  if (n > a.S) n = a.S;
  if (n > ctx) n = ctx;
  const bool live = ctx > 0 && n > 0;
  const int64_t p = ctx - n;
  float* cs = cs_lds[wave][r];

  for (int64_t j = wave; j < a.S; j += kWaves) {
    const int64_t qvec = ((b * a.S + j) * 4 + r) * kDim;
    const int64_t t = p + j;
    if (live && j < n && t < a.maxPositions) {
      const Piece raw = stream_piece(a.indexQk, (b * a.S + j) * kRow + r * kDim, c);
      stage_cos_sin(cs, load_cs(a.cosSin + t * kCsW, c), c);
      wave_lds_sync();
      store_piece(a.qNormed, qvec, c, q_token<T>(raw, w1q, a.eps, cs, c));
      wave_lds_sync();
    } else {
      store_piece(a.qNormed, qvec, c, zero_piece());
    }
  }
  if (!live) return;

  if (wave == kWaves - 1 && r < kTailSlots) {
    int64_t t = ctx - (ctx & 3);
    if (t < p) t = p;
    t += r;
    if (t < ctx) {
      const int64_t off = tail_offset(a.pool, b, 0, t);
      if (off >= 0)
        store_piece(a.pool.base, off, c,
                    stream_piece(a.indexQk, (b * a.S + (t - p)) * kRow + kKCol, c));
    }
  }

  const int64_t gEnd = ctx >> 2;
  for (int64_t g = (p >> 2) + 4 * wave + r; g < gEnd; g += 4 * kWaves) {
    const int64_t t0 = 4 * g;
    if (t0 >= a.maxPositions) continue;
    Piece kk[4];
    bool ok = true;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t t = t0 + j;
      if (t >= p) {
        kk[j] = stream_piece(a.indexQk, (b * a.S + (t - p)) * kRow + kKCol, c);
      } else {
        const int64_t off = tail_offset(a.pool, b, 0, t);
        if (off < 0) ok = false;
        else kk[j] = load_piece(a.pool.base, off, c);
      }
    }
    if (!ok) continue;
    stage_cos_sin(cs, load_cs(a.cosSin + t0 * kCsW, c), c);
    wave_lds_sync();
    float ma[4], mb[4];
    block_mean<T>(kk, ma, mb);
    const Piece out = norm_rope<T, false>(ma, mb, w1k, a.eps, cs, c, RowDbg{});
    const int64_t off = tail_offset(a.pool, b, 1, t0);
    if (off >= 0) store_piece(a.pool.base, off, c, out);
    wave_lds_sync();
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

hipError_t launch_pre_decode(const PreDecodeArgs& a, Dt dt, hipStream_t stream) {
  const dim3 grid((unsigned)a.B), block(kThreads);
  const bool nl = a.newLens != nullptr;
  if (dt == Dt::BF16) {
    if (nl) hipLaunchKernelGGL((pre_decode_kernel<Bf16, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((pre_decode_kernel<Bf16, false>), grid, block, 0, stream, a);
  } else {
    if (nl) hipLaunchKernelGGL((pre_decode_kernel<F16, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((pre_decode_kernel<F16, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace qsa
