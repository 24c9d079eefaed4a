// qsa_device.h — device helpers shared by the gfx950 kernels of the QSA indexer: constants of
// the method's geometry, the per-lane share of a 128-element vector, element conversions,
// DPP row operations, LDS staging of cosSin rows, the norm + rope + cast of one vector, the
// fixed-order block mean, and pool addressing.  What they compute is defined on the
// "Qsa Indexer Kernels" page; the design notes are at the top of qsa_kernels.hip.
#pragma once

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

__device__ __forceinline__ uint4 load16_u4(const void* base, int64_t elem_off) {
  return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
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

}  // namespace
}  // namespace qsa
