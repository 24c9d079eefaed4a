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

#include "qsa_device.h"

namespace qsa {
namespace {

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
