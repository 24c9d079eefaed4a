// qsa_scores.hip — block-relevance scores of the QSA indexer on gfx950.
//
// "Qsa Indexer Kernels": launchQsaIndexScores (prefill) and launchQsaIndexScoresDecode (decode,
// kbar gathered from the V-tails).  For query row (b, t) and block g:
//   logit = (1/sqrtf(128)) * sum over heads h = 0..3, ascending, of relu(q_h . kbar_g)
// with FP32 dots (order left open by the page), ReLU per head, the scale after the sum.  In
// prefill, blocks g >= (t+1)/4 and padded rows (t >= ctx, or ctx <= 0) are -FLT_MAX; padded q
// rows and blocks no row of a tile can see are not read.
//
// Prefill is a dense contraction and runs on MFMA (v_mfma_f32_32x32x16 for bf16 / fp16):
//  * A operand: 32 rows = 8 consecutive tokens x 4 heads of one sequence.  qNormed is
//    [B, S, 4, 128], so these 32 head vectors are contiguous and row i = 4*token + head.
//  * B operand: 32 consecutive kbar rows (blocks).  A workgroup (4 waves, 8 tokens each) keeps
//    its q fragments in registers and walks 2048 blocks, 128 at a time staged in LDS and
//    shared by the 4 waves; each wave runs the 4 column tiles of a chunk on 4 independent
//    accumulators, so consecutive MFMAs do not wait on each other.
//  * K = 128 in 8 steps of 16.  Every lane loads A and B with the same lane -> k mapping, so
//    the dot products do not depend on how the instruction orders k.
//  * In the 32x32 accumulator a lane holds rows 8*(v/4) + 4*(lane/32) + v%4 of column lane%32
//    for its 16 registers v: registers 4m..4m+3 are the four heads of token 2m + lane/32.  ReLU,
//    the ascending head sum and the scale are in-lane, and lanes 0..31 store 32 consecutive
//    logits of a token (128 bytes).
//  * Column tiles that no token of the workgroup can see skip the contraction and store
//    -FLT_MAX.  The kernel is bound by the FP32 logits it writes.
//
// Decode gathers kbar rows from the paged pool (one 16-lane DPP row per block, the 4+4 dims
// split of qsa_device.h), four FP32 dot products per block reduced by DPP, on the VALU.

#include <float.h>

#include "qsa_device.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSTokWave = 8;                       // tokens per wave
constexpr int kSTokWG = kSTokWave * kWaves;        // tokens per workgroup (32)
constexpr int kSColTile = 32;                      // blocks per MFMA column tile
constexpr int kSColTiles = 4;                      // column tiles per staged chunk
constexpr int kSChunk = kSColTile * kSColTiles;    // blocks staged in LDS at a time (128)
constexpr int kSRange = 2048;                      // blocks walked by one workgroup

__device__ __forceinline__ float score_scale() { return 1.0f / __builtin_sqrtf(128.0f); }

__device__ __forceinline__ f32x16 mfma32(Bf16, const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(F16, const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 4x4 transpose within each DPP quad: on return, lane e of a quad holds in x[m] what lane m
// held in x[e].  Two butterfly stages (partner lane xor 1, then xor 2), each exchanging the
// registers whose index differs from the lane's in that bit.
__device__ __forceinline__ void quad_transpose(float (&x)[4], int e) {
  float y[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float t = dpp_f<0xB1>(x[m ^ 1]);  // quad_perm [1,0,3,2]: lane e ^ 1
    y[m] = ((e ^ m) & 1) ? t : x[m];
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float t = dpp_f<0x4E>(y[m ^ 2]);  // quad_perm [2,3,0,1]: lane e ^ 2
    x[m] = ((e ^ m) & 2) ? t : y[m];
  }
}

// Global rows [rowLo, rowHi) of the logits chunk.  Workgroup tile `tile0 + blockIdx.x` is
// tokens [32*(tile % tilesPerSeq), +32) of sequence tile / tilesPerSeq; blockIdx.y picks a
// range of 2048 blocks, walked in chunks of 128 staged in LDS (double-buffered: the next
// chunk's loads are in flight while the current one is contracted).  The q fragments of the
// workgroup's tokens stay in registers for the whole range.
template <class T>
__global__ __launch_bounds__(kThreads) void scores_kernel(ScoresArgs a) {
  // 2 x 128 kbar rows x 256 bytes, rows padded to 272 bytes so that 32 lanes reading one
  // 16-byte piece of 32 different rows spread over the LDS banks
  __shared__ uint4 kb_lds[2][kSChunk][17];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tile = a.tile0 + blockIdx.x;
  const int64_t b = tile / a.tilesPerSeq;
  const int64_t t0 = (tile % a.tilesPerSeq) * kSTokWG;
  const int64_t S = a.S, nB = a.numBlocks;
  const int64_t rangeLo = (int64_t)blockIdx.y * kSRange;
  const int64_t rangeHi = rangeLo + kSRange < nB ? rangeLo + kSRange : nB;
  const int64_t rowLo = a.rowStart, rowHi = a.rowStart + a.numRows;
  const int64_t ctx = a.ctx[b];
  // last token of the workgroup that is a real, unpadded row of the chunk
  int64_t tLast = t0 + kSTokWG - 1;
  if (tLast > S - 1) tLast = S - 1;
  if (tLast > ctx - 1) tLast = ctx - 1;
  if (tLast > rowHi - 1 - b * S) tLast = rowHi - 1 - b * S;
  const int64_t nVisWG = tLast >= t0 ? (tLast + 1) / 4 : 0;  // blocks any row here can see
  const int64_t computeHi = nVisWG < rangeHi ? nVisWG : rangeHi;  // contraction needed below
  const float scale = score_scale();

  // A fragments: row i = lane % 32 -> token tw0 + i/4, head i % 4; k-group lane / 32
  const int64_t tw0 = t0 + kSTokWave * wave;
  const int i = lane & 31, kg = lane >> 5;
  const int64_t tokA = tw0 + (i >> 2);
  const bool readA = tokA < S && tokA < ctx && b * S + tokA >= rowLo && b * S + tokA < rowHi &&
                     rangeLo < computeHi;
  uint4 qa[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qa[ks] = readA ? load16_u4(a.qNormed, ((b * S + tokA) * 4 + (i & 3)) * kDim + 16 * ks + 8 * kg)
                   : make_uint4(0, 0, 0, 0);

  // Output mapping after the quad transpose: lane (i = 4p + e, kg) stores blocks
  // [4p, 4p+4) of the column tile for token tw0 + 2e + kg (16 bytes).
  const int e = i & 3, p4 = (i >> 2) * 4;
  const int64_t tOut = tw0 + 2 * e + kg;
  const int64_t rOut = b * S + tOut;
  const bool live = tOut < S && rOut >= rowLo && rOut < rowHi;
  const int64_t nVisOut = tOut < ctx ? (tOut + 1) / 4 : 0;
  float* outRow = a.logits + (rOut - rowLo) * nB;
  // 16-byte stores need every row start 16-byte aligned
  const bool vec = (nB & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0;

  // staging: 128 rows x 16 pieces per chunk, 8 per thread; rows that no token of the
  // workgroup can see, or past the range, are zeros and are not read
  auto fetch = [&](int64_t c0, uint4 (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = tid + kThreads * k, row = idx >> 4, piece = idx & 15;
      const int64_t g = c0 + row;
      v[k] = g < computeHi ? load16_u4(a.kbar, (b * nB + g) * kDim + 8 * piece)
                           : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf, const uint4 (&v)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = tid + kThreads * k;
      kb_lds[buf][idx >> 4][idx & 15] = v[k];
    }
  };

  uint4 v[8];
  if (rangeLo < computeHi) {
    fetch(rangeLo, v);
    stash(0, v);
  }
  // chunks at or past fillLo hold nothing any row of the workgroup can see: they are written
  // as -FLT_MAX row by row after the contraction loop
  const int64_t fillLo = rangeLo + (computeHi > rangeLo ? (computeHi - rangeLo + kSChunk - 1) /
                                                               kSChunk * kSChunk : 0);
  int buf = 0;
  for (int64_t c0 = rangeLo; c0 < fillLo; c0 += kSChunk) {
    __syncthreads();  // chunk c0 is in kb_lds[buf]; every wave is done with the other buffer
    const bool more = c0 + kSChunk < computeHi;
    if (more) fetch(c0 + kSChunk, v);  // in flight during the contraction
    f32x16 acc[kSColTiles];
#pragma unroll
    for (int ct = 0; ct < kSColTiles; ++ct) acc[ct] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int ct = 0; ct < kSColTiles; ++ct)
        acc[ct] = mfma32(T{}, qa[ks], kb_lds[buf][kSColTile * ct + i][2 * ks + kg], acc[ct]);
    // epilogue: registers 4m..4m+3 hold the four heads of token 2m + kg for block i of the
    // column tile; ReLU per head, ascending head sum, scale, then the quad transpose
#pragma unroll
    for (int ct = 0; ct < kSColTiles; ++ct) {
      float x[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float s = __builtin_fmaxf(acc[ct][4 * m], 0.0f);
        s = s + __builtin_fmaxf(acc[ct][4 * m + 1], 0.0f);
        s = s + __builtin_fmaxf(acc[ct][4 * m + 2], 0.0f);
        s = s + __builtin_fmaxf(acc[ct][4 * m + 3], 0.0f);
        x[m] = scale * s;
      }
      quad_transpose(x, e);  // x[k]: token tOut, block p4 + k of the tile
      const int64_t g = c0 + kSColTile * ct + p4;
      if (!live || g >= rangeHi) continue;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (g + k >= nVisOut) x[k] = -FLT_MAX;
      if (vec && g + 4 <= rangeHi) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]},
                                    reinterpret_cast<f32x4*>(outRow + g));
      } else {
        for (int k = 0; k < 4; ++k)
          if (g + k < rangeHi) outRow[g + k] = x[k];
      }
    }
    if (more) stash(buf ^ 1, v);
    buf ^= 1;
  }
  // -FLT_MAX over [fillLo, rangeHi) of each of the wave's 8 token rows, each row written in
  // contiguous 1 KB runs (64 lanes x 16 bytes)
  for (int k = 0; k < kSTokWave; ++k) {
    const int64_t t = tw0 + k, r = b * S + t;
    if (t >= S || r < rowLo || r >= rowHi) continue;
    float* row = a.logits + (r - rowLo) * nB;
    for (int64_t g = fillLo + 4 * lane; g < rangeHi; g += 4 * 64) {
      if (vec && g + 4 <= rangeHi) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(f32x4{-FLT_MAX, -FLT_MAX, -FLT_MAX, -FLT_MAX},
                                    reinterpret_cast<f32x4*>(row + g));
      } else {
        for (int j = 0; j < 4; ++j)
          if (g + j < rangeHi) row[g + j] = -FLT_MAX;
      }
    }
  }
}

// Decode: grid (B, ceil(maxBlocks / 64)); DPP row R = 4*wave + r of a workgroup takes blocks
// g = 64*blockIdx.y + R + 16*k, k < 4.  q of the sequence is held by every row (4 heads x the
// lane's 8 dims).
template <class T>
__global__ __launch_bounds__(kThreads) void scores_decode_kernel(ScoresDecodeArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane >> 4, c = lane & 15;
  const int64_t b = blockIdx.x;
  const int64_t ctx = a.ctx[b];
  int64_t nVis = ctx > 0 ? ctx / 4 : 0;
  if (nVis > a.maxBlocks) nVis = a.maxBlocks;
  const int64_t gBase = 64 * (int64_t)blockIdx.y;
  if (gBase >= nVis) return;
  float qa[4][4], qb[4][4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const Piece p = load_piece(a.qNormed, (b * 4 + h) * kDim, c);
    widen4(T{}, p.a, qa[h]);
    widen4(T{}, p.b, qb[h]);
  }
  const float scale = score_scale();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int64_t g = gBase + 4 * wave + r + 16 * k;
    if (g >= nVis) break;
    const int64_t off = tail_offset(a.pool, b, 1, 4 * g);
    if (off < 0) {
      if (c == 0) a.logits[b * a.maxBlocks + g] = -FLT_MAX;
      continue;
    }
    const Piece kp = load_piece(a.pool.base, off, c);
    float ka[4], kb[4];
    widen4(T{}, kp.a, ka);
    widen4(T{}, kp.b, kb);
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float d = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) d = __builtin_fmaf(qa[h][e], ka[e], d);
#pragma unroll
      for (int e = 0; e < 4; ++e) d = __builtin_fmaf(qb[h][e], kb[e], d);
      d = row_sum16(d);
      s = s + __builtin_fmaxf(d, 0.0f);
    }
    if (c == 0) a.logits[b * a.maxBlocks + g] = scale * s;
  }
}

}  // namespace

hipError_t launch_scores(const ScoresArgs& a, Dt dt, hipStream_t stream) {
  const dim3 grid((unsigned)a.numTiles, (unsigned)((a.numBlocks + kSRange - 1) / kSRange));
  if (dt == Dt::BF16) hipLaunchKernelGGL((scores_kernel<Bf16>), grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL((scores_kernel<F16>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_scores_decode(const ScoresDecodeArgs& a, Dt dt, hipStream_t stream) {
  const dim3 grid((unsigned)a.B, (unsigned)((a.maxBlocks + 63) / 64));
  if (dt == Dt::BF16)
    hipLaunchKernelGGL((scores_decode_kernel<Bf16>), grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL((scores_decode_kernel<F16>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qsa
