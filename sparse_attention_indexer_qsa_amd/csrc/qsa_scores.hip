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
//  * B operand: 32 consecutive kbar rows (blocks).  A workgroup (8 waves, 16 tokens each as
//    two A tiles) keeps its q fragments in registers and walks 4096 blocks, 64 at a time
//    staged in LDS (double-buffered) and shared by the 8 waves; each kbar fragment a wave
//    reads from LDS feeds the MFMAs of both its A tiles.  64-block chunks keep the LDS at
//    35 KB and the registers below 128 per lane, so two workgroups (4 waves per SIMD) share a
//    CU.
//  * K = 128 in 8 steps of 16.  Every lane loads A and B with the same lane -> k mapping, so
//    the dot products do not depend on how the instruction orders k.
//  * In the 32x32 accumulator a lane holds rows 8*(v/4) + 4*(lane/32) + v%4 of column lane%32
//    for its 16 registers v: registers 4m..4m+3 are the four heads of token 2m + lane/32 of
//    the tile.  ReLU, the ascending head sum and the scale are in-lane; lanes 0..31 then store
//    32 consecutive logits of one token (a 128-byte line) and lanes 32..63 those of the next.
//  * Chunks that every token of the workgroup sees in full run in a loop of their own with no
//    masks (buffer stores from a scalar row base), walked from a chunk that depends on the
//    tile (then around), so that the workgroups in flight write different column offsets of
//    their rows rather than all the same one; the chunks holding visibility edges mask
//    per entry.  Column tiles that no token of the workgroup can see skip the contraction
//    and store -FLT_MAX.  The kernel is bound by the FP32 logits it writes: the visible
//    pieces and the -FLT_MAX runs share the HBM write bandwidth.
//
// Decode gathers kbar rows from the paged pool and scores them on MFMA too (16x16x32, the
// sequence's four heads as the A rows): the kernel is bound by those gathers.

#include <float.h>

#include <type_traits>

#include "qsa_device.h"

namespace qsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kSTokWave = 16;                      // tokens per wave (two 32-row A tiles)
constexpr int kSWaves = 8;                         // waves per workgroup
constexpr int kSThreads = 64 * kSWaves;
static_assert(kSThreads == kScoresThreads, "the ABI layer bounds the launch with kScoresThreads");
constexpr int kSTokWG = kSTokWave * kSWaves;       // tokens per workgroup (128)
constexpr int kSColTile = 32;                      // blocks per MFMA column tile
constexpr int kSColTiles = 2;                      // column tiles per staged chunk
constexpr int kSChunk = kSColTile * kSColTiles;    // blocks staged in LDS at a time (64)
constexpr int kSPieces = kSChunk * 16 / kSThreads;  // 16-byte kbar pieces staged per thread
constexpr int kSRange = 4096;                      // blocks walked by one workgroup

__device__ __forceinline__ float score_scale() { return 1.0f / __builtin_sqrtf(128.0f); }

__device__ __forceinline__ f32x16 mfma32(Bf16, const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(F16, const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Sum over the four heads, ascending, of relu(d_h) = d_h > 0 ? d_h : +0 (so -0 and NaN give
// +0), as ((relu(d0) + relu(d1)) + relu(d2)) + relu(d3).  For p >= +0, p + relu(d) has the
// same bits as max(p + d, p) (d <= 0, -0, NaN or -inf leave p; otherwise the rounded p + d is
// >= p), and both operands of that max are results of IEEE operations, so the compiler needs
// no canonicalising instruction before it: 2 instructions per head after the first.
__device__ __forceinline__ float relu_head_sum(float d0, float d1, float d2, float d3) {
  float p = d0 > 0.0f ? d0 : 0.0f;
  p = __builtin_fmaxf(p + d1, p);
  p = __builtin_fmaxf(p + d2, p);
  return __builtin_fmaxf(p + d3, p);
}

// Global rows [rowLo, rowHi) of the logits chunk.  Workgroup tile `tile` is tokens
// [128*(tile % tilesPerSeq), +128) of sequence tile / tilesPerSeq, over one range of 4096
// blocks, walked in chunks of 64 staged in LDS (double-buffered: the next chunk's loads are in
// flight while the current one is contracted).  Each wave holds the q fragments of its 16
// tokens (two 32-row A tiles) in registers for the whole range, so every kbar fragment it
// reads from LDS feeds two MFMAs.
template <class T>
__global__ __launch_bounds__(kSThreads) __attribute__((amdgpu_waves_per_eu(4, 4)))
void scores_kernel(ScoresArgs a) {
  // 2 x 64 kbar rows x 256 bytes, rows padded to 272 bytes so that 32 lanes reading one
  // 16-byte piece of 32 different rows spread over the LDS banks
  __shared__ uint4 kb_lds[2][kSChunk][17];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches below
  // workgroup w takes tile tile0 + w % numTiles over range w / numTiles: the workgroups in
  // flight together read the same few kbar ranges, which stay in cache
  const int64_t tile = a.tile0 + blockIdx.x % a.numTiles;
  const int rangeIdx = (int)(blockIdx.x / a.numTiles);
  const int64_t b = tile / a.tilesPerSeq;
  const int t0 = (int)(tile % a.tilesPerSeq) * kSTokWG;
  const int S = a.S, nB = a.numBlocks;
  const int rangeLo = rangeIdx * kSRange;
  const int rangeHi = rangeLo + kSRange < nB ? rangeLo + kSRange : nB;
  const int64_t rowLo = a.rowStart, rowHi = a.rowStart + a.numRows;
  const int64_t seqRow0 = b * S;                    // global row of token 0 of the sequence
  const int ctx = a.ctx[b];
  // token range [tLo, tHi) of the sequence whose rows are in the chunk
  const int tLo = rowLo > seqRow0 ? (int)(rowLo - seqRow0) : 0;
  const int tHi = rowHi - seqRow0 < S ? (int)(rowHi - seqRow0) : S;
  // last token of the workgroup that is a real, unpadded row of the chunk
  int tLast = t0 + kSTokWG - 1;
  if (tLast > tHi - 1) tLast = tHi - 1;
  if (tLast > ctx - 1) tLast = ctx - 1;
  const int nVisWG = tLast >= t0 ? (tLast + 1) / 4 : 0;  // blocks any row here can see
  const int computeHi = nVisWG < rangeHi ? nVisWG : rangeHi;  // contraction needed below
  const float scale = score_scale();

  // A fragments of row tile rt: row i = lane % 32 -> token tw0 + 8 rt + i/4, head i % 4;
  // k-group lane / 32
  const int tw0 = t0 + kSTokWave * wave;
  const int i = lane & 31, kg = lane >> 5;
  uint4 qa[2][8];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int tokA = tw0 + 8 * rt + (i >> 2);
    const bool readA = tokA >= tLo && tokA < tHi && tokA < ctx && rangeLo < computeHi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qa[rt][ks] = readA ? load16_u4(a.qNormed,
                                     ((seqRow0 + tokA) * 4 + (i & 3)) * kDim + 16 * ks + 8 * kg)
                         : make_uint4(0, 0, 0, 0);
  }

  // Output: in row tile rt, lane (i, kg) holds block i of a column tile for the tokens
  // tw0 + 8 rt + 2m + kg, m < 4, at byte offset boff + (8 rt + 2m) * rowBytes from the wave's
  // first row (the host bounds numBlocks so that 16 rows of offsets fit 32 bits)
  char* waveRow = reinterpret_cast<char*>(a.logits + (seqRow0 + tw0 - rowLo) * (int64_t)nB);
  const uint32_t boff = ((uint32_t)kg * (uint32_t)nB + (uint32_t)i) * 4u;
  const uint32_t rowBytes = (uint32_t)nB * 4u;

  // staging: 64 rows x 16 pieces per chunk, rows srow + 32 p for each thread.  Rows
  // that no token of the workgroup can see, or past the range, repeat the last row the
  // workgroup can see (fetch runs only when that row exists, i.e. when computeHi > rangeLo):
  // the logits they feed are all masked (-FLT_MAX) or not stored.  Straight-line loads with no
  // zero fill keep the compiler from waiting on them before they are needed.
  const uint16_t* kbSeq = static_cast<const uint16_t*>(a.kbar) + b * nB * (int64_t)kDim;
  constexpr int kRowsPerPass = kSThreads / 16;   // rows staged by one piece index (32)
  const int srow = tid >> 4, spiece = 8 * (tid & 15);
  uint4 v[kSPieces];
  auto fetch = [&](int c0) {
    const int last = computeHi - 1;
#pragma unroll
    for (int p = 0; p < kSPieces; ++p) {
      const int g = min(c0 + srow + kRowsPerPass * p, last);
      v[p] = *reinterpret_cast<const uint4*>(kbSeq + (int64_t)g * kDim + spiece);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < kSPieces; ++p) kb_lds[buf][srow + kRowsPerPass * p][tid & 15] = v[p];
  };

  // chunks below fastAll are seen in full by all 128 tokens of the workgroup, all live; the
  // two loops keep the unmasked one free of branches, so its waits are exact.  The unmasked
  // chunks are walked from a start that differs between tiles (then around), so that the
  // workgroups in flight write different column offsets of their rows at a time
  const bool wgLive = t0 >= tLo && t0 + kSTokWG <= tHi && t0 + kSTokWG <= ctx;
  const int fastAll = wgLive ? ((t0 + 1) / 4 < rangeHi ? (t0 + 1) / 4 : rangeHi) : rangeLo;
  const int nFast = fastAll > rangeLo ? (fastAll - rangeLo) / kSChunk : 0;
  const int rot = nFast > 0 ? (int)(tile % nFast) : 0;
  if (rangeLo < computeHi) {
    fetch(rangeLo + kSChunk * rot);
    stash(0);
  }
  // chunks at or past fillLo hold nothing any row of the workgroup can see: they are written
  // as -FLT_MAX row by row after the contraction loop
  const int fillLo = rangeLo + (computeHi > rangeLo ? (computeHi - rangeLo + kSChunk - 1) /
                                                          kSChunk * kSChunk : 0);
  // no global load may be outstanding on entry: a wait for the q fragments inside the loop
  // would also wait for the next chunk's prefetch (vmcnt(0); expcnt and lgkmcnt unchanged)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  int buf = 0;
  // One chunk of 64 blocks.  The next chunk's kbar loads are issued first, the contraction and
  // this chunk's stores follow, and the loaded pieces go to LDS last.  Vector memory operations
  // complete in issue order, so the wait for those loads covers only stores issued before
  // them, those of the previous chunk, never the ones just issued.  The compiler would move
  // the LDS writes up to the loads (ending the overlap); an empty asm statement that claims to
  // rewrite the loaded registers, placed after the stores, keeps them there.  kFast: every
  // token of every wave sees the whole chunk, so the stores take no masks; they go through a
  // buffer descriptor on the chunk's first row (scalar registers) with the lane's offset in one
  // VGPR and the row offset in a scalar register.
  auto chunk = [&](int c0, int cNext, auto fastTag) {
    constexpr bool kFast = decltype(fastTag)::value;
    __syncthreads();  // chunk c0 is in kb_lds[buf]; every wave is done with the other buffer
    fetch(cNext);  // past computeHi: the last row again, staged but never read
    char* chunkRow = waveRow + 4 * (int64_t)c0;
    // data format 32 bits (the field must be non-zero for untyped stores); no range limit:
    // every offset used is below 16 * 4 * numBlocks <= 2^32
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(chunkRow, 0, -1, 0x00020000);
#pragma unroll
    for (int ct = 0; ct < kSColTiles; ++ct) {
      f32x16 acc0 = f32x16{}, acc1 = f32x16{};
      // raised wave priority while the MFMAs issue: a wave in its epilogue (VALU) yields the
      // issue slot to one still feeding the matrix core, so the two overlap across waves
      // (241-247 -> 236-238 us on the long-prefill rows)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const uint4 bk = kb_lds[buf][kSColTile * ct + i][2 * ks + kg];
        acc0 = mfma32(T{}, qa[0][ks], bk, acc0);
        acc1 = mfma32(T{}, qa[1][ks], bk, acc1);
      }
      __builtin_amdgcn_s_setprio(0);
      // epilogue: registers 4m..4m+3 of tile rt hold the four heads of token 8 rt + 2m + kg
      // for block i of the column tile; ReLU per head, ascending head sum, scale
      float x[2][4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[0][m] = scale * relu_head_sum(acc0[4 * m], acc0[4 * m + 1], acc0[4 * m + 2],
                                        acc0[4 * m + 3]);
        x[1][m] = scale * relu_head_sum(acc1[4 * m], acc1[4 * m + 1], acc1[4 * m + 2],
                                        acc1[4 * m + 3]);
      }
      const int g = c0 + kSColTile * ct + i;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t rowOff = 4u * kSColTile * ct + (8u * rt + 2u * m) * rowBytes;
          if constexpr (kFast) {
            // cache policy 2: non-temporal
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x[rt][m]), rs,
                                                  (int)boff, (int)rowOff, 2);
          } else {
            const int tok = tw0 + 8 * rt + 2 * m + kg;
            const int nVisOut = tok < ctx ? (tok + 1) / 4 : 0;
            if (tok >= tLo && tok < tHi && g < rangeHi)
              __builtin_nontemporal_store(
                  g < nVisOut ? x[rt][m] : -FLT_MAX,
                  reinterpret_cast<float*>(chunkRow + boff + rowOff));
          }
        }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int p = 0; p < kSPieces; ++p)
      asm volatile("" : "+v"(v[p].x), "+v"(v[p].y), "+v"(v[p].z), "+v"(v[p].w) :: "memory");
    stash(buf ^ 1);
    buf ^= 1;
  };
  int j = rot;
  for (int k = 0; k < nFast; ++k) {
    const int jn = j + 1 == nFast ? 0 : j + 1;
    // the last unmasked chunk prefetches the first masked one
    chunk(rangeLo + kSChunk * j, rangeLo + kSChunk * (k + 1 < nFast ? jn : nFast),
          std::true_type{});
    j = jn;
  }
  for (int c0 = rangeLo + kSChunk * nFast; c0 < fillLo; c0 += kSChunk)
    chunk(c0, c0 + kSChunk, std::false_type{});
  // -FLT_MAX over [fillLo, rangeHi) of each of the wave's 16 token rows, each row written in
  // contiguous 1 KB runs (64 lanes x 16 bytes)
  const bool vec = (nB & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0;
  for (int k = 0; k < kSTokWave; ++k) {
    const int t = tw0 + k;
    if (t < tLo || t >= tHi) continue;
    float* row = a.logits + (seqRow0 + t - rowLo) * (int64_t)nB;
    for (int g = fillLo + 4 * lane; g < rangeHi; g += 4 * 64) {
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

// Decode on MFMA (v_mfma_f32_16x16x32): one wave per workgroup takes kDecGroups groups of
// 16 consecutive blocks, 16-aligned, so that a group's 64 tokens lie in one 128-token page:
// one page-table entry per group (a scalar load), issued for every group before anything
// else.  The sequence's q is the A operand (rows 0..3 = heads, rows 4..15 zero), the group's
// 16 gathered kbar rows the B operand: for k-step s lane l holds the 8 dims
// [8 (l / 16) + 32 s, +8) of block l % 16 (A: the same dims of head l % 16), so that the four
// lanes of a block read 64 contiguous bytes per load.  Lane l < 16 of the accumulator holds
// the four heads of block l % 16: ReLU, the ascending head sum and the scale there.
// Workgroup w takes chunk w % nChunks of sequence w / nChunks: consecutive workgroups, which
// the dispatcher spreads over the XCDs in turn, cover consecutive chunks of one sequence, so
// every XCD gets a share of every sequence (sequence-major placement left one XCD with 22 %
// more blocks than the mean on the decode batch, and the time followed it).  Measured on the
// 64-sequence decode batch (77 MB): 14.9 us, against 20.3 us for the earlier VALU kernel
// (DPP-row dot products, 256-thread workgroups, sequence-major); the VALU kernel with this
// placement took 17.7 us, MFMA workgroups of 4 waves 18.3 us.
constexpr int kDecGroups = 8;                    // 16-block groups per workgroup (6: 15.2 us,
                                                 // 12: 15.2 us, 16: spills)
constexpr int kDecBlocks = 16 * kDecGroups;      // blocks per workgroup

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(Bf16, const uint4& a, const uint4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(F16, const uint4& a, const uint4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <class T>
__global__ __launch_bounds__(64) void scores_decode_kernel(ScoresDecodeArgs a) {
  const int lane = threadIdx.x;
  const int n = lane & 15, kq = lane >> 4;  // block of the group; 8-dim slice of each k-step
  const int nChunks = (a.maxBlocks + kDecBlocks - 1) / kDecBlocks;
  const int64_t b = blockIdx.x / nChunks;
  const int64_t g0 = (int64_t)kDecBlocks * (blockIdx.x % nChunks);
  const int32_t* vt = a.pool.pageTable + (b * 2 + 1) * a.pool.maxPagesPerSeq;
  // The page-table entries and q depend on the block index alone: issued before the context
  // length is known (a memory clobber keeps them ahead of the early return)
  int32_t id[kDecGroups];
#pragma unroll
  for (int k = 0; k < kDecGroups; ++k) {
    const int64_t slot = (g0 + 16 * k) >> 5;  // page slot of tokens 4 (g0 + 16k) .. + 63
    id[k] = vt[slot < a.pool.maxPagesPerSeq ? slot : a.pool.maxPagesPerSeq - 1];
  }
  uint4 qa[4];
  const uint16_t* qrow =
      static_cast<const uint16_t*>(a.qNormed) + (b * 4 + (n & 3)) * kDim + 8 * kq;
#pragma unroll
  for (int s = 0; s < 4; ++s) qa[s] = *reinterpret_cast<const uint4*>(qrow + 32 * s);
  asm volatile("" ::: "memory");
  const int64_t ctx = a.ctx[b];
  int64_t nVis = ctx > 0 ? ctx / 4 : 0;
  if (nVis > a.maxBlocks) nVis = a.maxBlocks;
  if (g0 >= nVis) return;
#pragma unroll
  for (int s = 0; s < 4; ++s)
    if (n >= 4) qa[s] = make_uint4(0u, 0u, 0u, 0u);
  // V-tail rows: a group behind an entry that fails a guard of tail_offset (slot in range,
  // entry not -1 and inside the pool) reads page 0's rows and scores -FLT_MAX; rows of blocks
  // past the context are read from their page (inside the pool) and not stored
  bool ok[kDecGroups];
  uint4 kv[kDecGroups][4];
#pragma unroll
  for (int k = 0; k < kDecGroups; ++k) {
    const int64_t g = g0 + 16 * k, slot = g >> 5;
    ok[k] = (slot < a.pool.maxPagesPerSeq) & (id[k] >= 0) & (id[k] < a.pool.numIds);
    const int64_t row =
        (int64_t)(ok[k] ? id[k] : 0) * kPageTokens + ((4 * (g + n)) & (kPageTokens - 1));
    const uint16_t* p = static_cast<const uint16_t*>(a.pool.base) + row * a.pool.rowElems +
                        a.pool.headSize + 8 * kq;
#pragma unroll
    for (int s = 0; s < 4; ++s) kv[k][s] = *reinterpret_cast<const uint4*>(p + 32 * s);
  }
  const float scale = score_scale();
#pragma unroll
  for (int k = 0; k < kDecGroups; ++k) {
    const int64_t g = g0 + 16 * k;
    if (g >= nVis) break;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma16(T{}, qa[s], kv[k][s], acc);
    if (lane < 16 && g + n < nVis) {
      float sum = 0.0f;
#pragma unroll
      for (int h = 0; h < 4; ++h) sum = sum + __builtin_fmaxf(acc[h], 0.0f);
      a.logits[b * a.maxBlocks + g + n] = ok[k] ? scale * sum : -FLT_MAX;
    }
  }
}

}  // namespace

int64_t scores_workgroups(ScoresArgs& t) {
  // tiles of kSTokWG tokens covering rows [rowStart, rowStart + numRows), times the ranges
  t.tilesPerSeq = (t.S + kSTokWG - 1) / kSTokWG;
  const int64_t last = t.rowStart + t.numRows - 1;
  t.tile0 = (t.rowStart / t.S) * t.tilesPerSeq + (t.rowStart % t.S) / kSTokWG;
  t.numTiles = (last / t.S) * t.tilesPerSeq + (last % t.S) / kSTokWG - t.tile0 + 1;
  return t.numTiles * ((t.numBlocks + kSRange - 1) / kSRange);
}

hipError_t launch_scores(const ScoresArgs& a, Dt dt, hipStream_t stream) {
  ScoresArgs t = a;
  const dim3 grid((unsigned)scores_workgroups(t));
  if (dt == Dt::BF16)
    hipLaunchKernelGGL((scores_kernel<Bf16>), grid, dim3(kSThreads), 0, stream, t);
  else hipLaunchKernelGGL((scores_kernel<F16>), grid, dim3(kSThreads), 0, stream, t);
  return hipGetLastError();
}

int64_t scores_decode_workgroups(int32_t B, int32_t maxBlocks) {
  return (int64_t)B * ((maxBlocks + kDecBlocks - 1) / kDecBlocks);
}

hipError_t launch_scores_decode(const ScoresDecodeArgs& a, Dt dt, hipStream_t stream) {
  const dim3 grid((unsigned)scores_decode_workgroups(a.B, a.maxBlocks));
  if (dt == Dt::BF16)
    hipLaunchKernelGGL((scores_decode_kernel<Bf16>), grid, dim3(64), 0, stream, a);
  else hipLaunchKernelGGL((scores_decode_kernel<F16>), grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qsa
