// qsa_select.hip — top-512 block selection and expansion to token indices on gfx950.
//
// "Qsa Indexer Kernels": launchQsaIndexIdsFill, launchQsaIndexExpand (K4) and
// launchQsaTopKExpandDecode (B3).  The page's prefill selection is ids fill + a stable
// descending segmented radix sort of every row + K4 over the first kSel = min(512, nVis)
// entries; here it is one kernel per row that finds the kSel largest keys by radix select and
// sorts only those, which gives the same first kSel ids in the same order.
//
//  * Keys are the monotone map of the FP32 bits, u = bits >= 0 ? bits | 0x80000000 : ~bits; a
//    row's order is descending u, equal u in ascending block id (the stable sort's order).
//  * Radix select, MSB first, four 8-bit digits: per pass each wave histograms the digit of
//    the keys that match the prefix found so far (LDS atomics into its own 256 bins), a block
//    suffix scan over the bins finds the digit of the kSel-th largest key.  After four passes
//    the threshold key T is known with the number `need` of keys equal to T that are taken.
//  * Compaction in ascending id: 256 ids per step, wave ballots give each lane its rank among
//    keys equal to T and its output position.  Decode writes the expansion directly (its
//    selection is emitted in ascending id); prefill collects the <= 512 (key, id) pairs in
//    LDS and sorts them by a bitonic network before expanding.
//  * One workgroup of 256 threads per row; the row's keys are re-read from L2 on every pass.

#include <float.h>

#include "qsa_device.h"

namespace qsa {
namespace {

constexpr int kTopK = 512;
constexpr int kIndexWidth = 2051;   // 4 * 512 + 3
constexpr int kSelThreads = 256;

__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Inclusive suffix sum over the 256 threads of the block: thread j returns sum_{i >= j} v_i.
__device__ __forceinline__ int block_suffix_sum(int v, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
#pragma unroll
  for (int off = 1; off < kSelThreads; off <<= 1) {
    const int add = tid + off < kSelThreads ? sh[tid + off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int r = sh[tid];
  __syncthreads();
  return r;
}

// Exclusive prefix count of `flag` over the block in thread order; *total = count of flags.
__device__ __forceinline__ int block_rank(bool flag, int* shWave, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint64_t m = __ballot(flag);
  const int inWave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) shWave[wave] = __popcll(m);
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    before += w < wave ? shWave[w] : 0;
    all += shWave[w];
  }
  __syncthreads();
  *total = all;
  return before + inWave;
}

struct SelectShared {
  int hist[kSelThreads / 64][256];
  int scan[kSelThreads];
  int wave[kSelThreads / 64];
  int found[2];
};

// The kSel-th largest orderable key T of keys[0, n) and the number of keys equal to T that
// the selection takes (in ascending id): every key > T is selected.
__device__ void radix_select(const float* keys, int n, int kSel, SelectShared& sh,
                             uint32_t* thr, int* need) {
  const int tid = threadIdx.x, wave = tid >> 6;
  uint32_t prefix = 0, mask = 0;
  int kRem = kSel;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int j = tid; j < (kSelThreads / 64) * 256; j += kSelThreads) (&sh.hist[0][0])[j] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const uint32_t u = orderable(keys[i]);
      if ((u & mask) == prefix) atomicAdd(&sh.hist[wave][(u >> shift) & 0xFF], 1);
    }
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kSelThreads / 64; ++w) tot += sh.hist[w][tid];
    const int cum = block_suffix_sum(tot, sh.scan);        // keys with digit >= tid
    const int above = cum - tot;                           // keys with digit > tid
    if (cum >= kRem && above < kRem) {                     // exactly one bin
      sh.found[0] = tid;
      sh.found[1] = above;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.found[0] << shift;
    mask |= 0xFFu << shift;
    kRem -= sh.found[1];
    __syncthreads();
  }
  *thr = prefix;
  *need = kRem;
}

__device__ __forceinline__ void write_tail_and_pad(int* out, int from, int64_t nVis, int tail) {
  for (int s = from + threadIdx.x; s < kIndexWidth; s += kSelThreads)
    out[s] = s - from < tail ? (int)(4 * nVis + (s - from)) : -1;
}

// ------------------------------------------------------------------------------ kernels ---

__global__ __launch_bounds__(kSelThreads) void ids_fill_kernel(int32_t* ids, int64_t total,
                                                               int32_t numBlocks) {
  for (int64_t i = (int64_t)blockIdx.x * kSelThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kSelThreads)
    ids[i] = (int32_t)(i % numBlocks);
}

// K4: one workgroup per row of the chunk; threads stride the 2051 output slots.
__global__ __launch_bounds__(kSelThreads) void expand_kernel(ExpandArgs a) {
  const int64_t i = blockIdx.x, r = a.rowStart + i, b = r / a.S, t = r % a.S;
  int32_t* out = a.outIdx + r * kIndexWidth;
  const int64_t c = a.ctx[b];
  if (c <= 0 || t >= c) {
    for (int s = threadIdx.x; s < kIndexWidth; s += kSelThreads) out[s] = -1;
    return;
  }
  const int64_t nVis = (t + 1) / 4;
  const int kSel = (int)(nVis < kTopK ? nVis : kTopK);
  const int tail = (int)((t + 1) % 4);
  const int32_t* srt = a.sortedIds + i * a.numBlocks;
  for (int s = threadIdx.x; s < 4 * kSel; s += kSelThreads) out[s] = srt[s >> 2] * 4 + (s & 3);
  write_tail_and_pad(out, 4 * kSel, nVis, tail);
}

// Prefill selection + K4 for one row of the chunk.  Candidates are the row's visible blocks
// [0, nVis): the entries past them are -FLT_MAX by the scores contract and are not read.
__global__ __launch_bounds__(kSelThreads) void topk_expand_kernel(TopkArgs a) {
  __shared__ SelectShared sh;
  __shared__ uint32_t selKey[kTopK];
  __shared__ int32_t selId[kTopK];
  const int tid = threadIdx.x;
  const int64_t i = blockIdx.x, r = a.rowStart + i, b = r / a.S, t = r % a.S;
  int32_t* out = a.outIdx + r * kIndexWidth;
  const int64_t c = a.ctx[b];
  if (c <= 0 || t >= c) {
    for (int s = tid; s < kIndexWidth; s += kSelThreads) out[s] = -1;
    return;
  }
  const int64_t nVisT = (t + 1) / 4;
  const int n = (int)(nVisT < a.numBlocks ? nVisT : a.numBlocks);
  const int kSel = n < kTopK ? n : kTopK;
  const float* keys = a.logits + i * a.numBlocks;
  uint32_t thr = 0;
  int need = n;  // n <= kTopK: every candidate is taken
  if (n > kTopK) radix_select(keys, n, kSel, sh, &thr, &need);
  // compaction in ascending id
  int eqBefore = 0, selBefore = 0;
  for (int base = 0; base < n; base += kSelThreads) {
    const int g = base + tid;
    const uint32_t u = g < n ? orderable(keys[g]) : 0u;
    const bool eq = g < n && (n <= kTopK || u == thr);
    int eqTot, selTot;
    const int eqRank = block_rank(eq, sh.wave, &eqTot) + eqBefore;
    const bool sel = g < n && (n <= kTopK || u > thr || (eq && eqRank < need));
    const int pos = block_rank(sel, sh.wave, &selTot) + selBefore;
    if (sel && pos < kTopK) {
      selKey[pos] = u;
      selId[pos] = g;
    }
    eqBefore += eqTot;
    selBefore += selTot;
  }
  // pad to 512 with entries that sort last, then bitonic sort: key descending, id ascending
  for (int s = kSel + tid; s < kTopK; s += kSelThreads) {
    selKey[s] = 0u;
    selId[s] = 0x7FFFFFFF;
  }
  __syncthreads();
  for (int size = 2; size <= kTopK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int x = tid; x < kTopK; x += kSelThreads) {
        const int y = x ^ stride;
        if (y > x) {
          const bool descBlock = (x & size) == 0;  // this half of the network sorts "first"
          const uint32_t kx = selKey[x], ky = selKey[y];
          const int32_t ix = selId[x], iy = selId[y];
          // "first" = larger key, then smaller id
          const bool yFirst = ky > kx || (ky == kx && iy < ix);
          if (yFirst == descBlock) {
            selKey[x] = ky;
            selKey[y] = kx;
            selId[x] = iy;
            selId[y] = ix;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int s = tid; s < 4 * kSel; s += kSelThreads) out[s] = selId[s >> 2] * 4 + (s & 3);
  write_tail_and_pad(out, 4 * kSel, nVisT, (int)((t + 1) % 4));
}

// Decode selection + expand for one sequence: nVis = ctx/4 (capped at maxBlocks); nVis <= 512
// takes every block without reading logits; the selection is emitted in ascending block id.
// The sequence's split counters of the attention that follows are zeroed first.
__global__ __launch_bounds__(kSelThreads) void topk_expand_decode_kernel(TopkDecodeArgs a) {
  __shared__ SelectShared sh;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  int32_t* out = a.outIdx + b * kIndexWidth;
  if (a.splitCounters != nullptr)
    for (int h = tid; h < a.numKVHeads; h += kSelThreads) a.splitCounters[b * a.numKVHeads + h] = 0;
  const int64_t c = a.ctx[b];
  if (c <= 0) {
    for (int s = tid; s < kIndexWidth; s += kSelThreads) out[s] = -1;
    return;
  }
  const int64_t nVisC = c / 4;
  const int n = (int)(nVisC < a.maxBlocks ? nVisC : a.maxBlocks);
  const int kSel = n < kTopK ? n : kTopK;
  if (n <= kTopK) {
    for (int s = tid; s < 4 * n; s += kSelThreads) out[s] = s;  // block s/4, token s%4
  } else {
    const float* keys = a.logits + b * a.maxBlocks;
    uint32_t thr;
    int need;
    radix_select(keys, n, kSel, sh, &thr, &need);
    int eqBefore = 0, selBefore = 0;
    for (int base = 0; base < n; base += kSelThreads) {
      const int g = base + tid;
      const uint32_t u = g < n ? orderable(keys[g]) : 0u;
      const bool eq = g < n && u == thr;
      int eqTot, selTot;
      const int eqRank = block_rank(eq, sh.wave, &eqTot) + eqBefore;
      const bool sel = g < n && (u > thr || (eq && eqRank < need));
      const int pos = block_rank(sel, sh.wave, &selTot) + selBefore;
      if (sel && pos < kSel) {
#pragma unroll
        for (int j = 0; j < 4; ++j) out[4 * pos + j] = 4 * g + j;
      }
      eqBefore += eqTot;
      selBefore += selTot;
    }
  }
  write_tail_and_pad(out, 4 * kSel, n, (int)(c % 4));
}

}  // namespace

hipError_t launch_ids_fill(int32_t* ids, int64_t total, int32_t numBlocks, hipStream_t stream) {
  int64_t wg = (total + kSelThreads - 1) / kSelThreads;
  if (wg > 65536) wg = 65536;
  hipLaunchKernelGGL(ids_fill_kernel, dim3((unsigned)wg), dim3(kSelThreads), 0, stream, ids,
                     total, numBlocks);
  return hipGetLastError();
}

hipError_t launch_expand(const ExpandArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)a.numRows), dim3(kSelThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_topk_expand(const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(topk_expand_kernel, dim3((unsigned)a.numRows), dim3(kSelThreads), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_topk_expand_decode(const TopkDecodeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(topk_expand_decode_kernel, dim3((unsigned)a.B), dim3(kSelThreads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace qsa
