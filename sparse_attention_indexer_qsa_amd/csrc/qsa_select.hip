// qsa_select.hip — top-512 block selection and expansion to token indices on gfx950.
//
// "Qsa Indexer Kernels": launchQsaIndexIdsFill, launchQsaIndexExpand (K4) and
// launchQsaTopKExpandDecode (B3).  The page's prefill selection is ids fill + a stable
// descending segmented radix sort of every row + K4 over the first kSel = min(512, nVis)
// entries; here one kernel per row finds the kSel largest keys and sorts only those, which
// gives the same first kSel ids in the same order.
//
// Keys are the monotone map of the FP32 bits, u = bits >= 0 ? bits | 0x80000000 : ~bits; a
// row's order is descending u, equal u in ascending block id (the stable sort's order).
//
// Register-resident rows (prefill: 256 threads, up to 72 keys each, 18432 blocks at most;
// decode: 512 threads per sequence, up to 64 keys each, which shortens a sequence's latency,
// 32768 blocks at most):
//  * The row is read from HBM once, 16 bytes per lane, into registers.  Thread t holds the
//    ids ((g * threads + t) * 4 + e) for its register groups g and e < 4.
//  * Padding: registers past the row hold u = 0 with ids >= n.  In the (u desc, id asc)
//    order every padding key comes after every real key, so while kSel <= n the kSel first
//    keys of the padded row are those of the row, and no step needs to tell them apart.
//  * Window: lo is the smallest of the maxima of 512 disjoint key sets that each hold a real
//    key, so at least 512 keys are at or above it: the even and the odd register groups of
//    each of 256 threads once n >= 2048 (prefill), all the keys of each of 512 threads once
//    n >= 2048 (decode); shorter rows take lo = the row minimum.  With hi the row maximum, the
//    kSel-th largest key lies in [lo, hi], and rows with many equal low keys (a ReLU's zeros)
//    keep them out of the histograms.
//  * Radix select inside the window, MSB first: each pass histograms (LDS atomics, 256 bins)
//    only the keys inside the current window, at a shift that spreads the window over the 256
//    bins, and a one-wave suffix scan picks the bin holding the kSel-th largest.  The window
//    holds a few thousand keys of a row (about 512 ln 512 for independent keys), so the bins
//    are spread and the atomics rarely collide.  After the first pass the keys at or above
//    the chosen bin (a few hundred) are compacted into LDS and the later passes run on them
//    alone.  The result is the threshold key T, the number `need` of keys equal to T that are
//    taken (ascending id) and their count `ties`.
//  * Prefill: the keys >= T (kSel - need + ties of them; ties normally = need) are gathered as
//    64-bit (u, ~id) composites and sorted descending by a bitonic network (strides < 64 by
//    DPP moves and permlane swaps, 64 and 128 through LDS, larger ones within a thread), so
//    equal keys come out in ascending id and the first kSel are the result.  More than 1024
//    such keys (many equal keys at T), or candidates too many for LDS after the first pass,
//    take the ordered path below, then the same sort.
//  * Decode: the selection is emitted in ascending id: the counts before each key of keys
//    above T and of keys equal to T come from per-wave counts of each register group (one
//    barrier) and ballots within the wave; each key writes its id to its rank in LDS (or to
//    a spare slot when not taken), and the ranks are written out in order.
//
// Prefill rows longer than 18432 blocks take the one-wave-per-row kernel (a walk of the row
// against a running threshold into an LDS candidate buffer, below).  Decode rows longer than
// 32768 blocks (up to 262144) are cut into at most 8 chunks, each selected by a workgroup of
// its own, and a second kernel merges the chunks' candidates (below); longer ones take the
// streaming kernel at the end of the file (the same radix select with 8-bit digits over the
// whole key range, the row re-read from L2 on every pass), 256 threads per row.

#include <float.h>

#include "qsa_device.h"

namespace qsa {
namespace {

constexpr int kTopK = 512;
constexpr int kIndexWidth = 2051;   // 4 * 512 + 3
constexpr int kSelThreads = 256;    // streaming kernels
constexpr int kRT = 256;            // register-resident prefill kernel: threads per row
constexpr int kDT = 512;            // register-resident decode kernel: threads per sequence
constexpr int kMaxW = kDT / 64;     // most waves of a register-resident workgroup
constexpr int kCandCap = 2048;      // keys kept in LDS after the first radix pass
constexpr int kRegMaxKeys = 72;     // prefill: most keys per thread of the register kernel

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ uint32_t orderable_bits(uint32_t b) {
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

__device__ __forceinline__ void write_tail_and_pad(int* out, int from, int64_t nVis, int tail,
                                                   int nthreads) {
  for (int s = from + (int)threadIdx.x; s < kIndexWidth; s += nthreads)
    out[s] = s - from < tail ? (int)(4 * nVis + (s - from)) : -1;
}

// ------------------------------------------------------------------ register-resident ---

struct RegShared {
  int hist[3][256];          // radix histograms, taking turns between passes
  int wcnt[2][kMaxW];        // per-wave counts (double-buffered by caller's parity)
  int gcnt[16 * kMaxW];      // ordered_select: per register group and wave, packed counts
  uint32_t red[2][kMaxW];    // per-wave max / min
  int ncand;                 // keys placed in candU/candId so far (compact_keys)
  int rankBig;               // rank_sort: a bucket holds more than kRankMaxBin composites
  // 256-byte aligned: a candidate's slot is addressed from one base with constant offsets
  alignas(256) uint32_t candU[kCandCap];
  alignas(256) int32_t candId[kCandCap];
  uint64_t sortBuf[2 * kTopK];
  union {
    // rank_sort: per bucket, count | first slot << 16; dead once the composites are placed
    uint32_t rankBins[1024];
    int32_t selId[kTopK + 64];  // ordered_select: ranks kTopK.. take the unselected keys' writes
  };
};

// Id of register key r of thread tid in a workgroup of NT threads.
template <int NT>
__device__ __forceinline__ int key_id(int r, int tid) {
  return (((r >> 2) * NT + tid) << 2) + (r & 3);
}

// threadIdx.x through an empty asm, for per-key id computations: the compiler cannot merge them
// with those of another code path and hoist them, which would hold registers per key across
// the radix select (measured: 15 VGPRs at 64 keys per thread in the decode kernel).
__device__ __forceinline__ int fresh_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ uint64_t composite(uint32_t u, int id) {
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)id;
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Value of lane (lane ^ j) of the wave, j in {1, 2, 4, 8, 16, 32}, by DPP and the permlane
// swaps (VALU; no LDS round trip): quad_perm [1,0,3,2] and [2,3,0,1] for 1 and 2;
// row_half_mirror then quad_perm [3,2,1,0] for 4 (lane ^ 7 ^ 3); row_ror:8 for 8; for 16 and
// 32 the swap of a register with itself leaves the wanted row (pair) in one of its two results.
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int j) {
  const int lane = threadIdx.x & 63;
  switch (j) {
    case 1: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);
    case 4:
      return __builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false), 0x1B,
                                      0xF, 0xF, false);
    case 8: return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);
    case 16: {
      const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (lane & 16) ? p[0] : p[1];
    }
    default: {
      const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (lane & 32) ? p[0] : p[1];
    }
  }
}

__device__ __forceinline__ uint64_t xor_lane64(uint64_t v, int j) {
  return ((uint64_t)xor_lane((uint32_t)(v >> 32), j) << 32) | xor_lane((uint32_t)v, j);
}

// Inclusive sums over the 64 lanes of a wave by DPP: within each 16-lane row by shifts of 1,
// 2, 4 and 8 lanes (zero from outside the row), then the totals of the other rows, read from
// their end lanes.  wave_prefix gives lane l the sum over lanes 0..l, wave_suffix over l..63.
__device__ __forceinline__ int wave_prefix(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

__device__ __forceinline__ int wave_suffix(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x101, 0xF, 0xF, true);  // row_shl:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x102, 0xF, 0xF, true);  // row_shl:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, true);  // row_shl:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x108, 0xF, 0xF, true);  // row_shl:8
  const int r1 = __builtin_amdgcn_readlane(x, 16), r2 = __builtin_amdgcn_readlane(x, 32),
            r3 = __builtin_amdgcn_readlane(x, 48);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row < 1 ? r1 : 0) + (row < 2 ? r2 : 0) + (row < 3 ? r3 : 0);
}

// The row's keys into registers (padding u = 0).  No load sits behind a branch, so the
// compiler keeps several in flight (a per-group branch had it wait for each load in turn).
// Group g of thread tid holds keys 4 (g NT + tid) + e, e < 4.  Each group's loads go through a
// buffer resource that starts at the group's first key and ends at key n, so keys past n read
// as 0 without touching memory: no address clamp, and a thread's offset is the same in every
// group.  kVec: rows 16-byte aligned with a length that is a multiple of 4, the resource's end
// rounded up to a whole 16-byte group (inside the row), one 16-byte load per group; otherwise
// one load per key.  Keys past n are masked to 0, only in the groups that reach past n.
template <int NT, int KPT, bool kVec>
__device__ __forceinline__ void load_keys(const float* row, int n, uint32_t (&u)[KPT]) {
  const int tid = threadIdx.x;
  const int nr = kVec ? (n + 3) & ~3 : n;  // keys the resources cover
  // every load first, into the key registers themselves, so that all of them are in flight
  // together; the scheduling fence keeps the compiler from mapping (and so waiting for) the
  // first groups while later loads are still to be issued
#pragma unroll
  for (int g = 0; g < KPT / 4; ++g) {
    const int left = 4 * (nr - g * NT * 4);  // bytes from the group's first key to the end
    // data format 32 bits (the field must be non-zero for untyped accesses)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(row) + g * NT * 4, 0, left > 0 ? left : 0, 0x00020000);
    if constexpr (kVec) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * tid, 0, 2));  // non-temporal
      u[4 * g + 0] = v.x;
      u[4 * g + 1] = v.y;
      u[4 * g + 2] = v.z;
      u[4 * g + 3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        u[4 * g + e] = __builtin_amdgcn_raw_buffer_load_b32(rs, 16 * tid + 4 * e, 0, 2);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int g = 0; g < KPT / 4; ++g) {
    if (n >= (g + 1) * NT * 4) {  // uniform: every thread's group lies inside the row
#pragma unroll
      for (int e = 0; e < 4; ++e) u[4 * g + e] = orderable_bits(u[4 * g + e]);
    } else {
      const int lim = n - (g * NT + tid) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) u[4 * g + e] = lim > e ? orderable_bits(u[4 * g + e]) : 0u;
    }
  }
}

// Exclusive prefix over the block in thread order of a packed pair of small counts
// (low 16 bits, high 16 bits; block totals stay below 65536); *total = block sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* slot, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int incl = wave_prefix(v);
  if (lane == 63) slot[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int s = slot[w];
    before += w < wave ? s : 0;
    all += s;
  }
  *total = all;
  return before + incl - v;
}

// Empty asm that "modifies" each register key: keeps the compiler from holding one lane mask
// per key between the two loops of compact() (64 SGPR pairs at 64 keys per thread) instead of
// evaluating the predicate again.
template <int KPT>
__device__ __forceinline__ void launder(uint32_t (&u)[KPT]) {
#pragma unroll
  for (int r = 0; r < KPT; ++r) asm volatile("" : "+v"(u[r]));
}

// Block-wide compaction in an unspecified order: every item k < ITEMS of the thread for which
// pred(k) holds is passed to store(pos, k) with distinct pos in [0, total); returns the total.
// refresh() runs between the counting and the storing loop.
template <int NT, int ITEMS, class Pred, class Store, class Refresh>
__device__ __forceinline__ int compact(Pred pred, Store store, Refresh refresh, RegShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int cnt = 0;
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    cnt += __popcll(__ballot(pred(k)));
    // keeps the scheduler from issuing every comparison first and holding all the lane masks
    // (two scalar registers per item, spilled to vector lanes at 72 items)
    if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);
  }
  if (lane == 0) sh.wcnt[0][wave] = cnt;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int c = sh.wcnt[0][w];
    base += w < wave ? c : 0;
    total += c;
  }
  // wave-uniform: kept in a scalar register, so the running base costs no vector work per key
  base = __builtin_amdgcn_readfirstlane(base);
  refresh();
#pragma unroll
  for (int k = 0; k < ITEMS; ++k) {
    const bool p = pred(k);
    const uint64_t m = __ballot(p);
    if (p) store(base + lanes_below(m), k);
    base += __popcll(m);
  }
  __syncthreads();
  return total;
}

// The register keys >= T, with their ids, into candU/candId[0, sh.ncand) in an unspecified
// order (every later use of the candidates is independent of it); sh.ncand must be 0 before.
// More than kCandCap such keys are counted in sh.ncand but not all stored.
// Each thread counts its keys >= T, a wave prefix of the counts gives every thread its first
// slot in the wave's run, one LDS atomic (by lane 0, on the wave's total) reserves the run, and
// each thread then stores its keys one after another: per key one comparison, and a store only
// where some lane of the wave stores.  Ends with a barrier.
template <int NT, int KPT>
__device__ __forceinline__ void compact_keys(const uint32_t (&u)[KPT], uint32_t T,
                                             RegShared& sh) {
  // 4 * tid through an empty asm: each key's id is then one add of a constant
  int ft4 = fresh_tid() << 2;
  asm volatile("" : "+v"(ft4));
  // a zero the compiler cannot see: the counter's address then looks lane-dependent, so the
  // one-lane atomic is not rewritten into a wave reduction
  int zero = 0;
  asm volatile("" : "+v"(zero));
  int c = 0;
#pragma unroll
  for (int r = 0; r < KPT; ++r) c += u[r] >= T ? 1 : 0;
  const int incl = wave_prefix(c);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  if (total != 0) {  // wave-uniform
    int base = 0;
    if ((threadIdx.x & 63) == 0) base = atomicAdd(&sh.ncand + zero, total);
    base = __builtin_amdgcn_readfirstlane(base);
    if (base + total <= kCandCap) {  // else over capacity (an estimated T): counted only
      int pos = base + incl - c;
#pragma unroll
      for (int r = 0; r < KPT; ++r) {
        if (u[r] >= T) {
          sh.candU[pos] = u[r];
          sh.candId[pos] = ft4 + ((r >> 2) * NT * 4 + (r & 3));  // key_id<NT>(r, tid)
          ++pos;
        }
      }
    }
  }
  __syncthreads();
}

// Every wave finds, on its own, the bin of a 256-bin histogram holding the kRem-th largest key
// (counting from bin 255 down), the number of keys in bins above it and in it (wave-uniform
// results; no barrier).  Lane l reads bins 4l..4l+3.  kRem <= the histogram's total.
struct BinPick {
  int bin, above, inBin;
};
__device__ __forceinline__ BinPick find_bin(const int* hist, int kRem) {
  const int l = threadIdx.x & 63;
  const int4 h = reinterpret_cast<const int4*>(hist)[l];
  const int s3 = h.w, s2 = h.z + s3, s1 = h.y + s2, s0 = h.x + s1;
  const int incl = wave_suffix(s0);  // keys in bins >= 4l
  const int ex = incl - s0;          // keys in bins >= 4l + 4
  const int src = __builtin_ctzll(__ballot(ex < kRem && kRem <= incl));
  // within the lane: the highest bin 4l+q whose keys in bins >= 4l+q reach kRem
  const int q = ex + s3 >= kRem ? 3 : ex + s2 >= kRem ? 2 : ex + s1 >= kRem ? 1 : 0;
  const int above = q == 3 ? ex : q == 2 ? ex + s3 : q == 1 ? ex + s2 : ex + s1;
  const int inBin = q == 3 ? h.w : q == 2 ? h.z : q == 1 ? h.y : h.x;
  return BinPick{4 * src + __builtin_amdgcn_readlane(q, src),
                 __builtin_amdgcn_readlane(above, src), __builtin_amdgcn_readlane(inBin, src)};
}

// Radix window [wlo, wlo + wm1] holding the kRem-th largest of the keys it covers.
struct RadixWindow {
  uint32_t wlo, wm1;
  int kRem;
  int inBin;  // after a pass: keys in the chosen bin
  int shift;  // after a pass: the shift it used (0: the window is now a single key value)
};

// One radix pass: histogram of the window's keys (registers, or the nc LDS candidates) over
// 256 bins at a shift that spreads the window over them, then narrow the window to the bin
// holding the kRem-th largest.  Pass p histograms into buffer p % 3, which was cleared before
// the barrier that precedes the pass, and clears buffer (p + 1) % 3 for the next pass: every
// wave last read that buffer in pass p - 2, before the barrier of pass p - 1.  One barrier.
template <int NT, int KPT, bool kLds>
__device__ __forceinline__ void radix_pass(const uint32_t (&u)[KPT], int nc, RadixWindow& w,
                                           RegShared& sh, int p) {
  const int tid = threadIdx.x;
  const int bits = w.wm1 ? 32 - __clz(w.wm1) : 0;
  const int shift = bits > 8 ? bits - 8 : 0;
  const uint32_t wlo = w.wlo, wm1 = w.wm1;
  int* hist = sh.hist[p % 3];
  if constexpr (kLds) {
    for (int c = tid; c < nc; c += NT) {
      const uint32_t d = sh.candU[c] - wlo;
      if (d <= wm1) atomicAdd(&hist[d >> shift], 1);
    }
  } else {
    int one = 1;  // the increment in a register the compiler cannot re-create for every key
    asm volatile("" : "+v"(one));
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const uint32_t d = u[r] - wlo;
      if (d <= wm1) atomicAdd(&hist[d >> shift], one);
    }
  }
  int* next = sh.hist[(p + 1) % 3];
  for (int j = tid; j < 256; j += NT) next[j] = 0;
  __syncthreads();  // the histogram is complete
  const BinPick pick = find_bin(hist, w.kRem);
  w.inBin = pick.inBin;
  w.kRem -= pick.above;
  const uint32_t off = (uint32_t)pick.bin << shift;
  w.wlo = wlo + off;
  const uint32_t binM1 = (1u << shift) - 1u, restM1 = wm1 - off;
  w.wm1 = binM1 < restM1 ? binM1 : restM1;
  w.shift = shift;
}

struct Threshold {
  uint32_t T;   // the kSel-th largest key (kCands: a lower bound, see select_threshold)
  int need;     // keys equal to T that are selected (the smallest ids among them); -1: kCands
  int ties;     // keys equal to T
  int nc;       // keys in LDS candidates (candU/candId), -1 when the passes ran on registers
  uint32_t hi;  // the row's largest key
};

// Exact radix select of the kSel-th largest key of the (padded) row held in registers, kSel <= n.
// kCands: when the keys at or above the first pass's bin, kSel to 2 kTopK of them, are what the
// compaction placed in LDS, stop there: T is then that bin's lower bound, every key >= T is
// among candU/candId[0, nc) and the kSel largest of them are the selection (need = -1).
template <int NT, int KPT, bool kCands = false>
__device__ __forceinline__ Threshold select_threshold(uint32_t (&u)[KPT], int n, int kSel,
                                                     RegShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // window [lo, hi]: at least kSel keys are >= lo.  lo is the smallest of the maxima of 512
  // disjoint sets of keys each holding a real key, so each set has a distinct real key at or
  // above it (padding keys are 0, below or equal to any real key).  The fewer the sets, the
  // larger they are and the higher lo: 512 threads each form one set, every thread holding a
  // real key from n = 4 * NT on; 256 threads split each thread's register groups into even
  // and odd, both holding real keys from n = 8 * NT on.  Below that, lo is the smallest real
  // key.
  uint32_t mA = 0u, mB = 0u;
#pragma unroll
  for (int r = 0; r < KPT; ++r) {
    if ((r >> 2) & 1) mB = u[r] > mB ? u[r] : mB;
    else mA = u[r] > mA ? u[r] : mA;
  }
  uint32_t tmax = mA > mB ? mA : mB;
  uint32_t tmin = mA < mB ? mA : mB;
  static_assert(NT == 512 || NT == 256, "512 sets: threads of 512 or halves of 256");
  if constexpr (NT == 512) tmin = tmax;  // the thread's maximum
  if (n < (NT == 512 ? 4 : 8) * NT) {
    tmin = 0xFFFFFFFFu;
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      if (key_id<NT>(r, tid) < n) tmin = u[r] < tmin ? u[r] : tmin;
  }
  // wave maximum and minimum by DPP and permlane swaps (written out: xor_lane needs constant
  // strides)
  auto step = [&](int o) {
    const uint32_t a = xor_lane(tmax, o), b = xor_lane(tmin, o);
    tmax = a > tmax ? a : tmax;
    tmin = b < tmin ? b : tmin;
  };
  step(32);
  step(16);
  step(8);
  step(4);
  step(2);
  step(1);
  if (lane == 0) {
    sh.red[0][wave] = tmax;
    sh.red[1][wave] = tmin;
  }
  for (int j = tid; j < 256; j += NT) sh.hist[0][j] = 0;  // the first pass's histogram
  if (tid == 0) sh.ncand = 0;
  __syncthreads();
  uint32_t hi = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    hi = sh.red[0][w] > hi ? sh.red[0][w] : hi;
    lo = sh.red[1][w] < lo ? sh.red[1][w] : lo;
  }
  RadixWindow w{lo, hi - lo, kSel, 0, 0};
  radix_pass<NT, KPT, false>(u, 0, w, sh, 0);
  if (w.shift == 0) return Threshold{w.wlo, w.kRem, w.inBin, -1, hi};
  // keep the keys >= wlo in LDS (those above the new window are selected for certain).  Kept
  // out of the pass loop below, so that no per-key value of it is hoisted into registers that
  // stay live across the passes.
  int nc = -1;
  const int nCand = (kSel - w.kRem) + w.inBin;  // the keys >= wlo
  if (nCand <= kCandCap) {
    compact_keys<NT, KPT>(u, w.wlo, sh);
    nc = nCand;
    if (kCands && nc <= 2 * kTopK) return Threshold{w.wlo, -1, 0, nc, hi};
  }
  for (int pass = 1; pass < 5; ++pass) {
    if (nc >= 0) radix_pass<NT, KPT, true>(u, nc, w, sh, pass);
    else radix_pass<NT, KPT, false>(u, 0, w, sh, pass);
    if (w.shift == 0) return Threshold{w.wlo, w.kRem, w.inBin, nc, hi};
  }
  return Threshold{w.wlo, w.kRem, 0, nc, hi};  // not reached: the shift reaches 0 within 4 passes
}

// The selected keys in ascending id (registers): above T, then the first `need` keys equal to
// T (padding keys have the largest ids and are never among them).  sh.selId[pos] receives
// value(id, r) of the key of rank pos in ascending id (register index r), pos < kTopK.
// Ids run group-major (register group g = r / 4 holds ids [4 NT g, 4 NT (g + 1))), then by
// thread, then by the key's place in its group.  One barrier: each wave first publishes its
// count of keys above T and equal to T per group; the counts before a key are then the sums
// over earlier (group, wave) pairs, over lower lanes of its wave (ballots), and over its own
// earlier keys of the group.  No branch per key: a key not selected writes to a slot of its
// lane past kTopK.
template <int NT, int KPT, class Value>
__device__ __forceinline__ void ordered_select(const uint32_t (&u)[KPT], uint32_t T, int need,
                                               RegShared& sh, Value value) {
  constexpr int G = KPT / 4, W = NT / 64;
  static_assert(G * W <= 128 && W % 2 == 0, "the count table holds 128 entries, 2 per lane");
  const int tid = fresh_tid(), lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  // counts of a group's keys above T (low 16 bits) and equal to T (high 16 bits) over the
  // wave; block totals stay below 65536
#pragma unroll
  for (int g = 0; g < G; ++g) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c += __popcll(__ballot(u[4 * g + e] > T));
      c += __popcll(__ballot(u[4 * g + e] == T)) << 16;
    }
    if (lane == 0) sh.gcnt[g * W + wave] = c;
  }
  __syncthreads();
  // exclusive prefix over the table in (group, wave) order: lane l holds entries 2l, 2l + 1
  const int2 pr = lane < (G * W) / 2 ? reinterpret_cast<const int2*>(sh.gcnt)[lane]
                                     : make_int2(0, 0);
  const int pair = pr.x + pr.y;
  const int exPair = wave_prefix(pair) - pair;
  // T through an empty asm: the comparisons are made again per group rather than the first
  // loop's lane masks held across the barrier (two SGPR pairs per key)
  uint32_t T2 = T;
  asm volatile("" : "+v"(T2));
  const int dummy = kTopK + lane;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    // entry g * W + wave sits in lane (g * W + wave) / 2, as its second half for odd waves
    const int src = (g * W + wave) >> 1;
    int base = __builtin_amdgcn_readlane(exPair, src);
    if (wave & 1) base += __builtin_amdgcn_readlane(pr.x, src);
    bool ab[4], ti[4];
    int a = base & 0xFFFF, t = base >> 16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ab[e] = u[4 * g + e] > T2;
      ti[e] = u[4 * g + e] == T2;
      a += lanes_below(__ballot(ab[e]));
      t += lanes_below(__ballot(ti[e]));
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * g + e;
      const int pos = a + (ab[e] ? (t < need ? t : need) : t);
      const bool sel = (ab[e] || (ti[e] && t < need)) && pos < kTopK;
      sh.selId[sel ? pos : dummy] = value(key_id<NT>(r, tid), r);
      a += ab[e] ? 1 : 0;
      t += ti[e] ? 1 : 0;
    }
  }
  __syncthreads();
}

// The same selection, emitted from the LDS candidates when select_threshold kept them (every
// key >= T is then among candU/candId[0, nc)): the selected ids are marked in two bitmaps over
// [0, n) (keys above T, keys equal to T) and each thread ranks the ids of its own 64-id
// stretch from the counts of the stretches below it (one block scan).  sh.selId[pos] =
// value(id).  The bitmaps live in sh.sortBuf: clear_select_bits must have cleared them
// before the select.  NT * 64 >= n.
constexpr int kBitWords = 1024;  // bitmap words: ids below 32768
// From 32 keys per thread on the bitmap emission is the faster one (rows of 16384 / 32768
// blocks: 9.6 / 13.0 us per 64 sequences against 11.7 / 18.7; 262144-block rows split into
// 32768-key chunks: 33.6 against 43.4); with 16 keys per thread or fewer the register form
// is (16: 11.6 against 15.9 us on the 64-sequence decode batch).
constexpr int kBitsMinKeys = 32;
template <int NT>
__device__ __forceinline__ void clear_select_bits(int n, RegShared& sh) {
  static_assert(sizeof(sh.sortBuf) >= 2 * kBitWords * 4, "two bitmaps fit sortBuf");
  uint32_t* bits = reinterpret_cast<uint32_t*>(sh.sortBuf);
  const int words = 2 * ((n + 63) / 64);
  for (int q = threadIdx.x; q < words; q += NT) {
    bits[q] = 0u;
    bits[kBitWords + q] = 0u;
  }
}

template <int NT, class Value>
__device__ __forceinline__ void ordered_select_bits(int n, int nc, uint32_t T, int need,
                                                    RegShared& sh, Value value) {
  static_assert(NT * 64 >= 32 * kBitWords, "a 64-id stretch per thread covers the bitmaps");
  uint32_t* bitsA = reinterpret_cast<uint32_t*>(sh.sortBuf);
  uint32_t* bitsT = bitsA + kBitWords;
  const int tid = threadIdx.x;
  for (int q = tid; q < nc; q += NT) {
    const uint32_t uq = sh.candU[q];
    if (uq >= T) {
      const int id = sh.candId[q];
      atomicOr(uq > T ? &bitsA[id >> 5] : &bitsT[id >> 5], 1u << (id & 31));
    }
  }
  __syncthreads();
  uint64_t am = 0ull, tm = 0ull;
  if (64 * tid < n) {
    am = (uint64_t)bitsA[2 * tid] | ((uint64_t)bitsA[2 * tid + 1] << 32);
    tm = (uint64_t)bitsT[2 * tid] | ((uint64_t)bitsT[2 * tid + 1] << 32);
  }
  int total;
  const int ex = block_excl_scan<NT>(__popcll(am) | (__popcll(tm) << 16), sh.wcnt[0], &total);
  int aRun = ex & 0xFFFF, tRun = ex >> 16;  // keys above T / equal to T with smaller ids
  for (uint64_t m = am | tm; m != 0ull; m &= m - 1ull) {
    const int bit = __builtin_ctzll(m);
    const int id = 64 * tid + bit;
    if ((am >> bit) & 1ull) {
      const int pos = aRun + (tRun < need ? tRun : need);
      if (pos < kTopK) sh.selId[pos] = value(id);
      ++aRun;
    } else {
      if (tRun < need) sh.selId[aRun + tRun] = value(id);
      ++tRun;
    }
  }
  __syncthreads();
}

// ordered_select over the row in memory rather than registers: the same selection in
// ascending id, 1024 keys per step (4 consecutive ids per thread).  Used by prefill only for
// rows with many keys equal to T, where the cached row is read again.
template <class Emit>
__device__ __forceinline__ void ordered_select_row(const float* row, int n, uint32_t T, int need,
                                                   RegShared& sh, Emit emit) {
  const int tid = threadIdx.x;
  int aboveRun = 0, tieRun = 0;
  for (int base = 0, step = 0; base < n; base += 4 * kRT, ++step) {
    bool ab[4], ti[4];
    uint32_t uk[4];
    int packed = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int id = base + 4 * tid + e;
      uk[e] = id < n ? orderable(row[id]) : 0u;
      ab[e] = id < n && uk[e] > T;
      ti[e] = id < n && uk[e] == T;
      packed += (ab[e] ? 1 : 0) + (ti[e] ? 0x10000 : 0);
    }
    int tot;
    const int ex = block_excl_scan<kRT>(packed, sh.wcnt[step & 1], &tot);
    int a = aboveRun + (ex & 0xFFFF), t = tieRun + (ex >> 16);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int id = base + 4 * tid + e;
      if (ab[e]) {
        emit(a + (t < need ? t : need), id, uk[e]);
        ++a;
      } else if (ti[e]) {
        if (t < need) emit(a + t, id, uk[e]);
        ++t;
      }
    }
    aboveRun += tot & 0xFFFF;
    tieRun += tot >> 16;
  }
  __syncthreads();
}


// Bitonic sort, descending, of kRT * E 64-bit values; thread t holds elements e * kRT + t.
// The stages with strides 64 and 128 go through LDS, alternating between buf0 and buf1: a
// stage writes one buffer while others may still read the other, and the barrier of the next
// stage orders every read of a buffer before it is written again.
template <int E>
__device__ __forceinline__ void sort_desc(uint64_t (&v)[E], uint64_t* buf0, uint64_t* buf1) {
  const int tid = threadIdx.x;
  constexpr int P = kRT * E;
  int ldsStage = 0;
#pragma unroll
  for (int k = 2; k <= P; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= kRT) {
        const int je = j / kRT;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e & je) continue;
          const bool desc = ((e * kRT + tid) & k) == 0;
          const uint64_t x = v[e], y = v[e | je];
          const bool sw = desc ? x < y : x > y;
          v[e] = sw ? y : x;
          v[e | je] = sw ? x : y;
        }
      } else {
        uint64_t* buf = (ldsStage & 1) ? buf1 : buf0;
        if (j >= 64) {
#pragma unroll
          for (int e = 0; e < E; ++e) buf[e * kRT + tid] = v[e];
          __syncthreads();
          ++ldsStage;
        }
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int x = e * kRT + tid;
          const uint64_t w = j >= 64 ? buf[x ^ j] : xor_lane64(v[e], j);
          const bool keepMax = ((x & k) == 0) == ((x & j) == 0);
          const bool wBig = w > v[e];
          v[e] = (keepMax == wBig) ? w : v[e];
        }
      }
    }
  }
}

// Sort the m composites of sh.sortBuf[0, m) and leave the ids of the first kSel in sh.selId.
template <int E>
__device__ __forceinline__ void sort_selected(int m, int kSel, RegShared& sh) {
  const int tid = threadIdx.x;
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = e * kRT + tid < m ? sh.sortBuf[e * kRT + tid] : 0ull;
  __syncthreads();
  // the candidates are consumed by now: their 16 KB hold the second sort buffer
  sort_desc<E>(v, sh.sortBuf, reinterpret_cast<uint64_t*>(sh.candU));
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (e * kRT + tid < kSel) sh.selId[e * kRT + tid] = (int32_t)~(uint32_t)v[e];
  __syncthreads();
}

// Ordering of the m selected composites (keys >= T; hi their largest key, or an estimate of it:
// keys above it share the top bucket) by bucket ranks, where the buckets
// are small: the key range [T, hi] is cut into kRankBins buckets by its top bits (a bucket's
// composites all exceed those of every lower bucket), the buckets are counted and laid out in
// descending order by one block scan, each composite is placed in its bucket, and its rank
// inside the bucket is the number of the bucket's composites greater than it.  The composites
// are distinct (ids differ), so the ranks are too, and the result is the order of the
// descending sort.  A bucket of more than kRankMaxBin composites (many keys in a narrow range,
// e.g. ties) makes the whole row take the bitonic sort of the placed composites instead; the
// decision is the same for every thread of the row.
// load(k, &v) gives thread tid its k-th item (k < KC) and whether it is one of the m; placed
// (2 * kTopK entries) receives the composites in bucket order and must not alias the items'
// source; the bitonic fallback then sorts placed[0, m) with sortBuf / candU as its buffers,
// so placed is sortBuf, or the items are in sortBuf already and placed is any other buffer.
// sh.rankBins and sh.rankBig must be zero before the barrier that precedes the call
// (clear_rank_bins).  Leaves the ids of the first kSel in sh.selId; ends with a barrier.
constexpr int kRankBins = 1024;
constexpr int kRankMaxBin = 32;
__device__ __forceinline__ void clear_rank_bins(RegShared& sh) {
  static_assert(kRankBins == 4 * kRT, "four buckets per thread");
  reinterpret_cast<uint4*>(sh.rankBins)[threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) sh.rankBig = 0;
}

template <int KC, class Load>
__device__ __forceinline__ void rank_sort(int m, int kSel, uint32_t T, uint32_t hi,
                                          uint64_t* placed, RegShared& sh, Load load) {
  const int tid = threadIdx.x;
  uint32_t* bins = sh.rankBins;  // per bucket in descending key order: count | start << 16
  const uint32_t range = hi - T;
  const int rbits = range ? 32 - __clz(range) : 0;
  const int shift = rbits > 10 ? rbits - 10 : 0;  // (hi - T) >> shift < kRankBins
  uint64_t v[KC];
  int bin[KC], slot[KC];
  bool ok[KC];
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    ok[k] = load(k, v[k]);
    // keys above hi (an estimated hi) join the top bucket, which keeps the buckets in order
    const uint32_t dq = ((uint32_t)(v[k] >> 32) - T) >> shift;
    bin[k] = dq < (uint32_t)kRankBins ? (kRankBins - 1) - (int)dq : 0;
    slot[k] = ok[k] ? (int)atomicAdd(&bins[bin[k]], 1u) : 0;
  }
  __syncthreads();
  {
    // every wave scans all the buckets (lane l: buckets 16l..16l+15), so no barrier is needed
    // between the scan and the starts; wave w writes the starts of buckets 16l+4w..16l+4w+3
    static_assert(kRT == 256 && kRankBins == 1024, "4 waves, 16 buckets per lane");
    const int l = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint4* b4 = reinterpret_cast<const uint4*>(bins) + 4 * l;
    const uint4 g0 = b4[0], g1 = b4[1], g2 = b4[2], g3 = b4[3];
    const uint32_t t0 = g0.x + g0.y + g0.z + g0.w, t1 = g1.x + g1.y + g1.z + g1.w,
                   t2 = g2.x + g2.y + g2.z + g2.w, t3 = g3.x + g3.y + g3.z + g3.w;
    const uint32_t seg = t0 + t1 + t2 + t3;
    uint32_t ex = (uint32_t)wave_prefix((int)seg) - seg;  // buckets before 16l
    const uint4 c4 = w == 0 ? g0 : w == 1 ? g1 : w == 2 ? g2 : g3;
    ex += (w > 0 ? t0 : 0u) + (w > 1 ? t1 : 0u) + (w > 2 ? t2 : 0u);
    if (max(max(c4.x, c4.y), max(c4.z, c4.w)) > (uint32_t)kRankMaxBin) sh.rankBig = 1;
    const uint32_t s1 = c4.x, s2 = s1 + c4.y, s3 = s2 + c4.z;
    reinterpret_cast<uint4*>(bins)[4 * l + w] =
        make_uint4(c4.x | ex << 16, c4.y | (ex + s1) << 16, c4.z | (ex + s2) << 16,
                   c4.w | (ex + s3) << 16);
  }
  __syncthreads();
  uint32_t bc[KC];  // read before the barrier below: selId overlays the buckets after it
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    bc[k] = ok[k] ? bins[bin[k]] : 0u;
    if (ok[k]) placed[(bc[k] >> 16) + slot[k]] = v[k];
  }
  __syncthreads();
  if (sh.rankBig) {  // uniform: a bucket too large for the in-bucket ranks
    if (m <= kTopK) sort_selected<kTopK / kRT>(m, kSel, sh);
    else sort_selected<2 * kTopK / kRT>(m, kSel, sh);
    return;
  }
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    if (ok[k]) {
      const int b0 = (int)(bc[k] >> 16), c = (int)(bc[k] & 0xFFFFu);
      int r = 0;
      for (int j = 0; j < c; ++j) r += placed[b0 + j] > v[k] ? 1 : 0;
      if (b0 + r < kSel) sh.selId[b0 + r] = (int32_t)~(uint32_t)v[k];
    }
  }
  __syncthreads();
}

// The candidates of a prefill row held in registers from an estimated threshold instead of a
// radix pass over all its keys: a sample of the first key of every other register group (256 x
// ceil(KPT / 8) keys spread over the row) gives, by one radix pass over the sample within the
// window [smallest thread maximum, largest key], the bin of its k-th largest key, k about 1.25
// times its expected share of the kSel largest plus 10; every key of the row at or above that
// bin's base T is compacted.  When they number kSel to 2 kTopK, they are the candidates of
// select_threshold's kCands form (need = -1, hi the sample's largest key: keys above it join
// the top rank bucket); otherwise need = -2 and the caller runs the exact select.  Three
// barriers, like the first pass of the exact select; n >= 8 NT (every thread's first two
// groups are real keys, so each thread's sample maximum is a distinct real key).  Rows short
// for the kernel (k above NT / 2) return need = -2 at once.
template <int NT, int KPT>
__device__ __forceinline__ Threshold estimate_candidates(const uint32_t (&u)[KPT], int n, int kSel,
                                                        RegShared& sh) {
  constexpr int NS = (KPT / 4 + 1) / 2;  // sample keys per thread: groups 0, 2, 4, ...
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // at least NT sample keys are >= lo (the threads' maxima, below); too large a k for that
  // (rows short for the kernel's registers) takes the exact select
  const int kS = (int)((int64_t)kSel * (5 * NT * NS) / (4 * (int64_t)n)) + 10;
  if (kS > NT / 2) return Threshold{0u, -2, 0, -1, 0u};
  uint32_t tmax = 0u;
#pragma unroll
  for (int j = 0; j < NS; ++j) tmax = u[8 * j] > tmax ? u[8 * j] : tmax;
  uint32_t wmax = tmax, wmin = tmax;
  auto step = [&](int o) {
    const uint32_t a = xor_lane(wmax, o), b = xor_lane(wmin, o);
    wmax = a > wmax ? a : wmax;
    wmin = b < wmin ? b : wmin;
  };
  step(32);
  step(16);
  step(8);
  step(4);
  step(2);
  step(1);
  if (lane == 0) {
    sh.red[0][wave] = wmax;
    sh.red[1][wave] = wmin;
  }
  for (int j = tid; j < 256; j += NT) sh.hist[0][j] = 0;
  if (tid == 0) sh.ncand = 0;
  __syncthreads();
  uint32_t hi = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    hi = sh.red[0][w] > hi ? sh.red[0][w] : hi;
    lo = sh.red[1][w] < lo ? sh.red[1][w] : lo;
  }
  const uint32_t wm1 = hi - lo;
  const int bits = wm1 ? 32 - __clz(wm1) : 0;
  const int shift = bits > 8 ? bits - 8 : 0;
  int one = 1;
  asm volatile("" : "+v"(one));
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const uint32_t d = u[8 * j] - lo;
    if (d <= wm1) atomicAdd(&sh.hist[0][d >> shift], one);
  }
  __syncthreads();
  const BinPick pick = find_bin(sh.hist[0], kS);
  const uint32_t T = lo + ((uint32_t)pick.bin << shift);
  compact_keys<NT, KPT>(u, T, sh);
  const int nc = sh.ncand;
  if (nc >= kSel && nc <= 2 * kTopK) return Threshold{T, -1, 0, nc, hi};
  return Threshold{T, -2, 0, -1, hi};
}

// Waves per SIMD the register allocation aims for at KPT keys per thread (512 VGPRs per SIMD
// lane shared by the waves): at most 80 keys leave room for 4 rows of 4 waves on a CU.
constexpr int reg_waves(int kpt) { return kpt <= 24 ? 5 : kpt <= 80 ? 4 : kpt <= 96 ? 3 : 2; }

template <int KPT, bool kVec>
__global__ __launch_bounds__(kRT) __attribute__((amdgpu_waves_per_eu(reg_waves(KPT))))
void topk_expand_reg_kernel(TopkArgs a) {
  __shared__ RegShared sh;
  const int tid = threadIdx.x;
  const int64_t i = blockIdx.x, r = a.rowStart + i, b = r / a.S, t = r % a.S;
  int32_t* out = a.outIdx + r * kIndexWidth;
  const int64_t c = a.ctx[b];
  if (c <= 0 || t >= c) {
    for (int s = tid; s < kIndexWidth; s += kRT) out[s] = -1;
    return;
  }
  const int64_t nVisT = (t + 1) / 4;
  const int n = (int)(nVisT < a.numBlocks ? nVisT : a.numBlocks);  // <= kRT * KPT (host)
  const int kSel = n < kTopK ? n : kTopK;
  const float* row = a.logits + i * a.numBlocks;
  uint32_t u[KPT];
  if (n > 0) load_keys<kRT, KPT, kVec>(row, n, u);
  if (n <= kTopK) {
    // every key is taken; ids < n <= 512 all sit in register group 0
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int id = key_id<kRT>(q, tid);
      if (id < n) sh.sortBuf[id] = composite(u[q], id);
    }
    __syncthreads();
    sort_selected<kTopK / kRT>(n, kSel, sh);
  } else {
    clear_rank_bins(sh);  // ordered before rank_sort by the select's barriers
    Threshold th{0u, -2, 0, -1, 0u};
    if constexpr (KPT >= 16)
      if (n >= 8 * kRT) th = estimate_candidates<kRT, KPT>(u, n, kSel, sh);
    if (th.need == -2) th = select_threshold<kRT, KPT, true>(u, n, kSel, sh);
    const uint32_t T = th.T;
    const int m = (kSel - th.need) + th.ties;
    if (th.need < 0) {
      // the candidates are every key >= T, kSel to 2 kTopK of them: rank them all
      const int nc = th.nc;
      rank_sort<kCandCap / kRT>(nc, kSel, T, th.hi, sh.sortBuf, sh, [&](int k, uint64_t& v) {
        const int q = k * kRT + tid;
        v = composite(q < nc ? sh.candU[q] : 0u, q < nc ? sh.candId[q] : 0);
        return q < nc;
      });
    } else if (th.nc >= 0 && m <= 2 * kTopK) {
      // the keys >= T are all among the LDS candidates: rank them from there
      const int nc = th.nc;
      rank_sort<kCandCap / kRT>(m, kSel, T, th.hi, sh.sortBuf, sh, [&](int k, uint64_t& v) {
        const int q = k * kRT + tid;
        const uint32_t uq = q < nc ? sh.candU[q] : 0u;
        v = composite(uq, q < nc ? sh.candId[q] : 0);
        return q < nc && uq >= T;
      });
    } else {
      // many keys equal to T: the exact selection in ascending id, from the row in memory
      ordered_select_row(row, n, T, th.need, sh, [&](int pos, int id, uint32_t uu) {
        if (pos < kTopK) sh.sortBuf[pos] = composite(uu, id);
      });
      rank_sort<kTopK / kRT>(kSel, kSel, T, th.hi, reinterpret_cast<uint64_t*>(sh.candId), sh,
                             [&](int k, uint64_t& v) {
                               const int q = k * kRT + tid;
                               v = q < kSel ? sh.sortBuf[q] : 0ull;
                               return q < kSel;
                             });
    }
  }
  for (int s = tid; s < 4 * kSel; s += kRT) out[s] = sh.selId[s >> 2] * 4 + (s & 3);
  write_tail_and_pad(out, 4 * kSel, nVisT, (int)((t + 1) % 4), kRT);
}

template <int KPT, bool kVec>
__global__ __launch_bounds__(kDT) __attribute__((amdgpu_waves_per_eu(reg_waves(KPT))))
void topk_expand_decode_reg_kernel(TopkDecodeArgs a) {
  __shared__ RegShared sh;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  int32_t* out = a.outIdx + b * kIndexWidth;
  if (a.splitCounters != nullptr)
    for (int h = tid; h < a.numKVHeads; h += kDT) a.splitCounters[b * a.numKVHeads + h] = 0;
  const int64_t c = a.ctx[b];
  if (c <= 0) {
    for (int s = tid; s < kIndexWidth; s += kDT) out[s] = -1;
    return;
  }
  const int64_t nVisC = c / 4;
  const int n = (int)(nVisC < a.maxBlocks ? nVisC : a.maxBlocks);  // <= kDT * KPT (host)
  const int kSel = n < kTopK ? n : kTopK;
  if (n <= kTopK) {
    for (int s = tid; s < 4 * n; s += kDT) out[s] = s;  // block s/4, token s%4
  } else {
    const float* row = a.logits + b * a.maxBlocks;
    uint32_t u[KPT];
    load_keys<kDT, KPT, kVec>(row, n, u);
    if (KPT >= kBitsMinKeys) clear_select_bits<kDT>(n, sh);
    const Threshold th = select_threshold<kDT, KPT>(u, n, kSel, sh);
    // the selection gathers in LDS by rank and is written out in order, 4 tokens per block
    if (KPT >= kBitsMinKeys && th.nc >= 0)
      ordered_select_bits<kDT>(n, th.nc, th.T, th.need, sh, [](int id) { return id; });
    else
      ordered_select<kDT, KPT>(u, th.T, th.need, sh, [](int id, int) { return id; });
    for (int s = tid; s < 4 * kSel; s += kDT) out[s] = 4 * sh.selId[s >> 2] + (s & 3);
  }
  write_tail_and_pad(out, 4 * kSel, n, (int)(c % 4), kDT);
}

// ------------------------------------------------------------- decode, split rows ---
//
// Decode rows longer than one register-resident workgroup holds.  The row is cut into
// numChunks chunks of `chunk` keys (8192, 16384 or 32768; 5 to 8 of them), one
// workgroup per chunk.  The 512 largest keys of a chunk (u desc, id asc) include every key
// of the row's 512 largest that lies in it: any other key of the chunk has 512 keys of its
// own chunk ranking above it.  The chunk pass writes those keys' chunk-local ids (< 32768),
// in ascending order, as 16-bit values into the sequence's own output row (512 per chunk;
// the row's 8204 bytes hold the 4096 of 8 chunks); a chunk of at most 512 keys writes
// nothing, all its keys being candidates.  The merge pass, one workgroup per sequence, reads
// the candidates back (ascending id: chunk by chunk, each in ascending order), gathers their
// keys from the row and selects among them exactly as the register kernel selects over a
// row, into the same output row once every candidate is read.  Each key is read from HBM
// once; the merge gathers at most 4096 keys of a sequence again.

constexpr int kSplitMaxChunks = 8;
constexpr int kSplitMaxChunk = kDT * 64;  // 32768 keys: 64 per thread

template <int KPT, bool kVec>
__global__ __launch_bounds__(kDT) __attribute__((amdgpu_waves_per_eu(reg_waves(KPT))))
void topk_decode_chunk_kernel(TopkDecodeArgs a) {
  __shared__ RegShared sh;
  const int64_t b = blockIdx.x / a.numChunks;
  const int j = (int)(blockIdx.x % a.numChunks);
  const int64_t c = a.ctx[b];
  if (c <= 0) return;
  const int64_t nVisC = c / 4;
  const int n = (int)(nVisC < a.maxBlocks ? nVisC : a.maxBlocks);
  const int nj = min(n - j * a.chunk, a.chunk);  // keys of this chunk (<= 0: none)
  if (nj <= kTopK) return;                       // n <= 512 included
  const float* row = a.logits + b * a.maxBlocks + (int64_t)j * a.chunk;
  uint32_t u[KPT];
  load_keys<kDT, KPT, kVec>(row, nj, u);
  if (KPT >= kBitsMinKeys) clear_select_bits<kDT>(nj, sh);
  const Threshold th = select_threshold<kDT, KPT>(u, nj, kTopK, sh);
  if (KPT >= kBitsMinKeys && th.nc >= 0)
    ordered_select_bits<kDT>(nj, th.nc, th.T, th.need, sh, [](int id) { return id; });
  else
    ordered_select<kDT, KPT>(u, th.T, th.need, sh, [](int id, int) { return id; });
  // two ids a word: chunk j's 512 ids are bytes [1024 j, 1024 j + 1024) of the output row
  uint32_t* st = reinterpret_cast<uint32_t*>(a.outIdx + b * kIndexWidth) + j * (kTopK / 2);
  const int tid = threadIdx.x;
  if (tid < kTopK / 2)
    st[tid] = (uint32_t)sh.selId[2 * tid] | ((uint32_t)sh.selId[2 * tid + 1] << 16);
}

// 8 keys per thread: 4096 candidate slots, the 512 of each of up to 8 chunks (a split row has
// 5 to 8 chunks: the chunk is the smallest length that leaves at most 8).
__global__ __launch_bounds__(kDT) void topk_decode_merge_kernel(TopkDecodeArgs a) {
  constexpr int KPT = 8;
  __shared__ RegShared sh;
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  int32_t* out = a.outIdx + b * kIndexWidth;
  if (a.splitCounters != nullptr)
    for (int h = tid; h < a.numKVHeads; h += kDT) a.splitCounters[b * a.numKVHeads + h] = 0;
  const int64_t c = a.ctx[b];
  if (c <= 0) {
    for (int s = tid; s < kIndexWidth; s += kDT) out[s] = -1;
    return;
  }
  const int64_t nVisC = c / 4;
  const int n = (int)(nVisC < a.maxBlocks ? nVisC : a.maxBlocks);
  const int kSel = n < kTopK ? n : kTopK;
  if (n <= kTopK) {
    for (int s = tid; s < 4 * n; s += kDT) out[s] = s;  // block s/4, token s%4
  } else {
    const int P = (n + a.chunk - 1) / a.chunk;         // chunks holding keys (<= numChunks)
    const int last = n - (P - 1) * a.chunk;            // keys of the last of them
    const int nCand = (P - 1) * kTopK + min(last, kTopK);
    const float* row = a.logits + b * a.maxBlocks;
    const uint32_t* st = reinterpret_cast<const uint32_t*>(out);  // two 16-bit ids a word
    // slots s .. s + 3 of group g (slot = candidate index, in ascending id) lie in one chunk
    uint32_t u[KPT];
    int ids[KPT];
#pragma unroll
    for (int g = 0; g < KPT / 4; ++g) {
      const int s = (g * kDT + tid) * 4;
      const int j = s / kTopK, k = s % kTopK;
      const int nj = j < P - 1 ? a.chunk : last;
      const uint32_t w0 = st[s / 2], w1 = st[s / 2 + 1];  // s / 2 + 1 < 2048 <= 2051 words
      const int staged[4] = {(int)(w0 & 0xFFFFu), (int)(w0 >> 16), (int)(w1 & 0xFFFFu),
                             (int)(w1 >> 16)};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // a staged id is below nj by construction; the clamp keeps the gather inside the row
        const int local = nj > kTopK ? min(staged[e], nj - 1) : k + e;
        ids[4 * g + e] = s + e < nCand ? j * a.chunk + local : 0;
      }
    }
#pragma unroll
    for (int r = 0; r < KPT; ++r) u[r] = __float_as_uint(row[ids[r]]);
#pragma unroll
    for (int r = 0; r < KPT; ++r)
      u[r] = key_id<kDT>(r, tid) < nCand ? orderable_bits(u[r]) : 0u;
    // every staged id is read (the gathers use them): the row may be written from here on,
    // once the barriers of the select have passed
    const Threshold th = select_threshold<kDT, KPT>(u, nCand, kSel, sh);
    ordered_select<kDT, KPT>(u, th.T, th.need, sh, [&](int, int r) { return ids[r]; });
    for (int s = tid; s < 4 * kSel; s += kDT) out[s] = 4 * sh.selId[s >> 2] + (s & 3);
  }
  write_tail_and_pad(out, 4 * kSel, n, (int)(c % 4), kDT);
}

// -------------------------------------------------------------------- one wave per row ---
//
// Prefill rows longer than 18432 blocks.  Each wave of a workgroup takes a row of its own and
// walks it front to back, a step of keys at a time, against a running threshold thr: a
// wave-private LDS buffer holds candidates {u, id}; whenever the next step's keys above thr
// would not fit, the buffer is cut to its 512 largest (u desc, id asc) and at most kCap - 512
// - (one step) more, all of them at or above some value lo, and thr becomes lo.  Later keys have larger ids, so one of them can be
// among a prefix's 512 largest only if u > thr: equal u loses the tie.  The buffer therefore
// always holds the 512 largest keys seen so far; at the end it is cut to exactly those 512,
// which are sorted in registers.  No workgroup barrier: the waves of a workgroup share
// nothing, and several rows per CU overlap their loads with the others' selection.

constexpr int kWaveRows = 4;       // rows (waves) per workgroup of the one-wave-per-row kernel
// (candidate buffer entries, keys per lane per step): rows of up to 32768 blocks keep 16 rows
// per CU (36 KB of LDS per workgroup); longer ones a larger buffer and steps, so fewer cuts
constexpr int kWaveCapMid = 1024, kWaveKPLMid = 4;    // 256 keys per step
constexpr int kWaveCapLong = 1536, kWaveKPLLong = 8;  // 512 keys per step
constexpr int kWaveDepth = 2;  // steps of keys in registers: one filtered, the rest loading

template <int kCap>
struct WaveShared {
  uint32_t u[kCap];  // candidates: key
  uint32_t id[kCap]; //             block id
  int hist[256];
};

// Orders this wave's LDS accesses in program order (a wave's LDS instructions execute in
// issue order; the fence keeps the compiler from moving one across another).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int j = 1; j < 64; j <<= 1) {
    const uint32_t w = xor_lane(v, j);
    v = w > v ? w : v;
  }
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
#pragma unroll
  for (int j = 1; j < 64; j <<= 1) {
    const uint32_t w = xor_lane(v, j);
    v = w < v ? w : v;
  }
  return __builtin_amdgcn_readfirstlane(v);
}

// Radix select of the kRem-th largest of the wave's valid keys (SL per lane: key(i, c, valid)
// with c the entry count), inside the window [lo, lo + m1] that holds all of them: each pass
// histograms the window's keys over 256 bins (LDS atomics) at a shift that spreads the window
// over the bins, and narrows the window to the bin holding the kRem-th largest.  Stops once
// that bin holds at most `slack` keys more than are still to be taken, or is a single value.
// On return lo is the bin's base, kRem the number of its keys still to take (every key above
// the bin is taken) and inBin its count.
template <int SL, class Key>
__device__ __forceinline__ void wave_window_select(Key key, int cnt, int* hist, uint32_t& lo,
                                                   uint32_t m1, int& kRem, int& inBin,
                                                   int slack) {
  const int lane = threadIdx.x & 63;
#pragma unroll 1
  for (int pass = 0; pass < 5; ++pass) {
    // the entry count through an empty asm: the per-slot validity masks are evaluated again in
    // every pass rather than hoisted out of the loop and held (one SGPR pair per slot)
    int c = cnt;
    asm volatile("" : "+v"(c));
    const int bits = m1 ? 32 - __clz(m1) : 0;
    const int shift = bits > 8 ? bits - 8 : 0;
    *reinterpret_cast<int4*>(&hist[4 * lane]) = make_int4(0, 0, 0, 0);
    wave_sync();
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      bool valid;
      const uint32_t d = key(i, c, valid) - lo;
      if (valid && d <= m1) atomicAdd(&hist[d >> shift], 1);
    }
    wave_sync();
    // lane l holds bins 4l .. 4l + 3; suffix sums over the lanes from bin 255 down
    const int4 h = *reinterpret_cast<const int4*>(&hist[4 * lane]);
    const int s3 = h.w, s2 = h.z + s3, s1 = h.y + s2, s0 = h.x + s1;
    const int ex = wave_suffix(s0) - s0;  // keys in bins >= 4l + 4
    const int cum[4] = {ex + s0, ex + s1, ex + s2, ex + s3};
    const int hq[4] = {h.x, h.y, h.z, h.w};
    int myBin = 0, myAbove = 0, myIn = 0;
    bool hit = false;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (cum[q] >= kRem && cum[q] - hq[q] < kRem) {
        myBin = 4 * lane + q;
        myAbove = cum[q] - hq[q];
        myIn = hq[q];
        hit = true;
      }
    const uint64_t m = __ballot(hit);
    const int src = m ? (int)__builtin_ctzll(m) : 0;
    const int bin = __builtin_amdgcn_readlane(myBin, src);
    kRem -= __builtin_amdgcn_readlane(myAbove, src);
    inBin = __builtin_amdgcn_readlane(myIn, src);
    const uint32_t off = (uint32_t)bin << shift;
    lo += off;
    const uint32_t binM1 = (1u << shift) - 1u, restM1 = m1 - off;
    m1 = binM1 < restM1 ? binM1 : restM1;
    if (inBin - kRem <= slack || shift == 0) return;
  }
}

// Cut the wave's buffer (cnt > K entries) in place to its K largest (u desc, id asc), or, with
// slack > 0, to at most K + slack entries that include them: every entry at or above a value
// lo.  Sets cnt to the entries kept and returns the threshold that later keys, with larger
// ids, must exceed: the u of the K-th largest, or the lower value lo.
template <int kCap>
__device__ __forceinline__ uint32_t wave_keep_top(WaveShared<kCap>& sh, int& cnt, int K,
                                                  int slack) {
  constexpr int SL = kCap / 64;
  const int lane = threadIdx.x & 63;
  uint32_t u[SL];
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
  // each loop below takes the count through an empty asm of its own, so that no loop's
  // per-slot validity masks are held for a later one
  int c0 = cnt;
  asm volatile("" : "+v"(c0));
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    u[i] = sh.u[64 * i + lane];
    if (64 * i + lane < c0) {
      mx = u[i] > mx ? u[i] : mx;
      mn = u[i] < mn ? u[i] : mn;
    }
  }
  mx = wave_max(mx);
  mn = wave_min(mn);
  uint32_t T = mn;
  int kRem = K, inBin = 0;
  wave_window_select<SL>(
      [&](int i, int c, bool& valid) {
        valid = 64 * i + lane < c;
        return u[i];
      },
      cnt, sh.hist, T, mx - mn, kRem, inBin, slack);
  // keys >= T are kept when the bin fits the slack; otherwise the bin is the single value T
  // and of its inBin keys the kRem with the smallest ids are kept: a second select over ~id
  uint32_t nidMin = 0u;
  int kept = (K - kRem) + inBin;
  if (inBin - kRem > slack) {
    uint32_t a = 0u, z = 0xFFFFFFFFu;
    int c2 = cnt;
    asm volatile("" : "+v"(c2));
#pragma unroll
    for (int i = 0; i < SL; ++i) {
      if (64 * i + lane < c2 && u[i] == T) {
        const uint32_t nid = ~sh.id[64 * i + lane];
        a = nid > a ? nid : a;
        z = nid < z ? nid : z;
      }
    }
    a = wave_max(a);
    z = wave_min(z);
    nidMin = z;
    int kTie = kRem, inTie = 0;
    wave_window_select<SL>(
        [&](int i, int c, bool& valid) {
          valid = 64 * i + lane < c && u[i] == T;
          return ~sh.id[64 * i + lane];
        },
        cnt, sh.hist, nidMin, a - z, kTie, inTie, 0);
    kept = K;
  }
  int pos = 0;
  int c1 = cnt;
  asm volatile("" : "+v"(c1));
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const uint32_t eu = sh.u[64 * i + lane], eid = sh.id[64 * i + lane];
    const bool keep = 64 * i + lane < c1 && (eu > T || (eu == T && ~eid >= nidMin));
    const uint64_t m = __ballot(keep);
    // in place: the p-th kept entry moves to p <= its own index, and a slot is read before
    // any of its entries is written
    const int p = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, pos));
    if (keep) {
      sh.u[p] = eu;
      sh.id[p] = eid;
    }
    pos += __popcll(m);
  }
  wave_sync();
  cnt = kept;
  return T;
}

// Bitonic sort, descending, of 64 * E 64-bit values held by one wave; lane l holds elements
// e * 64 + l.  Strides below 64 by DPP moves and permlane swaps, larger ones within a lane.
template <int E>
__device__ __forceinline__ void sort_wave_desc(uint64_t (&v)[E]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64 * E; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 64) {
        const int je = j / 64;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (e & je) continue;
          const bool desc = ((e * 64) & k) == 0;  // k >= 128: the lane bits do not matter
          const uint64_t x = v[e], y = v[e | je];
          const bool sw = desc ? x < y : x > y;
          v[e] = sw ? y : x;
          v[e | je] = sw ? x : y;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int x = e * 64 + lane;
          const uint64_t w = xor_lane64(v[e], j);
          const bool keepMax = ((x & k) == 0) == ((x & j) == 0);
          const bool wBig = w > v[e];
          v[e] = (keepMax == wBig) ? w : v[e];
        }
      }
    }
  }
}

// The bucket ranks of rank_sort for one wave's 64 * E composites v (lane l holds entries
// e * 64 + l; the first m are real, all with keys in [T, hi]), with the wave's own LDS: the
// composites' source must be read already; `bins` (1024 words) and `placed` (64 * E entries)
// are this wave's.  Every lane gets pos[e], the descending-sort position of its entry e, or
// returns false (nothing written to pos) when a bucket holds more than kRankMaxBin of them:
// then the caller sorts v itself.  No workgroup barrier: a wave's LDS accesses take effect in
// issue order (wave_sync keeps the compiler from reordering them).
template <int E>
__device__ __forceinline__ bool rank_wave(const uint64_t (&v)[E], int m, uint32_t T, uint32_t hi,
                                          uint32_t* bins, uint64_t* placed, int (&pos)[E]) {
  static_assert(kRankBins == 1024, "16 buckets per lane");
  const int lane = threadIdx.x & 63;
  uint4* b4 = reinterpret_cast<uint4*>(bins) + 4 * lane;
#pragma unroll
  for (int q = 0; q < 4; ++q) b4[q] = make_uint4(0u, 0u, 0u, 0u);
  wave_sync();
  const uint32_t range = hi - T;
  const int rbits = range ? 32 - __clz(range) : 0;
  const int shift = rbits > 10 ? rbits - 10 : 0;
  int bin[E], slot[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool ok = 64 * e + lane < m;
    bin[e] = ((kRankBins - 1) - (int)(((uint32_t)(v[e] >> 32) - T) >> shift)) & (kRankBins - 1);
    slot[e] = ok ? (int)atomicAdd(&bins[bin[e]], 1u) : 0;
  }
  wave_sync();
  uint4 g[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) g[q] = b4[q];
  uint32_t big = 0u, seg = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    big = max(big, max(max(g[q].x, g[q].y), max(g[q].z, g[q].w)));
    seg += g[q].x + g[q].y + g[q].z + g[q].w;
  }
  if (__ballot(big > (uint32_t)kRankMaxBin) != 0ull) return false;
  uint32_t run = (uint32_t)wave_prefix((int)seg) - seg;  // buckets before 16 lane
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint4 w = g[q];
    w.x |= run << 16; run += g[q].x;
    w.y |= run << 16; run += g[q].y;
    w.z |= run << 16; run += g[q].z;
    w.w |= run << 16; run += g[q].w;
    b4[q] = w;
  }
  wave_sync();
  uint32_t bc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    bc[e] = bins[bin[e]];
    if (64 * e + lane < m) placed[(bc[e] >> 16) + slot[e]] = v[e];
  }
  wave_sync();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int b0 = (int)(bc[e] >> 16), c = 64 * e + lane < m ? (int)(bc[e] & 0xFFFFu) : 0;
    int r = 0;
    for (int j = 0; j < c; ++j) r += placed[b0 + j] > v[e] ? 1 : 0;
    pos[e] = b0 + r;
  }
  return true;
}

// KPL keys per lane of the step starting at id s: lane l takes the 16-byte groups
// s + 4 (g * 64 + l).  kVec: one 16-byte load per group; otherwise one load per key.  The loads
// go through a buffer resource that starts at key s and ends at key n (kVec: rounded up to a
// whole 16-byte group, which the row holds), so that keys past it read as 0 without touching
// memory; its base and size are scalar, and the lane's offset is the same in every step.  Raw
// FP32 bits, non-temporal; the caller masks.
template <int KPL, bool kVec>
__device__ __forceinline__ void load_step(const float* row, int n, int s, uint32_t (&raw)[KPL]) {
  const int lane = threadIdx.x & 63;
  const int left = 4 * ((kVec ? (n + 3) & ~3 : n) - s);  // bytes from key s to the end
  // data format 32 bits (the field must be non-zero for untyped accesses)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(row) + s, 0, left > 0 ? left : 0, 0x00020000);
#pragma unroll
  for (int g = 0; g < KPL / 4; ++g) {
    if constexpr (kVec) {
      const u32x4 v = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane + 1024 * g, 0, 2));
      raw[4 * g + 0] = v.x;
      raw[4 * g + 1] = v.y;
      raw[4 * g + 2] = v.z;
      raw[4 * g + 3] = v.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        raw[4 * g + e] =
            __builtin_amdgcn_raw_buffer_load_b32(rs, 16 * lane + 1024 * g + 4 * e, 0, 2);
    }
  }
}

// One wave walks keys [0, n) of `row` and leaves the min(n, kTopK) largest of those above
// thr0, by (u desc, id asc), in sh.u / sh.id[0, cnt); returns cnt (fewer than min(n, kTopK)
// only when fewer keys are above thr0).  thr0 = 0: the buffer first takes the first
// min(n, kCap) keys as they are (so a later key with u = 0 can never be among the kTopK
// largest); thr0 > 0: only keys above thr0 ever enter.  Then a step of keys at a time, with
// the next step's loads in flight: keys above the running threshold thr enter the buffer, and
// a step that would not fit cuts the buffer first (wave_keep_top) and raises thr.  The step
// past the end makes the exact cut to kTopK.
template <int kCap, int KPL, bool kVec>
__device__ __forceinline__ int walk_row(const float* row, int n, uint32_t thr0,
                                        WaveShared<kCap>& sh) {
  constexpr int kStep = 64 * KPL;
  constexpr int kSlack = kCap - kStep - kTopK;  // a cut during the walk leaves room for a step
  static_assert(kCap % 256 == 0 && kSlack >= 0, "a step must fit a cut buffer");
  static_assert(KPL % 4 == 0, "keys are loaded in 16-byte groups of 4 per lane");
  const int lane = threadIdx.x & 63;
  int cnt = 0, first = 0;
  if (thr0 == 0u) {
    // the first min(n, kCap) keys, each at its id
    constexpr int FL = kCap / 64;
    uint32_t raw[FL];
    load_step<FL, kVec>(row, n, 0, raw);
#pragma unroll
    for (int g = 0; g < FL / 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int id = (g * 64 + lane) * 4 + e;
        sh.u[id] = orderable_bits(raw[4 * g + e]);
        sh.id[id] = (uint32_t)id;
      }
    cnt = n < kCap ? n : kCap;
    first = kCap;
    wave_sync();
  }
  // kWaveDepth register buffers take turns (the loop is unrolled by that many, so no buffer is
  // copied): the loads of the next kWaveDepth - 1 steps are in flight while a step is
  // filtered.  They are unconditional (past n they read nothing and give 0): behind a branch,
  // the wait for a step's keys at the join would also wait for the later steps' loads.
  constexpr int D = kWaveDepth;
  uint32_t thr = thr0;
  uint32_t ring[D][KPL];
#pragma unroll
  for (int d = 0; d + 1 < D; ++d) load_step<KPL, kVec>(row, n, first + d * kStep, ring[d]);
  bool done = false;
  for (int s0 = first; !done; s0 += D * kStep) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int s = s0 + d * kStep;
      load_step<KPL, kVec>(row, n, s + (D - 1) * kStep, ring[(d + D - 1) % D]);
      uint32_t (&cur)[KPL] = ring[d];
      const bool more = s < n;
      // the step is counted first only when it might not fit: a buffer with room for a whole
      // step takes it as it is
      const bool mightOverflow = cnt + kStep > kCap;
      int total = 0;
      if (more) {
#pragma unroll
        for (int k = 0; k < KPL; ++k) cur[k] = orderable_bits(cur[k]);
        if (s + kStep > n) {
          asm volatile("");  // a branch: only the last step masks its keys past n
#pragma unroll
          for (int k = 0; k < KPL; ++k)
            if (s + ((k >> 2) * 64 + lane) * 4 + (k & 3) >= n) cur[k] = 0u;  // never > thr
        }
        if (mightOverflow) {
#pragma unroll
          for (int k = 0; k < KPL; ++k) total += __popcll(__ballot(cur[k] > thr));
        }
      }
      if (more ? cnt + total > kCap : cnt > kTopK)
        thr = wave_keep_top<kCap>(sh, cnt, kTopK, more ? kSlack : 0);
      if (!more) {
        done = true;
        break;
      }
      // thr through an empty asm: the comparisons are made again rather than the counting
      // loop's masks held across the cut
      uint32_t th = thr;
      asm volatile("" : "+v"(th));
#pragma unroll
      for (int k = 0; k < KPL; ++k) {
        const bool p = cur[k] > th;
        const uint64_t m = __ballot(p);
        // cnt + (keys of this step) <= kCap: room for a whole step, the count above, or a cut
        // to <= kCap - kStep
        const int pos = (int)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, cnt));
        if (p) {
          sh.u[pos] = cur[k];
          sh.id[pos] = (uint32_t)(s + ((k >> 2) * 64 + lane) * 4 + (k & 3));
        }
        cnt += __popcll(m);
      }
    }
  }
  wave_sync();
  return cnt;
}

// A key value below the row's kSel-th largest, as a rule, from a sample of 1024 of its keys (4
// runs of 256, one at each quarter of the row): the bin base, in a radix select over the sample,
// of its k-th largest key, k about 1.5 times the sample's expected share of the kSel largest
// plus 8; 0 when no estimate is made.  Only a speed-up: the walk counts the keys above it, and
// when fewer than kSel are, walks the row again without it.  n >= 1024.
template <int kCap, bool kVec>
__device__ __forceinline__ uint32_t sample_threshold(const float* row, int n, int kSel,
                                                     WaveShared<kCap>& sh) {
  constexpr int SG = 4;  // runs, one 16-byte group of 4 keys per lane each
  const int lane = threadIdx.x & 63;
  uint32_t u[4 * SG];
#pragma unroll
  for (int j = 0; j < SG; ++j) {
    const int base = ((int)((int64_t)j * n / SG) & ~3) + 4 * lane;  // base + 3 < n
    if constexpr (kVec) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + base);
      u[4 * j + 0] = v.x;
      u[4 * j + 1] = v.y;
      u[4 * j + 2] = v.z;
      u[4 * j + 3] = v.w;
    } else {
      const unsigned* r32 = reinterpret_cast<const unsigned*>(row);
#pragma unroll
      for (int e = 0; e < 4; ++e) u[4 * j + e] = r32[base + e];
    }
  }
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
  for (int i = 0; i < 4 * SG; ++i) {
    u[i] = orderable_bits(u[i]);
    mn = u[i] < mn ? u[i] : mn;
    mx = u[i] > mx ? u[i] : mx;
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const int kS = (int)((int64_t)kSel * (3 * 64 * 4 * SG) / (2 * (int64_t)n)) + 8;
  int kRem = kS, inBin = 0;
  uint32_t lo = mn;
  wave_window_select<4 * SG>(
      [&](int i, int c, bool& valid) {
        valid = true;
        return u[i];
      },
      64 * 4 * SG, sh.hist, lo, mx - mn, kRem, inBin, kS);
  return lo > 0u ? lo - 1u : 0u;  // keys above it: every key of the chosen bin and above
}

template <int kCap, int KPL, bool kVec>
__global__ __launch_bounds__(64 * kWaveRows) void topk_expand_wave_kernel(TopkArgs a) {
  __shared__ WaveShared<kCap> shAll[kWaveRows];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * kWaveRows + wave;
  if (i >= a.numRows) return;
  WaveShared<kCap>& sh = shAll[wave];
  const int64_t r = a.rowStart + i, b = r / a.S, t = r % a.S;
  int32_t* out = a.outIdx + r * kIndexWidth;
  const int64_t c = a.ctx[b];
  if (c <= 0 || t >= c) {
    for (int s = lane; s < kIndexWidth; s += 64) out[s] = -1;
    return;
  }
  const int64_t nVisT = (t + 1) / 4;
  const int n = (int)(nVisT < a.numBlocks ? nVisT : a.numBlocks);
  const int kSel = n < kTopK ? n : kTopK;
  const float* row = a.logits + i * a.numBlocks;
  int cnt = 0;
  if (n > 0) {
    const uint32_t est = n >= 4 * kCap ? sample_threshold<kCap, kVec>(row, n, kSel, sh) : 0u;
    cnt = walk_row<kCap, KPL, kVec>(row, n, est, sh);
    if (cnt < kSel) cnt = walk_row<kCap, KPL, kVec>(row, n, 0u, sh);  // estimate too high
  }
  // order the cnt = kSel selected keys: bucket ranks over [T, hi] (their smallest and largest
  // keys), or the bitonic sort when a bucket is crowded; padding composites are 0
  constexpr int E = kTopK / 64;
  static_assert(sizeof(sh.u) >= 8 * kTopK && sizeof(sh.id) >= 4 * kRankBins,
                "the placed composites and the buckets fit the candidate buffer");
  uint64_t v[E];
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = 64 * e + lane;
    v[e] = j < cnt ? composite(sh.u[j], (int)sh.id[j]) : 0ull;
    if (j < cnt) {
      const uint32_t uk = (uint32_t)(v[e] >> 32);
      lo = uk < lo ? uk : lo;
      hi = uk > hi ? uk : hi;
    }
  }
  lo = wave_min(lo);
  hi = wave_max(hi);
  wave_sync();  // the buffer is read: it now holds the buckets and the placed composites
  int pos[E];
  if (!rank_wave<E>(v, cnt, lo, hi, sh.id, reinterpret_cast<uint64_t*>(sh.u), pos)) {
    sort_wave_desc<E>(v);
#pragma unroll
    for (int e = 0; e < E; ++e) pos[e] = 64 * e + lane;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = pos[e];
    if (64 * e + lane < cnt && p < kSel) {
      const int id = (int)~(uint32_t)v[e];
#pragma unroll
      for (int j = 0; j < 4; ++j) out[4 * p + j] = 4 * id + j;
    }
  }
  const int tail = (int)((t + 1) % 4);
  for (int s = 4 * kSel + lane; s < kIndexWidth; s += 64)
    out[s] = s - 4 * kSel < tail ? (int)(4 * nVisT + (s - 4 * kSel)) : -1;
}

// ------------------------------------------------------------------------ streaming ---

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
// the selection takes (in ascending id): every key > T is selected.  Per pass each wave
// histograms the digit of the keys that match the prefix found so far into its own bins.
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

// Decode selection + expand for one sequence (rows longer than the register-resident kernels
// hold): the selection is emitted in ascending block id.  The sequence's split counters of
// the attention that follows are zeroed first.
__global__ __launch_bounds__(kSelThreads) void topk_expand_decode_stream_kernel(TopkDecodeArgs a) {
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
  write_tail_and_pad(out, 4 * kSel, n, (int)(c % 4), kSelThreads);
}

// ------------------------------------------------------------------------------ K4 etc ---

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
  write_tail_and_pad(out, 4 * kSel, nVis, tail, kSelThreads);
}

// Keys per thread for rows of up to n keys: a multiple of 4 from a short list, or 0 when the
// row is longer than the register-resident kernels hold.
int keys_per_thread(int64_t n, int threads) {
  static const int kList[] = {4, 8, 16, 24, 32, 48, 64, 72, 96, 128};
  for (int k : kList)
    if (k * threads <= 32768 && n <= (int64_t)k * threads) return k;
  return 0;
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

#define QSA_REG_CASE(KERNEL, K, NTH, GRID, ARGS)                                               \
  case K:                                                                                      \
    if (aligned) hipLaunchKernelGGL((KERNEL<K, true>), GRID, dim3(NTH), 0, stream, ARGS);      \
    else hipLaunchKernelGGL((KERNEL<K, false>), GRID, dim3(NTH), 0, stream, ARGS);             \
    break;

hipError_t launch_topk_expand(const TopkArgs& a, hipStream_t stream) {
  // largest number of complete blocks a row of the chunk can have
  const int64_t r0 = a.rowStart, r1 = a.rowStart + a.numRows - 1;
  const int64_t tMax = (r0 / a.S == r1 / a.S) ? r1 % a.S : (int64_t)a.S - 1;
  int64_t nMax = (tMax + 1) / 4;
  if (nMax > a.numBlocks) nMax = a.numBlocks;
  const bool aligned = (a.numBlocks & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0;
  const int kpt = keys_per_thread(nMax, kRT);
  const dim3 grid((unsigned)a.numRows);
  // past 72 keys per thread the register kernel holds fewer than 4 rows per CU and the
  // one-wave-per-row kernel is faster (rows of 18500 blocks: 129 against 145 us per 4096 rows;
  // 32768 blocks: 176 against 224 us)
  if (kpt == 0 || kpt > kRegMaxKeys) {
    const dim3 wgrid((unsigned)((a.numRows + kWaveRows - 1) / kWaveRows));
    const dim3 wblock(64 * kWaveRows);
    if (nMax <= 32768) {  // per 4096 rows of 20000 / 32768 blocks: 121 / 153 us (1536: 126 / 177)
      if (aligned)
        hipLaunchKernelGGL((topk_expand_wave_kernel<kWaveCapMid, kWaveKPLMid, true>), wgrid,
                           wblock, 0, stream, a);
      else
        hipLaunchKernelGGL((topk_expand_wave_kernel<kWaveCapMid, kWaveKPLMid, false>), wgrid,
                           wblock, 0, stream, a);
    } else {  // per 2048 rows of 65536 blocks: 129 us (1024: 175)
      if (aligned)
        hipLaunchKernelGGL((topk_expand_wave_kernel<kWaveCapLong, kWaveKPLLong, true>), wgrid,
                           wblock, 0, stream, a);
      else
        hipLaunchKernelGGL((topk_expand_wave_kernel<kWaveCapLong, kWaveKPLLong, false>), wgrid,
                           wblock, 0, stream, a);
    }
  } else {
    switch (kpt) {
      QSA_REG_CASE(topk_expand_reg_kernel, 4, kRT, grid, a)
      QSA_REG_CASE(topk_expand_reg_kernel, 8, kRT, grid, a)
      QSA_REG_CASE(topk_expand_reg_kernel, 16, kRT, grid, a)
      QSA_REG_CASE(topk_expand_reg_kernel, 24, kRT, grid, a)
      QSA_REG_CASE(topk_expand_reg_kernel, 32, kRT, grid, a)
      QSA_REG_CASE(topk_expand_reg_kernel, 48, kRT, grid, a)
      QSA_REG_CASE(topk_expand_reg_kernel, 64, kRT, grid, a)
      default: QSA_REG_CASE(topk_expand_reg_kernel, 72, kRT, grid, a)
    }
  }
  return hipGetLastError();
}

// Chunk of the split decode selection for rows of maxBlocks keys (0: not split): the smallest
// of 8192, 16384 and 32768 that cuts a row into at most 8 chunks (so 5 to 8 of them).
static int split_chunk(int32_t maxBlocks) {
  if (maxBlocks <= kDT * 64 || maxBlocks > kSplitMaxChunks * kSplitMaxChunk) return 0;
  int chunk = 8192;
  while ((int64_t)chunk * kSplitMaxChunks < maxBlocks) chunk *= 2;
  return chunk;
}

int64_t topk_decode_workgroups(int32_t B, int32_t maxBlocks) {
  const int chunk = split_chunk(maxBlocks);
  return chunk ? (int64_t)B * ((maxBlocks + chunk - 1) / chunk) : B;
}

#define QSA_CHUNK_CASE(K, GRID, ARGS)                                                          \
  case K:                                                                                      \
    if (aligned)                                                                               \
      hipLaunchKernelGGL((topk_decode_chunk_kernel<K, true>), GRID, dim3(kDT), 0, stream, ARGS); \
    else                                                                                       \
      hipLaunchKernelGGL((topk_decode_chunk_kernel<K, false>), GRID, dim3(kDT), 0, stream, ARGS); \
    break;

static hipError_t launch_split_decode(TopkDecodeArgs a, bool aligned, hipStream_t stream) {
  a.chunk = split_chunk(a.maxBlocks);
  a.numChunks = (a.maxBlocks + a.chunk - 1) / a.chunk;
  const dim3 cgrid((unsigned)((int64_t)a.B * a.numChunks));
  switch (a.chunk / kDT) {
    QSA_CHUNK_CASE(16, cgrid, a)
    QSA_CHUNK_CASE(32, cgrid, a)
    default: QSA_CHUNK_CASE(64, cgrid, a)
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(topk_decode_merge_kernel, dim3((unsigned)a.B), dim3(kDT), 0, stream, a);
  return hipGetLastError();
}

#undef QSA_CHUNK_CASE

hipError_t launch_topk_expand_decode(const TopkDecodeArgs& a, hipStream_t stream) {
  const bool aligned = (a.maxBlocks & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15) == 0;
  const int kpt = keys_per_thread(a.maxBlocks, kDT);
  const dim3 grid((unsigned)a.B);
  if (kpt == 0) {
    if (split_chunk(a.maxBlocks)) return launch_split_decode(a, aligned, stream);
    hipLaunchKernelGGL(topk_expand_decode_stream_kernel, grid, dim3(kSelThreads), 0, stream, a);
  } else {
    switch (kpt) {
      QSA_REG_CASE(topk_expand_decode_reg_kernel, 4, kDT, grid, a)
      QSA_REG_CASE(topk_expand_decode_reg_kernel, 8, kDT, grid, a)
      QSA_REG_CASE(topk_expand_decode_reg_kernel, 16, kDT, grid, a)
      QSA_REG_CASE(topk_expand_decode_reg_kernel, 24, kDT, grid, a)
      QSA_REG_CASE(topk_expand_decode_reg_kernel, 32, kDT, grid, a)
      QSA_REG_CASE(topk_expand_decode_reg_kernel, 48, kDT, grid, a)
      default: QSA_REG_CASE(topk_expand_decode_reg_kernel, 64, kDT, grid, a)
    }
  }
  return hipGetLastError();
}

#undef QSA_REG_CASE

}  // namespace qsa
