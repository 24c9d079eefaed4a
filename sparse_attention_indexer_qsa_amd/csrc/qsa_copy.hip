// qsa_copy.hip — a plain device-to-device copy, the streaming reference the benchmark sets
// beside the fused kernel: the same bytes read and written with no arithmetic, in the form
// that moves them fastest on gfx950 (one 16-byte chunk per thread, non-temporal load and
// store, 256-thread workgroups).  Not a step of the indexer.

#include "qsa_internal.h"

namespace qsa {
namespace {

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void stream_copy_kernel(u32x4_t* __restrict__ dst,
                                                                   const u32x4_t* __restrict__ src,
                                                                   int64_t chunks) {
  const int64_t i = (int64_t)blockIdx.x * kCopyThreads + threadIdx.x;
  if (i < chunks) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t launch_stream_copy(void* dst, const void* src, int64_t bytes, hipStream_t stream) {
  const int64_t chunks = bytes / 16;
  const dim3 grid((unsigned)((chunks + kCopyThreads - 1) / kCopyThreads));
  hipLaunchKernelGGL(stream_copy_kernel, grid, dim3(kCopyThreads), 0, stream,
                     static_cast<u32x4_t*>(dst), static_cast<const u32x4_t*>(src), chunks);
  return hipGetLastError();
}

}  // namespace qsa
