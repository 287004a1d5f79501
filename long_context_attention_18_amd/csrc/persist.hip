// persist.hip -- copies between a cache's per-sequence state and a contiguous snapshot buffer.
//
// The KV-cache section of velog.io "DeepSeek V4 논문 정리" keeps the compressed cache, the
// sliding-window state and the uncompressed tail as separate pieces and stores compressed KV on
// disk for requests that share a prefix. A sequence's state is a handful of contiguous runs in the
// cache's arrays (its compressed entries, indexer keys, tail rows, and at most two runs of window
// slots, since the window is a ring); snapshot and restore are the same kernel over a table of such
// runs, one grid row per destination sequence. The copy is a pure HBM stream: each run moves in the
// widest unit (16, 4 or 1 bytes) that its two addresses and its length allow.
#include "kernels.h"

namespace lca {

namespace {

__global__ __launch_bounds__(256) void copy_runs_kernel(CopyArgs a) {
  const int tid = threadIdx.x;
  if (a.header_dst && blockIdx.x == 0 && blockIdx.y == 0 && tid < kCopyHeaderWords)
    reinterpret_cast<uint32_t*>(a.header_dst)[tid] = a.header[tid];
  const uint64_t i0 = (uint64_t)blockIdx.x * blockDim.x + tid;
  const uint64_t step = (uint64_t)gridDim.x * blockDim.x;
  for (int s = 0; s < a.n_runs; ++s) {
    const CopyRun& r = a.run[s];
    const uint8_t* src = r.src ? r.src + (uint64_t)blockIdx.y * r.src_stride : nullptr;
    uint8_t* dst = r.dst + (uint64_t)blockIdx.y * r.dst_stride;
    if (!r.src) {
      for (uint64_t i = i0; i < r.bytes; i += step) dst[i] = 0;
    } else if (r.unit == 16) {
      const uint64_t n = r.bytes / 16;
      for (uint64_t i = i0; i < n; i += step)
        reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    } else if (r.unit == 4) {
      const uint64_t n = r.bytes / 4;
      for (uint64_t i = i0; i < n; i += step)
        reinterpret_cast<uint32_t*>(dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
    } else {
      for (uint64_t i = i0; i < r.bytes; i += step) dst[i] = src[i];
    }
  }
}

}  // namespace

hipError_t launch_copy_runs(CopyArgs& a, int32_t n_dst, hipStream_t s) {
  if (a.n_runs > kMaxCopyRuns || n_dst < 1) return hipErrorInvalidValue;
  uint64_t units = 0;
  for (int i = 0; i < a.n_runs; ++i) {
    CopyRun& r = a.run[i];
    const uintptr_t al = (uintptr_t)r.src | (uintptr_t)r.dst | (uintptr_t)r.bytes | (uintptr_t)r.src_stride |
                         (uintptr_t)r.dst_stride;
    r.unit = (al % 16 == 0) ? 16 : ((al % 4 == 0) ? 4 : 1);
    const uint64_t u = r.bytes / (uint64_t)r.unit;
    units = u > units ? u : units;
  }
  // about 16 units per thread for the longest run, within 1024 workgroups per destination
  uint64_t wgs = (units + 256 * 16 - 1) / (256 * 16);
  wgs = wgs < 1 ? 1 : (wgs > 1024 ? 1024 : wgs);
  hipLaunchKernelGGL(copy_runs_kernel, dim3((unsigned)wgs, (unsigned)n_dst), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lca
