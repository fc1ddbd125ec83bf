// Streaming-read measurement for gfx950 (not a step of the attention path).  It reads a buffer
// once with 16-byte non-temporal vector loads (the policy the attention kernels give a cache stream
// that no other workgroup shares): each workgroup takes 32 KiB chunks in turn (chunk c by workgroup
// c mod grid, so consecutive workgroups read consecutive chunks), eight loads in flight per lane,
// and folds the bytes into one value that is stored only if it equals a caller-given value, so
// that no load can be dropped and practically nothing is written.  Its rate is the device's plain
// streaming-read rate: the ceiling the attention kernels' cache streams are measured against,
// beside the published peak (page "Module 05 -- MLA: Compressing Per-Token History", section 5:
// decode is bandwidth-bound, and which regime a workload is in is measured, not counted).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr int kGrid = 8192;

typedef int i32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const i32x4* __restrict__ src, size_t chunks,
                                                               uint32_t never, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  for (size_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const i32x4* p = src + c * (kThreads * kUnroll);
    i32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(p + u * kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= (uint32_t)(v[u].x ^ v[u].y ^ v[u].z ^ v[u].w);
  }
  if (acc == never) atomicOr(sink, 1u);
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t never, uint32_t* sink, hipStream_t stream) {
  const size_t chunks = bytes / kStreamChunkBytes;
  const int grid = chunks < (size_t)kGrid ? (int)chunks : kGrid;
  const i32x4* s = (const i32x4*)src;
  void* args[] = {(void*)&s, (void*)&chunks, (void*)&never, (void*)&sink};
  return hipLaunchKernel((const void*)&stream_read_kernel, dim3(grid), dim3(kThreads), args, 0, stream);
}

}  // namespace mla
