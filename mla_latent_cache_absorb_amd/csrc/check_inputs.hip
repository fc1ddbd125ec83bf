// Device-side precondition check of the attention calls, for debugging callers: the calls
// themselves only guarantee memory safety on bad device data (page "Module 05 -- MLA:
// Compressing Per-Token History", section 4: query t sees j <= t; page "Module 08 -- Vision,
// MTP, and Hybrid Serving State", section 2: the Q new positions are the last Q of the cache;
// colibri "DSA with k-pooling": a query's positions are a sorted selection of its prefix).
//
// One workgroup scans every sequence and every index row, so the flag word is written once, by
// one thread, after a block-wide OR in LDS: no global atomics and no clearing launch are needed,
// and the call can be captured in a graph.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_inputs_kernel(CheckArgs a) {
  __shared__ int flags;
  if (threadIdx.x == 0) flags = 0;
  __syncthreads();
  int f = 0;
  for (int b = threadIdx.x; b < a.B; b += kCheckThreads) {
    const int L = a.cache_len[b];
    if (L < a.Q) f |= kBadCacheLenShort;
    if (L > a.max_cache_len) f |= kBadCacheLenLong;
  }
  if (a.idx != nullptr) {
    // one index slot per thread per pass; a slot compares itself with the one before it
    const int64_t slots = (int64_t)a.B * a.Q * a.K_max;
    for (int64_t e = threadIdx.x; e < slots; e += kCheckThreads) {
      const int64_t bq = e / a.K_max;
      const int s = (int)(e - bq * a.K_max);
      const int b = (int)(bq / a.Q), i = (int)(bq - (int64_t)b * a.Q);
      const int n = a.idx_len[bq];
      if (s == 0 && (n < 1 || n > a.K_max)) f |= kBadIdxLen;
      if (s >= min(max(n, 0), a.K_max)) continue;
      const int L = min(a.cache_len[b], a.max_cache_len);
      const int p = a.idx[e];
      if (p < 0 || p >= L) f |= kBadIdxRange;
      if (p > a.cache_len[b] - a.Q + i) f |= kBadIdxCausal;
      if (s > 0 && a.idx[e - 1] >= p) f |= kBadIdxOrder;
    }
  }
  if (f != 0) atomicOr(&flags, f);
  __syncthreads();
  if (threadIdx.x == 0) *a.flags = flags;
}

}  // namespace

hipError_t launch_check_inputs(const CheckArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<CheckArgs*>(&a)};
  return hipLaunchKernel((const void*)&check_inputs_kernel, dim3(1), dim3(kCheckThreads), args, 0, stream);
}

}  // namespace mla
