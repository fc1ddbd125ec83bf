// Value up-projection for gfx950: out_h = U_h^V o_lat,h (page "Module 05 -- MLA: Compressing
// Per-Token History", section 3: U_h^V does not depend on the position, so it factors out of
// the weighted sum and the accumulated latent is expanded once).
//
// Per head, out^T[D x rows] = U_h^V[D x R] . o_lat^T[R x rows].  U^V, stored [D][R] per head,
// is the A operand as it lies in memory (16-byte loads along R); the fp32 latents are the B
// operand, each split into two bf16 terms (hi = bf16(x), lo = bf16(x - hi)) and multiplied
// twice, so the result keeps about 16 bits of o_lat.  Bound by reading U^V (16 MiB).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kDBlock = 64;   // output dims per workgroup (32 per wave)
constexpr int kThreads = 128;

__global__ __launch_bounds__(kThreads) void up_v_kernel(const float* __restrict__ o_lat,
                                                        const uint16_t* __restrict__ w_v,
                                                        float* __restrict__ out, int rows, int H) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ndb = kHeadDim / kDBlock;
  const int h = blockIdx.x / ndb;
  const int d0 = (blockIdx.x % ndb) * kDBlock + 32 * wave;
  const int hl = lane & 31, hf = lane >> 5;

  // A operand: U_h^V row d0 + hl, latents 16ks + 8hf .. +7
  bf16x8 wa[32];
  const uint16_t* wrow = w_v + ((size_t)h * kHeadDim + d0 + hl) * kLatent + 8 * hf;
#pragma unroll
  for (int ks = 0; ks < 32; ++ks) wa[ks] = *(const bf16x8*)(wrow + 16 * ks);

  const int nblocks = (rows + 31) / 32;
  for (int nb = 0; nb < nblocks; ++nb) {
    const int row = nb * 32 + hl;
    const bool rvalid = row < rows;
    const float* src = o_lat + ((size_t)(rvalid ? row : 0) * H + h) * kLatent + 8 * hf;
    f32x16 acc;
#pragma unroll
    for (int k = 0; k < 16; ++k) acc[k] = 0.f;
#pragma unroll 8
    for (int ks = 0; ks < 32; ++ks) {
      const f32x4 x0 = *(const f32x4*)(src + 16 * ks);
      const f32x4 x1 = *(const f32x4*)(src + 16 * ks + 4);
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = rvalid ? (e < 4 ? x0[e] : x1[e - 4]) : 0.f;
        const __bf16 bh = (__bf16)x;
        hi[e] = bh;
        lo[e] = (__bf16)(x - (float)bh);
      }
      acc = mfma32(wa[ks], hi, acc);
      acc = mfma32(wa[ks], lo, acc);
    }
    if (rvalid) {
      // lane holds query row `row`, output dims d0 + 8ii + 4hf + j
      float* dst = out + ((size_t)row * H + h) * kHeadDim + d0 + 4 * hf;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        f32x4 v = {acc[4 * ii], acc[4 * ii + 1], acc[4 * ii + 2], acc[4 * ii + 3]};
        *(f32x4*)(dst + 8 * ii) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_up_v(const float* o_lat, const uint16_t* w_v, float* out, int rows, int H,
                       hipStream_t stream) {
  void* args[] = {(void*)&o_lat, (void*)&w_v, (void*)&out, (void*)&rows, (void*)&H};
  const dim3 grid(H * (kHeadDim / kDBlock)), block(kThreads);
  return hipLaunchKernel((const void*)&up_v_kernel, grid, block, args, 0, stream);
}

}  // namespace mla
