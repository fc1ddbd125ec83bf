// Query absorption for gfx950: q~_h = prescale * (U_h^K)^T q_h (page "Module 05 -- MLA:
// Compressing Per-Token History", section 3: the pre-transformed query is computed once per
// query and head, independently of the cached token it is later scored against).
//
// Per head this is a small GEMM, Q~^T[R x rows] = (U_h^K)^T[R x D] . Q_h^T[D x rows], bound by
// reading U^K (16 MiB for 64 heads).  U^K is stored as in the checkpoint, [D][R] per head, so
// its transpose is the A operand: a [256 d x 128 r] slab of it is staged in LDS (64 KiB,
// 16-byte chunks swizzled per row) and read with the LDS transpose read.  The queries are the
// B operand, 16-byte loads straight from memory.  Accumulation is fp32, the result is rounded
// to nearest-even bf16; on request the rounding's remainder is written as a second bf16 term
// (lo = bf16(x - hi)), so that hi + lo carries x to about 2^-17 of its magnitude.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kRBlock = 128;                 // latents per workgroup
constexpr int kSlabRowBytes = kRBlock * 2;   // 256 B per d-row of the slab
constexpr int kThreads = 128;

// AHEAD (more than one block of 32 rows): the next block's queries are loaded while this block
// multiplies; with one block the kernel is the plain form
template <bool AHEAD>
__global__ __launch_bounds__(kThreads) void absorb_q_kernel(const uint16_t* __restrict__ q,
                                                            const uint16_t* __restrict__ w_k,
                                                            uint16_t* __restrict__ q_abs,
                                                            uint16_t* __restrict__ q_abs_lo, int rows,
                                                            int H, float prescale) {
  __shared__ __attribute__((aligned(1024))) uint8_t slab[kHeadDim * kSlabRowBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nrb = kLatent / kRBlock;
  const int h = blockIdx.x / nrb;
  const int r0 = (blockIdx.x % nrb) * kRBlock;

  const int hl = lane & 31, hf = lane >> 5;
  const int nblocks = (rows + 31) / 32;
  // queries of row block nb as the B operand: lane (row hl, half hf) holds d = 16ks + 8hf .. +7
  bf16x8 bq[16], bq_next[AHEAD ? 16 : 1];
  auto load_q = [&](int nb) {
    const int row = nb * 32 + hl;
    const bool rvalid = row < rows;
    const uint16_t* qsrc = q + ((size_t)(rvalid ? row : 0) * H + h) * kHeadDim + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      bf16x8 v = *(const bf16x8*)(qsrc + 16 * ks);
      if (!rvalid) v = (bf16x8)(s16x8){0, 0, 0, 0, 0, 0, 0, 0};
      bq[ks] = v;
    }
  };
  // the next block's rows, zeroed when used if past the end
  auto load_next = [&](int nb) {
    if constexpr (AHEAD) {
      const int row = nb * 32 + hl;
      const uint16_t* qsrc = q + ((size_t)(row < rows ? row : 0) * H + h) * kHeadDim + 8 * hf;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) bq_next[ks] = *(const bf16x8*)(qsrc + 16 * ks);
    }
  };
  load_q(0);  // issued before the slab copies, so the two memory latencies overlap

  // stage U_h^K[0:256][r0:r0+128]: one instruction moves 4 d-rows (lane s: row 4k + s/16,
  // chunk slot s%16 holds global chunk (s%16) ^ swz(row))
  {
    const uint8_t* wsrc = (const uint8_t*)(w_k + ((size_t)h * kHeadDim) * kLatent + r0);
#pragma unroll 4
    for (int k = 0; k < 32; ++k) {
      const int inst = wave * 32 + k;
      const int row = 4 * inst + (lane >> 4);
      const int slot = lane & 15;
      const uint8_t* src = wsrc + (size_t)row * kRowBytes + ((slot ^ swz(row)) << 4);
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(slab + inst * 1024), 16, 0, 0);
    }
  }
  wait_vmcnt<0>();
  __syncthreads();

  // transpose-read addressing: group g = lane/16 supplies d-rows 16ks + 8(g/2) + 4r2 + e and
  // latent columns 32mb + 16(g&1) + 4c of the slab
  const int g = lane >> 4, ip = lane & 15, te = ip >> 2, tc = ip & 3;
  for (int nb = 0; nb < nblocks; ++nb) {
    const int row = nb * 32 + hl;
    const bool rvalid = row < rows;
    if constexpr (AHEAD) {
      if (nb > 0) {
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) bq[ks] = rvalid ? bq_next[ks] : (bf16x8)(s16x8){0, 0, 0, 0, 0, 0, 0, 0};
      }
      if (nb + 1 < nblocks) load_next(nb + 1);
    } else if (nb > 0) {
      load_q(nb);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int mb = 2 * wave + m;
      f32x16 acc;
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[k] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        s16x4 part[2];
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const int d = 16 * ks + 8 * (g >> 1) + 4 * r2 + te;
          const int chunk = 4 * mb + 2 * (g & 1) + (tc >> 1);
          part[r2] = lds_read_tr16(slab + d * kSlabRowBytes + ((chunk ^ swz(d)) << 4) + ((tc & 1) << 3));
        }
        acc = mfma32(concat_bf16(part[0], part[1]), bq[ks], acc);
      }
      if (rvalid) {
        // lane holds query row `row`, latents r0 + 32mb + 8ii + 4hf + j
        const size_t off = ((size_t)row * H + h) * kLatent + r0 + 32 * mb + 4 * hf;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          s16x4 v, vl;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float x = acc[4 * ii + j] * prescale;
            const uint16_t hb = f32_to_bf16_bits(x);
            v[j] = (short)hb;
            // x - hi is exact in fp32 (hi is x's nearest bf16)
            vl[j] = (short)f32_to_bf16_bits(x - bf16_bits_to_f32(hb));
          }
          *(s16x4*)(q_abs + off + 8 * ii) = v;
          if (q_abs_lo != nullptr) *(s16x4*)(q_abs_lo + off + 8 * ii) = vl;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_absorb_q(const uint16_t* q, const uint16_t* w_k, uint16_t* q_abs, uint16_t* q_abs_lo, int rows,
                           int H, float prescale, hipStream_t stream) {
  void* args[] = {(void*)&q, (void*)&w_k, (void*)&q_abs, (void*)&q_abs_lo, (void*)&rows, (void*)&H,
                  (void*)&prescale};
  const dim3 grid(H * (kLatent / kRBlock)), block(kThreads);
  const void* k = rows > 32 ? (const void*)&absorb_q_kernel<true> : (const void*)&absorb_q_kernel<false>;
  return hipLaunchKernel(k, grid, block, args, 0, stream);
}

}  // namespace mla
