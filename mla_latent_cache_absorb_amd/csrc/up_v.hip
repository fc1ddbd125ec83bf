// Value up-projection for gfx950: out_h = U_h^V o_lat,h (page "Module 05 -- MLA: Compressing
// Per-Token History", section 3: U_h^V does not depend on the position, so it factors out of
// the weighted sum and the accumulated latent is expanded once).
//
// Per head, out^T[D x rows] = U_h^V[D x R] . o_lat^T[R x rows].  A workgroup owns one head and 64
// output dims, four waves of 16.  U^V rows are the A operand, loaded straight into registers (16
// dims x 512 latents per wave, 64 VGPRs) and kept for every row.  The fp32 latents of 32 rows are
// staged once per workgroup in LDS, each split into two bf16 terms (hi = bf16(x), lo = bf16(x -
// hi)), and read as the B operand of two MFMA 16x16x32 per k-step, so the result keeps about 16
// bits of o_lat.  Bound by reading U^V (16 MiB) at decode sizes.
//
// merge_up_v_kernel fuses the log-sum-exp merge of split-K attention partials into the same
// product: a workgroup owns one head, all 256 output dims (sixteen waves of 16) and a group of
// rows.  It merges its rows' partials straight into the hi / lo LDS staging, so the merged
// latents never travel through HBM, and writes each row's log-sum-exp.  The groups of one head
// run on one XCD and share U_h^V through its L2.  Half of U_h^V (latents 0..255) is copied
// straight into LDS and half is held in registers; both copies are issued before the merge's
// loads, so the whole workgroup has one memory round trip.  Its time is set by the bytes each CU
// pulls in (256 KiB of U_h^V, the partials of its rows), not by HBM.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kDBlock = 64;           // output dims per workgroup (16 per wave)
constexpr int kUpWaves = 4;
constexpr int kThreads = 64 * kUpWaves;
constexpr int kUpRows = 32;           // o_lat rows staged per pass
constexpr int kMaxRowGroups = 32;

__device__ __forceinline__ f32x4 mfma16x16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS rows of 512 bf16 (64 chunks of 16 bytes); chunk c of row r at slot c ^ (r & 15), so the
// B-operand reads (16 consecutive rows at one chunk) fall in sixteen different bank groups
__device__ __forceinline__ int up_slot(int r, int c) { return c ^ (r & 15); }

__global__ __launch_bounds__(kThreads) void up_v_kernel(const float* __restrict__ o_lat,
                                                        const uint16_t* __restrict__ w_v,
                                                        float* __restrict__ out, int rows, int H) {
  __shared__ __attribute__((aligned(1024))) uint8_t hi_t[kUpRows * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lo_t[kUpRows * kRowBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ndb = kHeadDim / kDBlock;
  const int h = blockIdx.x / ndb;
  const int d0 = (blockIdx.x % ndb) * kDBlock + 16 * wave;
  const int ql = lane & 15, g = lane >> 4;

  // A operand: U_h^V row d0 + ql, latents 32s + 8g .. +7
  bf16x8 wa[16];
  {
    const uint16_t* wrow = w_v + ((size_t)h * kHeadDim + d0 + ql) * kLatent + 8 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) wa[s] = *(const bf16x8*)(wrow + 32 * s);
  }

  const int npass = (rows + kUpRows - 1) / kUpRows;
  for (int pass = blockIdx.y; pass < npass; pass += gridDim.y) {
    const int row0 = pass * kUpRows;
    __syncthreads();  // the previous pass's reads are done
    // stage rows row0 .. row0+31: task t = 8 consecutive latents (chunk t % 64) of row t / 64.
    // Every load is issued before any is used (rows past the end reload the last row and are
    // zeroed after), so the staging is one memory round trip.
    constexpr int kTasks = kUpRows * 64 / kThreads;
    f32x4 xs[kTasks][2];
#pragma unroll
    for (int k = 0; k < kTasks; ++k) {
      const int task = threadIdx.x + kThreads * k;
      const int row = min(row0 + (task >> 6), rows - 1);
      const float* src = o_lat + ((size_t)row * H + h) * kLatent + 8 * (task & 63);
      xs[k][0] = *(const f32x4*)src;
      xs[k][1] = *(const f32x4*)(src + 4);
    }
#pragma unroll
    for (int k = 0; k < kTasks; ++k) {
      const int task = threadIdx.x + kThreads * k;
      const int r = task >> 6, c = task & 63;
      f32x4 x0 = xs[k][0], x1 = xs[k][1];
      if (row0 + r >= rows) x0 = x1 = (f32x4){0.f, 0.f, 0.f, 0.f};
      bf16x8 vh, vl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? x0[e] : x1[e - 4];
        const __bf16 bh = (__bf16)x;
        vh[e] = bh;
        vl[e] = (__bf16)(x - (float)bh);
      }
      const int off = r * kRowBytes + 16 * up_slot(r, c);
      *(bf16x8*)(hi_t + off) = vh;
      *(bf16x8*)(lo_t + off) = vl;
    }
    __syncthreads();
#pragma unroll
    for (int rb = 0; rb < kUpRows / 16; ++rb) {
      const int r = 16 * rb + ql;
      // every operand of the block read from LDS before the first product (one LDS round trip)
      bf16x8 bh[16], bl[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int off = r * kRowBytes + 16 * up_slot(r, 4 * s + g);
        bh[s] = *(const bf16x8*)(hi_t + off);
        bl[s] = *(const bf16x8*)(lo_t + off);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        acc = mfma16x16(wa[s], bh[s], acc);
        acc = mfma16x16(wa[s], bl[s], acc);
      }
      // lane holds row row0 + r, output dims d0 + 4g .. +3
      const int row = row0 + r;
      if (row < rows) *(f32x4*)(out + ((size_t)row * H + h) * kHeadDim + d0 + 4 * g) = acc;
    }
  }
}

constexpr int kFuseWaves = kHeadDim / 16;  // one wave per 16 output dims
constexpr int kFuseThreads = 64 * kFuseWaves;
constexpr int kFuseMaxRows = 16;             // rows per group: the MFMA's 16 B columns

__global__ __launch_bounds__(kFuseThreads) void merge_up_v_kernel(MergeUpArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t hi_t[kFuseMaxRows * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lo_t[kFuseMaxRows * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t wv_t[kHeadDim * kRowBytes / 2];  // U_h^V, latents 0..255
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wg = xcd_remap(blockIdx.x, a.total_wg);
  const int h = wg / a.groups;  // the groups of one head are adjacent: one XCD, one L2 copy of U_h^V
  const int row0 = (wg % a.groups) * a.rows_per_group;
  const int d0 = 16 * wave;
  const int ql = lane & 15, g = lane >> 4;
  const uint16_t* wh = a.w_v + ((size_t)h * kHeadDim + d0) * kLatent;

  // U_h^V rows d0 .. d0+15 of this wave, latents 0..255, copied to LDS 1 KiB per instruction
  // (two half rows); slot p of local row r holds the 16-byte chunk p ^ (r & 15), so that the
  // operand reads below (16 rows at one chunk) fall in sixteen different bank groups
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 2 * j + (lane >> 5), p = lane & 31;
    copy16_to_lds(wh + (size_t)r * kLatent + 8 * (p ^ (r & 15)), lds_addr(wv_t + (d0 + 2 * j) * (kRowBytes / 2)));
  }
  // latents 256..511 as the A operand in registers: row d0 + ql, latents 256 + 32s + 8g .. +7
  bf16x8 wa[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) wa[s] = *(const bf16x8*)(wh + (size_t)ql * kLatent + 256 + 32 * s + 8 * g);

  // merge: task = (row r of the group, latents 4t .. 4t+3), 128 tasks per row
  const size_t prow_count = (size_t)a.rows * a.H;  // partial rows per split
  for (int task = threadIdx.x; task < kFuseMaxRows * 128; task += kFuseThreads) {
    const int r = task >> 7, t = task & 127;
    const int row = row0 + r;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (r < a.rows_per_group && row < a.rows) {
      const size_t prow = (size_t)row * a.H + h;
      float lse2;
      x = merge_splits(a.part_o + prow * kLatent + 4 * t, a.part_ml + 2 * prow, prow_count * kLatent,
                       2 * prow_count, a.num_splits, &lse2);
      if (a.lse != nullptr && t == 0) a.lse[prow] = lse2 * 0.69314718055994531f;
    }
    s16x4 vh, vl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const __bf16 bh = (__bf16)x[e];
      vh[e] = __builtin_bit_cast(short, bh);
      vl[e] = __builtin_bit_cast(short, (__bf16)(x[e] - (float)bh));
    }
    const int off = r * kRowBytes + 16 * up_slot(r, t >> 1) + 8 * (t & 1);
    *(s16x4*)(hi_t + off) = vh;
    *(s16x4*)(lo_t + off) = vl;
  }
  wait_vmcnt<0>();  // the U^V copies have landed
  __syncthreads();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const uint8_t* wrow = wv_t + (d0 + ql) * (kRowBytes / 2);
  // operands read from LDS kAhead k-steps ahead of the products that use them
  constexpr int kAhead = 4;
  bf16x8 ow[kAhead + 1], oh[kAhead + 1], ol[kAhead + 1];
  auto rd = [&](int s, int slot) {
    if (s < 8) ow[slot] = *(const bf16x8*)(wrow + 16 * ((4 * s + g) ^ ql));
    const int off = ql * kRowBytes + 16 * up_slot(ql, 4 * s + g);
    oh[slot] = *(const bf16x8*)(hi_t + off);
    ol[slot] = *(const bf16x8*)(lo_t + off);
  };
#pragma unroll
  for (int s = 0; s < kAhead; ++s) rd(s, s);
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    if (s + kAhead < 16) rd(s + kAhead, (s + kAhead) % (kAhead + 1));
    const int k = s % (kAhead + 1);
    const bf16x8 w = s < 8 ? ow[k] : wa[s - 8];
    __builtin_amdgcn_sched_barrier(0);
    acc = mfma16x16(w, oh[k], acc);
    acc = mfma16x16(w, ol[k], acc);
    __builtin_amdgcn_sched_barrier(0);
  }
  // lane holds row row0 + ql, output dims d0 + 4g .. +3
  const int row = row0 + ql;
  if (ql < a.rows_per_group && row < a.rows)
    *(f32x4*)(a.out + ((size_t)row * a.H + h) * kHeadDim + d0 + 4 * g) = acc;
}

}  // namespace

hipError_t launch_up_v(const float* o_lat, const uint16_t* w_v, float* out, int rows, int H,
                       hipStream_t stream) {
  void* args[] = {(void*)&o_lat, (void*)&w_v, (void*)&out, (void*)&rows, (void*)&H};
  const int npass = (rows + kUpRows - 1) / kUpRows;
  const dim3 grid(H * (kHeadDim / kDBlock), npass < kMaxRowGroups ? npass : kMaxRowGroups), block(kThreads);
  return hipLaunchKernel((const void*)&up_v_kernel, grid, block, args, 0, stream);
}

int merge_up_v_rows_per_group(int rows, int H, int cus) {
  // the largest group (at most 16 rows) that still gives every CU a workgroup
  int rg = kFuseMaxRows;
  while (rg > 4 && (int64_t)H * ((rows + rg - 1) / rg) < cus) rg >>= 1;
  return rg;
}

hipError_t launch_merge_up_v(MergeUpArgs a, int cus, hipStream_t stream) {
  a.rows_per_group = merge_up_v_rows_per_group(a.rows, a.H, cus);
  a.groups = (a.rows + a.rows_per_group - 1) / a.rows_per_group;
  a.total_wg = a.H * a.groups;
  void* args[] = {(void*)&a};
  return hipLaunchKernel((const void*)&merge_up_v_kernel, dim3(a.total_wg), dim3(kFuseThreads), args, 0, stream);
}

}  // namespace mla
