// Value up-projection for gfx950: out_h = U_h^V o_lat,h (page "Module 05 -- MLA: Compressing
// Per-Token History", section 3: U_h^V does not depend on the position, so it factors out of
// the weighted sum and the accumulated latent is expanded once).
//
// Per head, out^T[D x rows] = U_h^V[D x R] . o_lat^T[R x rows].  One kernel, up_v_kernel, serves
// both uses: the up-projection of given fp32 latents (mla_up_v, and the fused call with one
// split), and the fused merge of split-K attention partials (mla_latent_attn_up_v), whose merged
// latents never travel through HBM.
//
// A workgroup owns one head, half of its 256 output dims (eight waves of 16) and a group of rows.
// U^V rows are the MFMA A operand, loaded straight into registers (16 dims x 512 latents per wave,
// 64 VGPRs) and kept for every row of the group.  Rows are taken in passes of 16 (the MFMA's 16 B
// columns), spread over just enough row groups to give every CU a workgroup; each pass's latents
// (given, or merged from the partials, the merging workgroup of half 0 also writing each row's
// log-sum-exp) are staged in LDS as two bf16 terms (hi = bf16(x), lo = bf16(x - hi)) and read as
// the B operand of two MFMA 16x16x32 per k-step, so the result keeps about 16 bits of the latent.
// The first pass's loads are issued before U_h^V's, the next pass's before this pass's products.
// The workgroups of one head run on one XCD.  The time is set by the bytes each CU pulls in, not
// by HBM: half of U_h^V (128 KiB) and the latents or partials of its rows.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

__device__ __forceinline__ f32x4 mfma16x16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// LDS rows of 512 bf16 (64 chunks of 16 bytes); chunk c of row r at slot c ^ (r & 15), so the
// B-operand reads (16 consecutive rows at one chunk) fall in sixteen different bank groups
__device__ __forceinline__ int up_slot(int r, int c) { return c ^ (r & 15); }

constexpr int kFuseWaves = 8;                // 16 output channels each: half of a head's 256
constexpr int kFuseThreads = 64 * kFuseWaves;
constexpr int kFuseRows = 16;                // rows per group: the MFMA's 16 B columns
constexpr int kFuseHalf = 16 * kFuseWaves;   // output channels per workgroup
constexpr int kMaxFusePasses = 16;           // row passes per workgroup

// The partials of two chunks of eight latents of one row when there are at most eight splits (one
// group of merge slots): NS slots loaded as in merge_load8, slots past the last split reloading it.
// Held as loaded, so the next pass's loads can be in flight during this pass's products.
template <int NS>
struct FuseRaw {
  f16x8 v[2][NS];
  float2 ml[NS];
};

template <int NS>
__device__ __forceinline__ void fuse_load(FuseRaw<NS>& f, const uint16_t* po0, const uint16_t* po1, const float* pml,
                                          size_t o_step, size_t ml_step, int S) {
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const size_t s = (size_t)min(k, S - 1);
    f.ml[k] = *(const float2*)(pml + s * ml_step);
    f.v[0][k] = *(const f16x8*)(po0 + s * o_step);
    f.v[1][k] = *(const f16x8*)(po1 + s * o_step);
  }
}

// merge_splits8's steps for the two chunks of a FuseRaw (one group, merge_one_group8_blocks over
// their four blocks of four latents; the slots not loaded weigh nothing, as merge_slot_empty's), so
// the bits are those of merge_splits8
template <int NS>
__device__ __forceinline__ void fuse_merge(const FuseRaw<NS>& f, int S, float* lse2, f32x4 (&out)[2][2]) {
  float mm[8], ll[8];
  f32x4 v[4][8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    mm[k] = k < NS ? f.ml[k].x : 0.f;
    ll[k] = k < NS ? f.ml[k].y : 0.f;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        v[2 * c + h][k] = k < NS ? __builtin_convertvector((f16x4){f.v[c][k][4 * h], f.v[c][k][4 * h + 1],
                                                                    f.v[c][k][4 * h + 2], f.v[c][k][4 * h + 3]},
                                                           f32x4)
                                 : (f32x4){0.f, 0.f, 0.f, 0.f};
  }
  f32x4 o[4];
  merge_one_group8_blocks<4>(mm, ll, v, S, lse2, o);
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h) out[c][h] = o[2 * c + h];
}

// LATENTS: the rows' fp32 latents are given (o_lat); otherwise they are merged from split-K
// partials.  AHEAD: passes of 16 rows (with partials, at most eight splits), the next pass's loads
// issued before this pass's products; otherwise passes of 16 or 8 rows, each loaded when it starts
// (with partials, the general merge).  NS split slots loaded (merge_slots).
template <bool LATENTS, bool AHEAD, int NS>
__global__ __launch_bounds__(kFuseThreads) void up_v_kernel(MergeUpArgs a) {
  // two staging buffers: pass p writes buffer p & 1, so one barrier a pass suffices
  __shared__ __attribute__((aligned(1024))) uint8_t hi_t[2][kFuseRows * kRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lo_t[2][kFuseRows * kRowBytes];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wg = xcd_remap(blockIdx.x, a.total_wg);
  // logical order (head, row group, half): the workgroups of one head are adjacent, on one XCD,
  // and the two halves of a row group read the same partials through its L2
  const int half = wg & 1;
  const int grp = (wg >> 1) % a.groups;
  const int h = (wg >> 1) / a.groups;
  const int rpp = a.rows_per_pass;
  const int row0 = grp * rpp * a.passes;
  const int d0 = half * kFuseHalf + 16 * wave;
  const int ql = lane & 15, g = lane >> 4;


  // with 16 rows a pass, thread t takes row t / 32 and its chunks of eight latents c and c + 32
  // (c = t % 32); with 8 rows a pass (a single pass), row t / 64 and chunk t % 64.  Loads issued
  // ahead for rows past the end reload the last row; their results are dropped.
  const size_t prows = (size_t)a.rows * a.H;  // partial rows per split
  const size_t o_step = prows * kLatent, ml_step = 2 * prows;
  const bool two = AHEAD || rpp == kFuseRows;
  const int r = two ? threadIdx.x >> 5 : threadIdx.x >> 6;
  const int c = two ? threadIdx.x & 31 : threadIdx.x & 63;
  FuseRaw<NS> f;        // partials of the next pass
  f32x4 fl[2][2];       // latents of the next pass
  auto issue = [&](int p) {
    const size_t prow = (size_t)min(row0 + p * rpp + r, a.rows - 1) * a.H + h;
    if constexpr (LATENTS) {
      const float* src = a.o_lat + prow * kLatent + 8 * c;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        fl[k][0] = *(const f32x4*)(src + 256 * k);
        fl[k][1] = *(const f32x4*)(src + 256 * k + 4);
      }
    } else {
      const uint16_t* po = a.part_o + prow * kLatent;
      fuse_load(f, po + 8 * c, po + 8 * (c + 32), a.part_ml + 2 * prow, o_step, ml_step, a.num_splits);
    }
  };
  if constexpr (AHEAD) issue(0);
  // the first pass's latents or partials are requested before U_h^V (kept in that order by the
  // scheduling barrier): the merge or the staging of the first pass, which needs only them, then
  // runs while U_h^V is still arriving
  __builtin_amdgcn_sched_barrier(0);
  // A operand: U_h^V row d0 + ql, latents 32s + 8g .. +7, in registers for the whole kernel
  bf16x8 wa[16];
  {
    const uint16_t* wrow = a.w_v + ((size_t)h * kHeadDim + d0 + ql) * kLatent + 8 * g;
#pragma unroll
    for (int s = 0; s < 16; ++s) wa[s] = *(const bf16x8*)(wrow + 32 * s);
  }

  for (int p = 0; p < a.passes; ++p) {
    const int prow0 = row0 + p * rpp;
    if (prow0 >= a.rows) break;  // the same for the whole workgroup
    const int row = prow0 + r;
    const size_t prow = (size_t)row * a.H + h;
    f32x4 x[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
    float lse2 = 0.f;
    if constexpr (AHEAD) {
      if constexpr (LATENTS) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          x[k][0] = fl[k][0];
          x[k][1] = fl[k][1];
        }
      } else {
        fuse_merge(f, a.num_splits, &lse2, x);
      }
      __builtin_amdgcn_sched_barrier(0);  // this pass's loads consumed before the next ones land
      if (p + 1 < a.passes) issue(p + 1);
    } else if (LATENTS && row < a.rows) {
      const float* src = a.o_lat + prow * kLatent + 8 * c;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (k == 1 && !two) break;
        x[k][0] = *(const f32x4*)(src + 256 * k);
        x[k][1] = *(const f32x4*)(src + 256 * k + 4);
      }
    } else if (row < a.rows) {  // the general merge
      const uint16_t* po = a.part_o + prow * kLatent;
      const float* pml = a.part_ml + 2 * prow;
      merge_splits8<NS>(po + 8 * c, pml, o_step, ml_step, a.num_splits, &lse2, x[0]);
      if (two) {
        float unused;
        merge_splits8<NS>(po + 8 * (c + 32), pml, o_step, ml_step, a.num_splits, &unused, x[1]);
      }
    }
    if (!LATENTS && row < a.rows && a.lse != nullptr && half == 0 && c == 0) a.lse[prow] = lse2 * 0.69314718055994531f;
    // the latents as hi / lo bf16 terms; chunk cc of row r at slot cc ^ (r & 15); rows past the
    // end are zero
    uint8_t* hb = hi_t[p & 1];
    uint8_t* lb = lo_t[p & 1];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k == 1 && !two) break;
      bf16x8 vh, vl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = row < a.rows ? x[k][e >> 2][e & 3] : 0.f;
        const __bf16 bh = (__bf16)v;
        vh[e] = bh;
        vl[e] = (__bf16)(v - (float)bh);
      }
      const int off = r * kRowBytes + 16 * up_slot(r, c + 32 * k);  // k = 1 only with c < 32
      *(bf16x8*)(hb + off) = vh;
      *(bf16x8*)(lb + off) = vl;
    }
    __syncthreads();
    // the operands read from LDS in two halves of eight k-steps (registers hold the next pass's
    // partials meanwhile)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s0 = 0; s0 < 16; s0 += 8) {
      bf16x8 bh[8], bl[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int off = ql * kRowBytes + 16 * up_slot(ql, 4 * (s0 + s) + g);
        bh[s] = *(const bf16x8*)(hb + off);
        bl[s] = *(const bf16x8*)(lb + off);
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        acc = mfma16x16(wa[s0 + s], bh[s], acc);
        acc = mfma16x16(wa[s0 + s], bl[s], acc);
      }
    }
    // lane holds row prow0 + ql, output dims d0 + 4g .. +3 (with 8 rows a pass, rows 8..15 of the
    // staging were not written: those columns are dropped)
    const int orow = prow0 + ql;
    if (orow < a.rows && ql < rpp)  // the call's output: a non-temporal store
      __builtin_nontemporal_store(acc, (f32x4*)(a.out + ((size_t)orow * a.H + h) * kHeadDim + d0 + 4 * g));
  }
}

}  // namespace

namespace {

// passes of 16 rows, spread evenly over just enough row groups to give every CU a workgroup (each
// pass after the first reuses the U_h^V half in registers); passes of 8 rows, one each, where a
// single pass of 16 would already leave CUs idle
void plan_rows(MergeUpArgs& a, int cus) {
  const int p16 = (a.rows + kFuseRows - 1) / kFuseRows;
  if (2 * a.H * p16 >= cus) {
    const int want = (cus + 2 * a.H - 1) / (2 * a.H);  // row groups that fill the CUs
    const int n = (p16 + want - 1) / want;
    a.rows_per_pass = kFuseRows;
    a.passes = n < kMaxFusePasses ? n : kMaxFusePasses;
  } else {
    a.rows_per_pass = kFuseRows / 2;
    a.passes = 1;
  }
  const int per = a.rows_per_pass * a.passes;
  a.groups = (a.rows + per - 1) / per;
  a.total_wg = a.H * a.groups * 2;
}

}  // namespace

hipError_t launch_up_v(const float* o_lat, const uint16_t* w_v, float* out, int rows, int H, int cus,
                       hipStream_t stream) {
  MergeUpArgs a{};
  a.o_lat = o_lat;
  a.num_splits = 1;
  a.rows = rows;
  a.H = H;
  a.w_v = w_v;
  a.out = out;
  plan_rows(a, cus);
  void* args[] = {(void*)&a};
  const void* fn = a.rows_per_pass == kFuseRows ? (const void*)&up_v_kernel<true, true, 2>
                                                : (const void*)&up_v_kernel<true, false, 2>;
  return hipLaunchKernel(fn, dim3(a.total_wg), dim3(kFuseThreads), args, 0, stream);
}

hipError_t launch_merge_up_v(MergeUpArgs a, int cus, hipStream_t stream) {
  a.o_lat = nullptr;
  plan_rows(a, cus);
  void* args[] = {(void*)&a};
  const bool ahead = a.rows_per_pass == kFuseRows && a.num_splits <= 8;
  const int ns = merge_slots(a.num_splits);
  const void* fn = ahead ? (ns == 2   ? (const void*)&up_v_kernel<false, true, 2>
                            : ns == 4 ? (const void*)&up_v_kernel<false, true, 4>
                                      : (const void*)&up_v_kernel<false, true, 8>)
                         : (ns == 2   ? (const void*)&up_v_kernel<false, false, 2>
                            : ns == 4 ? (const void*)&up_v_kernel<false, false, 4>
                                      : (const void*)&up_v_kernel<false, false, 8>);
  return hipLaunchKernel(fn, dim3(a.total_wg), dim3(kFuseThreads), args, 0, stream);
}

}  // namespace mla
