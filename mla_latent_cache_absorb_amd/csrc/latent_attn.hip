// Split-K latent attention for gfx950: the scores and the value sum of absorbed MLA computed
// directly on the cached 512-wide latents (page "Module 05 -- MLA: Compressing Per-Token
// History", section 3; colibri "MLA is absorbed").
//
// One workgroup = one (sequence b, query i, group of 64 heads, split of positions); four
// waves, wave w owning heads 32*(w&1) .. +31 of the group and latents 256*(w>>1) .. +255.
// Per tile of 32 cached latents (32 KiB, staged in LDS straight from HBM with
// global_load_lds_dwordx4 while the previous tile is computed):
//   scores    S^T[32 pos x 32 heads] = C[32 x 512] . Q~^T[512 x 32]: each wave of a head pair
//             contracts its own 256 latents (16 MFMA 32x32x16; A = the tile row-major via
//             ds_read_b128, B = the absorbed query held in VGPRs); the two partial sums are
//             swapped through LDS and added, so both waves hold the same full scores
//   softmax   online, per head = per lane column; the running maximum only moves when it
//             grows by more than 2^8, so the accumulator is rarely rescaled
//   values    O^T[256 x 32 heads] += C^T[256 x 32 pos] . P^T[32 pos x 32 heads] (16 MFMA)
//             A = the SAME tile read transposed (ds_read_b64_tr_b16), B = P straight from
//             the score registers (the K order of the MFMA is permuted to match them)
// One latent row serves all 64 heads: the cache is read once per (query, split).
#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kTile = kTilePositions;
constexpr int kStages = 2;          // one tile computed while the next is in flight
constexpr int kThreads = 256;
constexpr int kRowsPerWave = kTile / 4;
constexpr float kRescaleLog2 = 8.0f;

// Two workgroups share a CU (8 waves, two per SIMD, 80 KiB of LDS each): gfx950 needs two
// waves per SIMD to approach its LDS read bandwidth, and the other workgroup's waves fill the
// matrix core while a wave waits at a barrier or on LDS.  Per wave and tile: 16 MFMAs for the
// partial scores, 16 for the values.
template <bool INDEXED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void latent_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages][kTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) f32x4 xbuf[4][4][64];  // partial scores [wave][reg/4][lane]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps it in SGPRs
  const int wg = xcd_remap(blockIdx.x, a.total_wg);
  // logical order (b, head group, split, query): the queries of one split of one sequence
  // are adjacent, so they run on the same XCD and share the tile through its L2
  const int i = wg % a.Q;
  int rest = wg / a.Q;
  const int split = rest % a.num_splits;
  rest /= a.num_splits;
  const int hg = rest % a.HG;
  const int b = rest / a.HG;
  const int bq = b * a.Q + i;
  const int hh = wave & 1;        // head half of the group
  const int lh = wave >> 1;       // latent half
  const int h0 = hg * 64 + hh * 32;
  const int hl = lane & 31;
  const int hf = lane >> 5;

  const int L = min(a.cache_len[b], a.max_cache_len);
  int n_slots;
  const int32_t* idx_row = nullptr;
  if constexpr (INDEXED) {
    idx_row = a.idx + (size_t)bq * a.K_max;
    n_slots = L > 0 ? min(a.idx_len[bq], a.K_max) : 0;
  } else {
    n_slots = L - a.Q + i + 1;  // positions 0 .. cache_len - Q + i
  }
  n_slots = max(n_slots, 0);
  const int s_begin = split * a.split_len;
  const int s_end = min(s_begin + a.split_len, n_slots);
  const int ntiles = s_end > s_begin ? (s_end - s_begin + kTile - 1) / kTile : 0;
  const uint8_t* seq = a.cache + (size_t)b * a.cache_bstride_bytes;
  const float c2 = a.scale_log2;

  // absorbed query of head h0+hl as the B operand: latents 256lh + 16ks + 8hf .. +7
  bf16x8 qf[16];
  {
    const uint16_t* qrow = a.q_abs + ((size_t)bq * a.H + h0 + hl) * kLatent + 256 * lh + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = *(const bf16x8*)(qrow + 16 * ks);
  }
  // complete these loads here: the loop's waits then count tile copies only
  wait_vmcnt<0>();

  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int k = 0; k < 16; ++k) o[mb][k] = 0.f;
  float m_run = -INFINITY;  // running maximum of scale*log2(e)*score
  float l_run = 0.f;        // running sum of 2^(scale*log2(e)*score - m_run)

  // ---- tile loader: wave w copies tile rows 8w .. 8w+7, one 1 KiB row per instruction;
  // lane s of row r takes global chunk s ^ swz(r) into slot s.
  // Every row read is a visible row: rows past the split repeat its last row and indexed
  // slots naming a position outside the cache read row 0; both are masked out of the scores.
  // Index lists are read with scalar loads, so waiting for them never waits for tile copies.
  const uint32_t lane16 = (uint32_t)lane << 4;
  const uint32_t lds0 = lds_addr(&smem[0][0]);
  auto issue = [&](int t) {
    const uint32_t dst = lds0 + (t % kStages) * (kTile * kRowBytes) + wave * kRowsPerWave * kRowBytes;
    const int base = s_begin + t * kTile + wave * kRowsPerWave;
#pragma unroll
    for (int rr = 0; rr < kRowsPerWave; ++rr) {
      int p;
      if constexpr (INDEXED) {
        p = idx_row[min(base + rr, s_end - 1)];
        p = (p >= 0 && p < L) ? p : 0;
      } else {
        p = min(base + rr, s_end - 1);
      }
      row_to_lds(seq + (size_t)p * kRowBytes, dst + rr * kRowBytes, lane16,
                 (uint32_t)(swz(wave * kRowsPerWave + rr) << 4));
    }
  };
  // rows of tile t that hold a visible position (bit r = tile row r)
  auto valid_rows = [&](int t) -> uint32_t {
    const int base = s_begin + t * kTile;
    const int nvalid = s_end - base;
    uint32_t v = nvalid >= kTile ? 0xffffffffu : ((1u << nvalid) - 1u);
    if constexpr (INDEXED) {
#pragma unroll
      for (int r = 0; r < kTile; ++r) {
        const int p = idx_row[min(base + r, s_end - 1)];
        if (!(p >= 0 && p < L)) v &= ~(1u << r);
      }
    }
    return v;
  };

  // ---- per-lane LDS addressing (byte offsets inside a stage)
  // scores: A row = tile row (lane & 31), global chunk 32lh + 2ks + hf; the swizzle flips
  // its low four bits, so with ks = 8u + v it sits at 32lh + 16u + ((2v + hf) ^ swz(row))
  const int prow = lane & 31;
  const int psw = swz(prow);
  const int qk_base = prow * kRowBytes + 512 * lh;
  // values: transpose read; group g = lane / 16 supplies tile rows trow + 8r2 (+16ks),
  // trow = 4(g/2) + e, and latent columns 256lh + 32mb + 16(g&1) + 4c: global chunk
  // 32lh + 16(mb>>2) + 4(mb&3) + x with x = 2(g&1) + c/2.  For rows trow + 8r2 the swizzle is
  // 4 fh + fl(r2) with fh = trow & 3 and fl(r2) = ((trow >> 2) + 2 r2) & 3, so the chunk sits at
  // 32lh + 16(mb>>2) + 4((mb&3) ^ fh) + (x ^ fl(r2)).
  const int g = lane >> 4, ip = lane & 15, te = ip >> 2, tc = ip & 3;
  const int trow = 4 * (g >> 1) + te;
  const int tx = 2 * (g & 1) + (tc >> 1);
  const int tfh = trow & 3;
  const int tr_b0 = trow * kRowBytes + 512 * lh + ((tx ^ ((trow >> 2) & 3)) << 4) + ((tc & 1) << 3);
  const int tr_b1 = (trow + 8) * kRowBytes + 512 * lh + ((tx ^ (((trow >> 2) + 2) & 3)) << 4) + ((tc & 1) << 3);

  // partial scores of tile t over this wave's 256 latents: sixteen k-steps in pairs (the
  // other wave on the SIMD covers the read latency)
  auto scores = [&](const uint8_t* tile, f32x16& sc) {
#pragma unroll
    for (int k = 0; k < 16; ++k) sc[k] = 0.f;
#pragma unroll
    for (int grp = 0; grp < 8; ++grp) {
      bf16x8 av[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int ks = 2 * grp + k;
        av[k] = *(const bf16x8*)(tile + qk_base + 256 * (ks >> 3) + (((2 * (ks & 7) + hf) ^ psw) << 4));
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) sc = mfma32(av[k], qf[2 * grp + k], sc);
    }
  };
  // add the partner's partial (same heads, other latents) and mask rows past the visible set
  auto complete_scores = [&](f32x16& sc, uint32_t valid) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 x = xbuf[wave ^ 2][k][lane];
      sc[4 * k] += x[0];
      sc[4 * k + 1] += x[1];
      sc[4 * k + 2] += x[2];
      sc[4 * k + 3] += x[3];
    }
    if (valid != 0xffffffffu) {
      const uint32_t vb = valid >> (4 * hf);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (!((vb >> (8 * ii + j)) & 1u)) sc[4 * ii + j] = -INFINITY;
    }
  };
  // online softmax of one tile's scores (lane column = head h0+hl; rows 8ii + 4hf + j are
  // tile positions); returns P^T as the B operand of the value MFMAs: k-slot e < 4 is
  // position 16ks + 4hf + e, e >= 4 is 16ks + 8 + 4hf + e - 4
  auto softmax = [&](const f32x16& sc, bf16x8 (&pf)[2]) {
    float tmax = sc[0];
#pragma unroll
    for (int k = 1; k < 16; ++k) tmax = fmaxf(tmax, sc[k]);
    tmax = half_swap_max(tmax) * c2;  // scale > 0 keeps the order
    const float m_new = fmaxf(m_run, tmax);
    const bool need = m_new > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_use = need ? m_new : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) o[mb] *= alpha;
      m_run = m_use;
    }
    const float msafe = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
    float p[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      p[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[k], c2, -msafe));
      psum += p[k];
    }
    l_run += half_swap_sum(psum);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ks][e] = (__bf16)p[4 * (2 * ks + (e >> 2)) + (e & 3)];
  };
  // values: O^T += C^T . P^T, A from the transpose read of the tile; sixteen MFMAs in eight
  // pairs, the reads of pair g+1 in flight while pair g computes
  auto values = [&](const uint8_t* tile, const bf16x8 (&pf)[2]) {
    s16x4 tv[2][2][2];
    auto load_g = [&](int grp, int buf) {
      const int ks = grp >> 2;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int mb = 2 * (grp & 3) + k;
        const int sh = 256 * (mb >> 2) + 64 * ((mb & 3) ^ tfh) + (16 * ks) * kRowBytes;
        tv[buf][k][0] = lds_read_tr16(tile + tr_b0 + sh);
        tv[buf][k][1] = lds_read_tr16(tile + tr_b1 + sh);
      }
    };
    load_g(0, 0);
#pragma unroll
    for (int grp = 0; grp < 8; ++grp) {
      if (grp + 1 < 8) load_g(grp + 1, (grp + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int mb = 2 * (grp & 3) + k;
        o[mb] = mfma32(concat_bf16(tv[grp & 1][k][0], tv[grp & 1][k][1]), pf[grp >> 2], o[mb]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (ntiles > 0) issue(0);
  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<0>();  // tile t (the only copy in flight) has landed
    __syncthreads();  // ... for every wave; every wave is done with tile t-1
    if (t + 1 < ntiles) issue(t + 1);  // into the stage tile t-1 used
    const uint8_t* tile = smem[t % kStages];
    f32x16 s;
    scores(tile, s);
#pragma unroll
    for (int k = 0; k < 4; ++k) xbuf[wave][k][lane] = (f32x4){s[4 * k], s[4 * k + 1], s[4 * k + 2], s[4 * k + 3]};
    __syncthreads();
    complete_scores(s, valid_rows(t));
    bf16x8 pf[2];
    softmax(s, pf);
    values(tile, pf);
  }

  // ---- results: lane holds head h0+hl, latents 256lh + 32mb + 8ii + 4hf + j
  const int h = h0 + hl;
  if (a.num_splits == 1) {
    const float inv_l = 1.0f / l_run;
    float* orow = a.o_lat + ((size_t)bq * a.H + h) * kLatent + 256 * lh + 4 * hf;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        f32x4 v = {o[mb][4 * ii] * inv_l, o[mb][4 * ii + 1] * inv_l, o[mb][4 * ii + 2] * inv_l,
                   o[mb][4 * ii + 3] * inv_l};
        *(f32x4*)(orow + 32 * mb + 8 * ii) = v;
      }
    // __builtin_amdgcn_logf is the hardware base-2 logarithm
    if (a.lse != nullptr && hf == 0 && lh == 0)
      a.lse[(size_t)bq * a.H + h] = (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f;
  } else {
    const size_t prow_idx = ((size_t)split * a.B * a.Q + bq) * a.H + h;
    float* orow = a.part_o + prow_idx * kLatent + 256 * lh + 4 * hf;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        f32x4 v = {o[mb][4 * ii], o[mb][4 * ii + 1], o[mb][4 * ii + 2], o[mb][4 * ii + 3]};
        *(f32x4*)(orow + 32 * mb + 8 * ii) = v;
      }
    if (hf == 0 && lh == 0) {
      a.part_ml[2 * prow_idx] = m_run;
      a.part_ml[2 * prow_idx + 1] = l_run;
    }
  }
}

// Log-sum-exp merge of the split partials (exact up to rounding: every split's sum is
// rescaled to the common maximum).  One workgroup per (b, i, head); thread t owns latents
// 4t .. 4t+3.
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a) {
  const int row = blockIdx.x;  // (b*Q + i)*H + h
  const int t = threadIdx.x;
  const size_t rows = (size_t)a.B * a.Q * a.H;
  const int S = a.num_splits;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) {
    const float l = a.part_ml[2 * (s * rows + row) + 1];
    if (l > 0.f) M = fmaxf(M, a.part_ml[2 * (s * rows + row)]);
  }
  float Ls = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < S; ++s) {
    const float m = a.part_ml[2 * (s * rows + row)];
    const float l = a.part_ml[2 * (s * rows + row) + 1];
    if (l > 0.f) {
      const float w = __builtin_amdgcn_exp2f(m - M);
      Ls += w * l;
      const f32x4 v = *(const f32x4*)(a.part_o + (s * rows + row) * kLatent + 4 * t);
      acc += w * v;
    }
  }
  const float inv = 1.0f / Ls;
  *(f32x4*)(a.o_lat + (size_t)row * kLatent + 4 * t) = acc * inv;
  if (a.lse != nullptr && t == 0) a.lse[row] = (M + __builtin_amdgcn_logf(Ls)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_latent_attn(const AttnArgs& a, bool indexed, hipStream_t stream) {
  void* args[] = {const_cast<AttnArgs*>(&a)};
  const dim3 grid(a.total_wg), block(kThreads);
  if (indexed) return hipLaunchKernel((const void*)&latent_attn_kernel<true>, grid, block, args, 0, stream);
  return hipLaunchKernel((const void*)&latent_attn_kernel<false>, grid, block, args, 0, stream);
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AttnArgs*>(&a)};
  const dim3 grid(a.B * a.Q * a.H), block(128);
  return hipLaunchKernel((const void*)&combine_kernel, grid, block, args, 0, stream);
}

}  // namespace mla
