// Split-K latent attention for gfx950: the scores and the value sum of absorbed MLA computed
// directly on the cached 512-wide latents (page "Module 05 -- MLA: Compressing Per-Token
// History", section 3; colibri "MLA is absorbed").
//
// One workgroup = one (sequence b, query i, group of 64 heads, split of positions); four
// waves, wave w owning heads 32*(w&1) .. +31 of the group and latents 256*(w>>1) .. +255.
// Per tile of 32 cached latents (32 KiB, staged in LDS straight from HBM with
// global_load_lds_dwordx4, double-buffered):
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
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kTile = kTilePositions;
constexpr int kStages = 2;
constexpr int kThreads = 256;
constexpr float kRescaleLog2 = 8.0f;

template <bool INDEXED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void latent_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kStages][kTile * kRowBytes];
  __shared__ __attribute__((aligned(16))) float xbuf[4][16][64];  // partial scores, [wave][reg][lane]

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

  // absorbed query of head h0+hl as the B operand: latents 256lh + 16ks + 8hf .. +7
  bf16x8 qf[16];
  {
    const uint16_t* qrow = a.q_abs + ((size_t)bq * a.H + h0 + hl) * kLatent + 256 * lh + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qf[ks] = *(const bf16x8*)(qrow + 16 * ks);
  }

  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int k = 0; k < 16; ++k) o[mb][k] = 0.f;
  float m_run = -INFINITY;  // running maximum of scale*log2(e)*score
  float l_run = 0.f;        // running sum of 2^(s - m_run)

  // ---- tile loader: wave w copies tile rows 8w .. 8w+7, one 1 KiB row per instruction;
  // lane s of row r takes global chunk s ^ swz(r) into slot s (swz(r) depends on r mod 8 only).
  // Rows past the split are clamped to its last valid row (read, then masked out), so every
  // read stays inside the visible rows; indexed slots that name a position outside the cache
  // read row 0 instead and are masked.
  uint32_t voff[8];
#pragma unroll
  for (int rr = 0; rr < 8; ++rr) voff[rr] = (uint32_t)((lane ^ swz(rr)) << 4);
  const uint32_t lds0 = lds_addr(&smem[0][0]);
  int idx_next = -1;  // indexed: the position of tile row (lane & 31) of the next tile to issue
  auto fetch_idx = [&](int t) {
    if constexpr (INDEXED) {
      const int s = s_begin + t * kTile + (lane & 31);
      idx_next = (t < ntiles && s < s_end) ? idx_row[s] : -1;
    }
  };
  auto issue = [&](int t, int stage) -> uint32_t {
    const uint32_t dst = lds0 + stage * (kTile * kRowBytes) + wave * 8 * kRowBytes;
    const int base = s_begin + t * kTile;
    uint32_t valid;
    if constexpr (INDEXED) {
      const bool ok = idx_next >= 0 && idx_next < L;
      const int rp = ok ? idx_next : 0;
      valid = (uint32_t)__builtin_amdgcn_ballot_w64(ok);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int p = __builtin_amdgcn_readlane(rp, wave * 8 + rr);
        row_to_lds(seq + (size_t)p * kRowBytes, dst + rr * kRowBytes, voff[rr]);
      }
    } else {
      const int nvalid = s_end - base;
      valid = nvalid >= 32 ? 0xffffffffu : ((1u << nvalid) - 1u);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const int p = min(base + wave * 8 + rr, s_end - 1);
        row_to_lds(seq + (size_t)p * kRowBytes, dst + rr * kRowBytes, voff[rr]);
      }
    }
    return valid;
  };

  // ---- per-lane LDS addressing (byte offsets inside a stage)
  // scores: A row = tile row (lane & 31), global chunk 32lh + 2ks + hf, stored at
  // chunk ^ swz(row); with ks = 4u + v that is 32lh + 8u + ((2v + hf) ^ swz(row))
  const int prow = lane & 31;
  const int psw = swz(prow);
  int qk_off[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) qk_off[v] = prow * kRowBytes + 512 * lh + (((2 * v + hf) ^ psw) << 4);
  // values: transpose read; group g = lane / 16 supplies rows 4(g/2) + e (+16ks + 8r2) and
  // latent columns 256lh + 32mb + 16(g&1) + 4c; the chunk 32lh + 4mb + x is stored at
  // 32lh + 4 (mb ^ sb) + (x ^ (sw & 3)), sb = sw >> 2
  const int g = lane >> 4, ip = lane & 15, te = ip >> 2, tc = ip & 3;
  const int trow = 4 * (g >> 1) + te;
  const int tsw = swz(trow);
  const int tx = (2 * (g & 1) + (tc >> 1)) ^ (tsw & 3);
  const int tsb = tsw >> 2;
  const int tr_base = trow * kRowBytes + 512 * lh + (tx << 4) + ((tc & 1) << 3);
  const int tr_even = tr_base + 64 * tsb;
  const int tr_odd = tr_base - 64 * tsb;

  uint32_t valid_cur = 0, valid_next = 0;
  if (ntiles > 0) {
    fetch_idx(0);
    valid_cur = issue(0, 0);
    fetch_idx(1);
  }

  for (int t = 0; t < ntiles; ++t) {
    wait_vmcnt<0>();
    __syncthreads();  // tile t is in LDS for every wave; all are done with tile t-1
    if (t + 1 < ntiles) {
      valid_next = issue(t + 1, (t + 1) & 1);
      fetch_idx(t + 2);
    }
    const uint8_t* tile = smem[t & 1];

    // ---- partial scores over this wave's 256 latents
    f32x16 s;
#pragma unroll
    for (int k = 0; k < 16; ++k) s[k] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      const bf16x8 av = *(const bf16x8*)(tile + qk_off[ks & 3] + 128 * (ks >> 2));
      s = mfma32(av, qf[ks], s);
    }
    // swap halves with the partner wave (same heads, other latents) and add
#pragma unroll
    for (int k = 0; k < 16; ++k) xbuf[wave][k][lane] = s[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) s[k] += xbuf[wave ^ 2][k][lane];

    // ---- online softmax (lane column = head h0+hl; rows 8ii + 4hf + j = tile positions)
    float tmax = -INFINITY;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 8 * ii + 4 * hf + j;
        const float x = ((valid_cur >> r) & 1u) ? s[4 * ii + j] * a.scale_log2 : -INFINITY;
        s[4 * ii + j] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const bool need = m_new > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_use = need ? m_new : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int k = 0; k < 16; ++k) o[mb][k] *= alpha;
      m_run = m_use;
    }
    const float msafe = (m_run == -INFINITY) ? 0.f : m_run;
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float p = __builtin_amdgcn_exp2f(s[k] - msafe);
      s[k] = p;
      psum += p;
    }
    psum += __shfl_xor(psum, 32);
    l_run += psum;

    // P^T as the B operand: k-slot e < 4 -> position 16ks + 4hf + e, e >= 4 -> 16ks + 8 + 4hf + e-4
    bf16x8 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ks][e] = (__bf16)s[4 * (2 * ks + (e >> 2)) + (e & 3)];

    // ---- values: O^T += C^T . P^T, A from the transpose read of the same tile
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const int base = (mb & 1) ? tr_odd : tr_even;
        const uint8_t* p0 = tile + base + 64 * mb + (16 * ks) * kRowBytes;
        const s16x4 lo = lds_read_tr16(p0);
        const s16x4 hi = lds_read_tr16(p0 + 8 * kRowBytes);
        o[mb] = mfma32(concat_bf16(lo, hi), pf[ks], o[mb]);
      }
    }
    valid_cur = valid_next;
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
