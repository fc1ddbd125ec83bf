// Split-K latent attention for gfx950: the scores and the value sum of absorbed MLA computed
// directly on the cached 512-wide latents (page "Module 05 -- MLA: Compressing Per-Token
// History", section 3; colibri "MLA is absorbed").
//
// One workgroup per CU: 512 threads, two subgroups of four waves.  In a subgroup, wave w owns
// heads 32*(w&1) .. +31 of a group of 64 and latents 256*(w>>1) .. +255.  Tiles of 32 cached
// latents (32 KiB) are copied from HBM straight into a four-tile LDS ring with
// global_load_lds_dwordx4, two tiles ahead of use.  Each tile passes two phases per subgroup:
//   A  scores    S^T[32 pos x 32 heads] = C[32 x 512] . Q~^T[512 x 32]: each wave contracts its
//                own 256 latents (16 MFMA 32x32x16; A operand = the tile row-major via
//                ds_read_b128, B operand = the absorbed query held in VGPRs) and posts its
//                partial sum to LDS for the wave holding the other 256 latents
//   B  softmax   add the partner's partial, mask, online softmax per head = per lane column
//                (the running maximum only moves when it grows by more than 2^8, so the
//                accumulator is rarely rescaled); then
//      values    O^T[256 x 32 heads] += C^T[256 x 32 pos] . P^T[32 pos x 32 heads] (16 MFMA;
//                A = the SAME tile read transposed with ds_read_b64_tr_b16, B = P straight
//                from the score registers, the MFMA's K order permuted to match them)
// The subgroups run one phase apart, so between two barriers one subgroup is in phase A
// (matrix core + row reads) while the other is in phase B (VALU + transpose reads + matrix
// core): on every SIMD one wave of each kind.
//   PAIR (dense, several queries): the subgroups take queries 2u and 2u+1 of a sequence over
//        the same tiles, so one copy of a tile serves both.
//   otherwise (one query, or index lists): the subgroups take alternate tiles of one query's
//        split and merge their two partial softmaxes through LDS at the end.
// One latent row serves all 64 heads: the cache is read once per (query pair, split).
#include <type_traits>

#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kTile = kTilePositions;
constexpr int kThreads = 512;
constexpr int kRing = 4;                  // LDS tiles: two in use, two in flight
constexpr int kTileBytes = kTile * kRowBytes;
constexpr int kRowsPerWave = kTile / 4;   // rows each wave of the copying subgroup copies per tile
constexpr float kRescaleLog2 = 8.0f;

// Log-sum-exp merge of the split partials of one output row (b, i, head), exact up to rounding:
// every split's sum is rescaled to the common maximum.  Thread t of a group of 128 owns
// latents 4t .. 4t+3; splits are taken eight at a time with all their loads in flight.
__device__ __forceinline__ void merge_row(const AttnArgs& a, size_t row, int t) {
  const size_t rows = (size_t)a.B * a.Q * a.H;
  const int S = a.num_splits;
  const float* ml = a.part_ml + 2 * row;
  const float* po = a.part_o + row * kLatent + 4 * t;
  float M = -INFINITY;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float mm[8], ll[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = min(s0 + k, S - 1);
      mm[k] = ml[2 * s * rows];
      ll[k] = ml[2 * s * rows + 1];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (ll[k] > 0.f) M = fmaxf(M, mm[k]);
  }
  float Ls = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *(const f32x4*)(po + (size_t)min(s0 + k, S - 1) * rows * kLatent);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int s = min(s0 + k, S - 1);
      const float m = ml[2 * s * rows];
      const float l = ml[2 * s * rows + 1];
      const float w = (s0 + k < S && l > 0.f) ? __builtin_amdgcn_exp2f(m - M) : 0.f;
      Ls += w * l;
      acc += w * v[k];
    }
  }
  const float inv = 1.0f / Ls;
  *(f32x4*)(a.o_lat + row * kLatent + 4 * t) = acc * inv;
  // __builtin_amdgcn_logf is the hardware base-2 logarithm
  if (a.lse != nullptr && t == 0) a.lse[row] = (M + __builtin_amdgcn_logf(Ls)) * 0.69314718055994531f;
}

template <bool INDEXED, bool PAIR>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void latent_attn_kernel(AttnArgs a) {
  static_assert(!(INDEXED && PAIR), "index lists are per query");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing][kTileBytes];
  __shared__ __attribute__((aligned(16))) f32x4 xbuf[2][4][4][64];  // partial scores [subgroup][wave][reg/4][lane]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps it in SGPRs
  const int sg = wave >> 2;       // subgroup
  const int w4 = wave & 3;        // wave within the subgroup
  const int hh = w4 & 1;          // head half of the group
  const int lh = w4 >> 1;         // latent half
  const int wg = xcd_remap(blockIdx.x, a.total_wg);
  // logical order (b, head group, split, query unit): the query units of one split of one
  // sequence are adjacent, so they run on the same XCD and share the tile through its L2
  const int qu = wg % a.q_units;
  int rest = wg / a.q_units;
  const int split = rest % a.num_splits;
  rest /= a.num_splits;
  const int hg = rest % a.HG;
  const int b = rest / a.HG;
  const int i = PAIR ? 2 * qu + sg : qu;  // this subgroup's query
  const bool active = i < a.Q;            // PAIR with odd Q: the last unit has one query
  const int bq = b * a.Q + (active ? i : a.Q - 1);
  const int h0 = hg * 64 + hh * 32;
  const int hl = lane & 31;
  const int hf = lane >> 5;

  const int L = min(a.cache_len[b], a.max_cache_len);
  int n_slots, n_range;  // visible slots of this subgroup's query / of the unit's longest query
  const int32_t* idx_row = nullptr;
  if constexpr (INDEXED) {
    idx_row = a.idx + (size_t)bq * a.K_max;
    n_slots = L > 0 ? min(a.idx_len[bq], a.K_max) : 0;
    n_range = n_slots;
  } else {
    n_slots = active ? L - a.Q + i + 1 : 0;  // positions 0 .. cache_len - Q + i
    n_range = PAIR ? L - a.Q + min(2 * qu + 1, a.Q - 1) + 1 : n_slots;
  }
  n_slots = max(n_slots, 0);
  n_range = max(n_range, 0);
  const int s_begin = split * a.split_len;
  const int s_end = min(s_begin + a.split_len, n_range);
  const int my_end = min(s_begin + a.split_len, n_slots);
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

  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int k = 0; k < 16; ++k) o[mb][k] = 0.f;
  float m_run = -INFINITY;  // running maximum of scale*log2(e)*score
  float l_run = 0.f;        // running sum of 2^(scale*log2(e)*score - m_run)

  // ---- tile loader: tiles are copied by the four waves of one subgroup, wave w4 taking
  // rows 8w4 .. 8w4+7, one 1 KiB row per instruction, lane s of row r taking global chunk
  // s ^ swz(r) into slot s.  Every row read is a visible row: rows past the split repeat its
  // last row and indexed slots naming a position outside the cache read row 0; both are
  // masked out of the scores.  Index lists are read with scalar loads, so waiting for them
  // never waits for tile copies.
  const uint32_t lane16 = (uint32_t)lane << 4;
  const uint32_t lds0 = lds_addr(&smem[0][0]);
  auto issue_row = [&](int t, int rr) {
    const int r = w4 * kRowsPerWave + rr;
    const int slot = s_begin + t * kTile + r;
    const uint32_t dst = lds0 + (t % kRing) * kTileBytes + r * kRowBytes;
    if constexpr (INDEXED) {
      int p = idx_row[min(slot, s_end - 1)];
      p = (p >= 0 && p < L) ? p : 0;
      row_to_lds(seq + (size_t)p * kRowBytes, dst, lane16, (uint32_t)(swz(r) << 4));
    } else {
      // positions are consecutive: one base per tile, the row as a byte offset
      const int first = s_begin + t * kTile;
      const int row = min(r, s_end - 1 - first);
      row_to_lds_at(seq + (size_t)first * kRowBytes, (uint32_t)(row * kRowBytes), dst, lane16,
                    (uint32_t)(swz(r) << 4));
    }
  };
  // rows of tile t that hold a position visible to this subgroup's query (bit r = tile row r)
  auto valid_rows = [&](int t) -> uint32_t {
    const int base = s_begin + t * kTile;
    const int nvalid = my_end - base;
    uint32_t v = nvalid >= kTile ? 0xffffffffu : (nvalid <= 0 ? 0u : ((1u << nvalid) - 1u));
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
  // With ks = 8u + v, the chunk offset ((2v + hf) ^ psw) << 4 equals ((v ^ p7) << 5) + x16,
  // p7 = psw >> 1, x16 = (hf ^ (psw & 1)) << 4: one xor and one shift-add per v on top of a
  // per-tile base, the 256-byte step of u folded into the instruction offset.
  const int qk_p7 = psw >> 1;
  const int qk_lane = qk_base + ((hf ^ (psw & 1)) << 4);
  // dma >= 0: also copy this wave's eight rows of tile `dma`, one row per two MFMAs; the
  // reads run three MFMAs ahead
  auto scores = [&](const uint8_t* tile, f32x16& sc, int dma) {
    const int p7 = opaque(qk_p7);
    const uint8_t* rb = tile + qk_lane;
    auto rd = [&](int ks) { return *(const bf16x8*)(rb + 256 * (ks >> 3) + (((ks & 7) ^ p7) << 5)); };
#pragma unroll
    for (int k = 0; k < 16; ++k) sc[k] = 0.f;
    bf16x8 av[4];
    av[0] = rd(0);
    av[1] = rd(1);
    av[2] = rd(2);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) {
      if (ks + 3 < 16) av[(ks + 3) % 4] = rd(ks + 3);
      if ((ks & 1) == 0 && dma >= 0) issue_row(dma, ks >> 1);
      __builtin_amdgcn_sched_barrier(0);
      sc = mfma32(av[ks % 4], qf[ks], sc);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // add the partner's partial (same heads, other latents) and mask rows past the visible set
  auto complete_scores = [&](f32x16& sc, uint32_t valid) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 x = xbuf[sg][w4 ^ 2][k][lane];
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
    // reductions as trees: four dependent steps instead of fifteen
    float mx[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) mx[k] = fmaxf(sc[k], sc[k + 8]);
#pragma unroll
    for (int k = 0; k < 4; ++k) mx[k] = fmaxf(mx[k], mx[k + 4]);
    float tmax = fmaxf(fmaxf(mx[0], mx[2]), fmaxf(mx[1], mx[3]));
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
    float p[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) p[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[k], c2, -msafe));
    float ps[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) ps[k] = p[k] + p[k + 8];
#pragma unroll
    for (int k = 0; k < 4; ++k) ps[k] = ps[k] + ps[k + 4];
    l_run += half_swap_sum((ps[0] + ps[2]) + (ps[1] + ps[3]));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[ks][e] = (__bf16)p[4 * (2 * ks + (e >> 2)) + (e & 3)];
  };
  // values: O^T += C^T . P^T, A from the transpose read of the tile; MFMA n covers latent
  // block mb = n & 7 and k-step ks = n >> 3, its reads issued two MFMAs ahead
  auto values = [&](const uint8_t* tile, const bf16x8 (&pf)[2]) {
    const int fh = opaque(tfh);
    const uint8_t* t0 = tile + tr_b0;
    const uint8_t* t1 = tile + tr_b1;
    s16x4 tv[2][2];
    auto load = [&](int n, int slot) {
      const int ks = n >> 3, mb = n & 7;
      const int sh = 256 * (mb >> 2) + 64 * ((mb & 3) ^ fh) + (16 * ks) * kRowBytes;
      tv[slot][0] = lds_read_tr16(t0 + sh);
      tv[slot][1] = lds_read_tr16(t1 + sh);
    };
    load(0, 0);
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      if (n + 1 < 16) load(n + 1, (n + 1) % 2);
      __builtin_amdgcn_sched_barrier(0);
      o[n & 7] = mfma32(concat_bf16(tv[n % 2][0], tv[n % 2][1]), pf[n >> 3], o[n & 7]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the interval loop.  One barrier opens every interval.  Subgroup sg runs phase A of
  // its j-th tile in interval 2j + sg and phase B in the next one; its j-th tile is tile j
  // (PAIR) or tile 2j + sg.  Tile t is first used in interval t (alternating tiles) or 2t
  // (PAIR).  The waves in phase A copy the tile two ahead of theirs, into the stage whose
  // last use ended with the previous interval: alternating, subgroup k&1 copies tile k+2 in
  // interval k; PAIR, subgroup 0 copies tile m+2 in interval 2m.  A copying wave waits for
  // its own rows of a tile just before the interval that first uses it opens.
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (t < ntiles)
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave / 2; ++rr) {
        // both subgroups share the first two copies: wave w takes rows 4w .. 4w+3
        const int r = wave * (kRowsPerWave / 2) + rr;
        const int slot = s_begin + t * kTile + r;
        int p;
        if constexpr (INDEXED) {
          p = idx_row[min(slot, s_end - 1)];
          p = (p >= 0 && p < L) ? p : 0;
        } else {
          p = min(slot, s_end - 1);
        }
        row_to_lds(seq + (size_t)p * kRowBytes, lds0 + t * kTileBytes + r * kRowBytes, lane16,
                   (uint32_t)(swz(r) << 4));
      }
  // waiting for the query loads and the first copies here leaves the loop's waits counting
  // tile copies only (the compiler's own wait for the query registers is then satisfied)
  wait_vmcnt<0>();
  auto open_interval = [&](int k) {
    if constexpr (PAIR) {
      const int m = k >> 1;  // tile first used now (k even); subgroup 0 copied it in interval k-4
      if (sg == 0 && (k & 1) == 0 && m < ntiles) {
        if (m + 1 < ntiles) wait_vmcnt<kRowsPerWave>();  // tile m+1 (interval k-2) may stay in flight
        else wait_vmcnt<0>();
      }
    } else {
      // tile k, copied in interval k-2 by subgroup k&1, which has copied nothing since
      if (sg == (k & 1) && k < ntiles) wait_vmcnt<0>();
    }
    __syncthreads();  // the copies are visible to all; the previous interval is done
  };
  // both subgroups pass the same number of barriers: J iterations of two, plus one
  const int J = PAIR ? ntiles : (ntiles + 1) / 2;
  if (sg == 1) open_interval(0);
  for (int j = 0; j < J; ++j) {
    const int t = PAIR ? j : 2 * j + sg;
    const bool have = active && t < ntiles;
    const uint8_t* tile = smem[t % kRing];
    open_interval(2 * j + sg);
    f32x16 s;
    if (have) {
      const bool copies = PAIR ? sg == 0 : true;
      scores(tile, s, (copies && t + 2 < ntiles) ? t + 2 : -1);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xbuf[sg][w4][q][lane] = (f32x4){s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
    }
    open_interval(2 * j + sg + 1);
    if (have) {
      complete_scores(s, valid_rows(t));
      bf16x8 pf[2];
      softmax(s, pf);
      values(tile, pf);
    }
  }
  if (sg == 0) open_interval(2 * J);

  // ---- results: lane holds head h0+hl, latents 256lh + 32mb + 8ii + 4hf + j
  const int h = h0 + hl;
  // MBLO: first latent block written (a compile-time constant: the accumulator array must be
  // indexed by constants to stay in registers)
  auto write_out = [&](auto mblo_c, bool write_ml) {
    constexpr int mb_lo = decltype(mblo_c)::value;
    if (a.num_splits == 1) {
      const float inv_l = 1.0f / l_run;
      float* orow = a.o_lat + ((size_t)bq * a.H + h) * kLatent + 256 * lh + 4 * hf;
#pragma unroll
      for (int mb = mb_lo; mb < mb_lo + (PAIR ? 8 : 4); ++mb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          f32x4 v = {o[mb][4 * ii] * inv_l, o[mb][4 * ii + 1] * inv_l, o[mb][4 * ii + 2] * inv_l,
                     o[mb][4 * ii + 3] * inv_l};
          *(f32x4*)(orow + 32 * mb + 8 * ii) = v;
        }
      // __builtin_amdgcn_logf is the hardware base-2 logarithm
      if (write_ml && a.lse != nullptr && hf == 0 && lh == 0)
        a.lse[(size_t)bq * a.H + h] = (m_run + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f;
    } else {
      const size_t prow_idx = ((size_t)split * a.B * a.Q + bq) * a.H + h;
      float* orow = a.part_o + prow_idx * kLatent + 256 * lh + 4 * hf;
#pragma unroll
      for (int mb = mb_lo; mb < mb_lo + (PAIR ? 8 : 4); ++mb)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          f32x4 v = {o[mb][4 * ii], o[mb][4 * ii + 1], o[mb][4 * ii + 2], o[mb][4 * ii + 3]};
          *(f32x4*)(orow + 32 * mb + 8 * ii) = v;
        }
      if (write_ml && hf == 0 && lh == 0) {
        a.part_ml[2 * prow_idx] = m_run;
        a.part_ml[2 * prow_idx + 1] = l_run;
      }
    }
  };
  if constexpr (PAIR) {
    if (active) write_out(std::integral_constant<int, 0>{}, true);
  } else {
    // merge the two subgroups' partial softmaxes (same query, heads and latents, disjoint
    // tiles): subgroup 0 finishes latent blocks mb 0-3, subgroup 1 blocks 4-7; each hands the
    // other its half through the (now free) tile ring, and (m, l) through the exchange buffer
    __syncthreads();
    f32x4* xo = (f32x4*)&smem[0][0];  // [w4][subgroup][16][64] f32x4 = 128 KiB
    float* xml = (float*)&xbuf[0][0][0][0];
    const int other = sg ^ 1;
    // GIVE: the blocks handed over; TAKE: the blocks finished here
    auto merge = [&](auto give_c) {
      constexpr int give = decltype(give_c)::value, take = 4 - give;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          xo[((w4 * 2 + sg) * 16 + 4 * mb + q) * 64 + lane] =
              (f32x4){o[give + mb][4 * q], o[give + mb][4 * q + 1], o[give + mb][4 * q + 2], o[give + mb][4 * q + 3]};
      xml[wave * 64 + lane] = m_run;
      xml[512 + wave * 64 + lane] = l_run;
      __syncthreads();
      const float m_o = xml[(other * 4 + w4) * 64 + lane];
      const float l_o = xml[512 + (other * 4 + w4) * 64 + lane];
      const float M = fmaxf(m_run, m_o);
      const float ws = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - M);
      const float wo = m_o == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_o - M);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 x = xo[((w4 * 2 + other) * 16 + 4 * mb + q) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[take + mb][4 * q + e] = o[take + mb][4 * q + e] * ws + x[e] * wo;
        }
      l_run = l_run * ws + l_o * wo;
      m_run = M;
      write_out(std::integral_constant<int, take>{}, give == 4);
    };
    if (sg == 0)
      merge(std::integral_constant<int, 4>{});
    else
      merge(std::integral_constant<int, 0>{});
  }
}

// Merge of the split partials: one workgroup of 128 threads per (b, i, head).
__global__ __launch_bounds__(128) void combine_kernel(AttnArgs a) { merge_row(a, blockIdx.x, threadIdx.x); }

}  // namespace

hipError_t launch_latent_attn(const AttnArgs& a, bool indexed, hipStream_t stream) {
  void* args[] = {const_cast<AttnArgs*>(&a)};
  const dim3 grid(a.total_wg), block(kThreads);
  const void* k;
  if (indexed)
    k = (const void*)&latent_attn_kernel<true, false>;
  else if (a.q_units < a.Q)
    k = (const void*)&latent_attn_kernel<false, true>;
  else
    k = (const void*)&latent_attn_kernel<false, false>;
  return hipLaunchKernel(k, grid, block, args, 0, stream);
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AttnArgs*>(&a)};
  const dim3 grid(a.B * a.Q * a.H), block(128);
  return hipLaunchKernel((const void*)&combine_kernel, grid, block, args, 0, stream);
}

}  // namespace mla
