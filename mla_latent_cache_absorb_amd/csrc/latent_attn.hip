// Split-K latent attention for gfx950: the scores and the value sum of absorbed MLA computed
// directly on the cached 512-wide latents (page "Module 05 -- MLA: Compressing Per-Token
// History", section 3; colibri "MLA is absorbed").
//
// One workgroup = one (sequence b, query i, group of 64 heads, split of positions), one per
// CU: 768 threads in twelve waves with two roles.  Tiles of 32 cached latents (32 KiB) are
// copied from HBM straight into a four-tile LDS ring with global_load_lds_dwordx4, two tiles
// ahead of use; one barrier opens each step.
//   score waves (0-3), wave s owning heads 16s .. 16s+15 of the group, in step t on tile t:
//     S^T[32 pos x 16 heads] = C[32 x 512] . Q~^T[512 x 16] over all 512 latents (32 MFMA
//     16x16x32; A operand = tile rows via ds_read_b128, B operand = the absorbed query held in
//     VGPRs for the whole kernel); online softmax per head (the running maximum moves only
//     when it grows by more than 2^8, so the accumulators are rarely rescaled); P is posted
//     to LDS in bf16 with the step's rescale factor
//   value waves (4-11), wave 4+v owning heads 32(v>>2) .. +31 and latents 128(v&3) .. +127,
//     in step t on tile t-1: O^T[128 x 32 heads] = O^T * alpha + C^T[128 x 32 pos] .
//     P^T[32 pos x 32 heads] (8 MFMA 32x32x16; A operand = the same tile read transposed with
//     ds_read_b64_tr_b16, B operand = P from LDS); they also copy the tiles, four rows each
// Each SIMD runs one score wave and two value waves, so its matrix core has work from both
// halves of the computation while either role waits on LDS, and no wave holds both the
// query registers and the accumulators.  One latent row serves all 64 heads: the cache is read
// once per (query, split); the queries of one split are placed on one XCD and share the tiles
// through its L2.  With several splits, each workgroup ends by staging its normalised partial in
// the idle tile ring and storing it as whole contiguous KiB (stage_value_rows,
// copy_partial_block).  Head counts that are not a multiple of 64 leave the last group partial:
// its missing heads reuse the last head's query and nothing of theirs is stored.
//
// Indexed calls gather the listed rows instead of a run of positions: each value wave stages its
// rows' index slots in LDS ahead of use (copied like the tiles, so no load waits on memory inside
// the loop) and posts each row's validity for the score waves' mask.
//
// Dense calls with an even number of queries per sequence use latent_attn_pair_kernel instead:
// the same twelve waves take two adjacent queries over one run of tiles, so that each LDS read of
// a tile feeds twice the matrix work (the single-query form is bound by its LDS traffic).
//
// A call given the absorbed query in two bf16 terms (q_abs + q_abs_lo, the second the rounding
// remainder of the first) runs the single-query form for every query: each score wave holds both
// terms and each tile read feeds two MFMAs into the same accumulator, so the scores see the query
// to about 2^-17 of its size instead of bf16's 2^-9.
//
// The split partials (m, l, u = o / l) are merged by log-sum-exp (merge_splits8): combine_kernel
// for up to eight splits, combine_wide_kernel above that (one thread group per group of eight
// splits), or the fused merge and up-projection of mla_latent_attn_up_v; all three give the same
// bits.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kTile = kTilePositions;
constexpr int kThreads = 768;
constexpr int kRing = 4;                  // LDS tiles: two in use, two in flight
constexpr int kTileBytes = kTile * kRowBytes;
constexpr int kRowsPerVWave = kTile / 8;  // rows each value wave copies per tile
constexpr int kPStride = 80;              // bytes per head in the P buffer: 32 bf16 + padding
constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum over the four lanes l, l^16, l^32, l^48 (one head's column of a 16x16 MFMA result)
__device__ __forceinline__ float quad_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  return half_swap_max(x);
}
__device__ __forceinline__ float quad_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  return half_swap_sum(x);
}

// Largest of this lane's eight scores of a tile and those of the other three lanes of its head
// (one column of the two 16x16 score blocks), times scale * log2(e).
__device__ __forceinline__ float tile_max(const float (&v)[8], float c2) {
  const float m = fmaxf(fmaxf(fmaxf(v[0], v[4]), fmaxf(v[1], v[5])), fmaxf(fmaxf(v[2], v[6]), fmaxf(v[3], v[7])));
  return quad_max(m) * c2;
}

// One tile of the online softmax for this lane's head (scale > 0 keeps the order of the maxima):
// the running maximum m_run (scale * log2(e) units) moves only when it grows by more than
// 2^kRescaleLog2, so the accumulators are rarely rescaled; p receives 2^(v c2 - m_run) and l_run
// their sum over the head's four lanes.  Returns the factor the head's accumulated values must be
// rescaled by.
__device__ __forceinline__ float softmax_step(const float (&v)[8], float tmax, float c2, float& m_run, float& l_run,
                                              float (&p)[8]) {
  const float m_new = fmaxf(m_run, tmax);
  const bool need = m_new > m_run + kRescaleLog2;
  float alpha = 1.f;
  if (__builtin_amdgcn_ballot_w64(need)) {
    const float m_use = need ? m_new : m_run;
    alpha = need ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.0f;
    l_run *= alpha;
    m_run = m_use;
  }
  const float msafe = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[k], c2, -msafe));
  l_run += quad_sum(((p[0] + p[4]) + (p[1] + p[5])) + ((p[2] + p[6]) + (p[3] + p[7])));
  return alpha;
}

// P of one head in bf16 at prow (its row, plus 8 bytes per lane group G).  Lane G holds positions
// 16 blk + 4jj + G; a 4 x 4 transpose across the lanes G = 0..3 of the head (pairs G^1 swapped
// first, then G^2) gives it positions 16 blk + 4G + jj, four consecutive entries of the row.
__device__ __forceinline__ void store_p_row(uint8_t* prow, const float (&p)[8]) {
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    unsigned u[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) u[jj] = __builtin_bit_cast(unsigned, p[4 * blk + jj]);
    auto r01 = __builtin_amdgcn_permlane16_swap(u[0], u[1], false, false);
    auto r23 = __builtin_amdgcn_permlane16_swap(u[2], u[3], false, false);
    auto r02 = __builtin_amdgcn_permlane32_swap(r01[0], r23[0], false, false);
    auto r13 = __builtin_amdgcn_permlane32_swap(r01[1], r23[1], false, false);
    s16x4 pv;
    pv[0] = __builtin_bit_cast(short, (__bf16)__builtin_bit_cast(float, (unsigned)r02[0]));
    pv[1] = __builtin_bit_cast(short, (__bf16)__builtin_bit_cast(float, (unsigned)r13[0]));
    pv[2] = __builtin_bit_cast(short, (__bf16)__builtin_bit_cast(float, (unsigned)r02[1]));
    pv[3] = __builtin_bit_cast(short, (__bf16)__builtin_bit_cast(float, (unsigned)r13[1]));
    *(s16x4*)(prow + 32 * blk) = pv;
  }
}

// Byte offsets, within a tile, of a value wave's transposed A-operand reads for latents 128lq ..
// (lane l: latent l % 32 of a 32-latent block, positions 8(l/32) .. +7 of a 16-position k-step):
// in each 16-lane group g, lane 4e + q names tile row base + e, latents 16(g&1) + 4q .. +3, and
// receives latent 16(g&1) + (lane & 15) of rows base .. base+3; rows 8(g>>1) + e (k-slots 0-3)
// and +4 (k-slots 4-7).  With the swizzle swz(r) = 4(r & 3) + ((r >> 2) & 3), latent block mb of
// quarter lq sits at byte 256lq + 64(mb ^ e) + 16(x ^ f) + 8(q & 1), x = 2(g&1) + (q >> 1),
// f = (row >> 2) & 3; te = e selects the block order.
struct TrOffsets {
  int tb0, tb1, te;
};
__device__ __forceinline__ TrOffsets transpose_offsets(int lane, int lq) {
  const int g = lane >> 4, ip = lane & 15, te = ip >> 2, tq = ip & 3;
  const int x = 2 * (g & 1) + (tq >> 1);
  const int row0 = 8 * (g >> 1) + te, row1 = row0 + 4;
  return {row0 * kRowBytes + 256 * lq + ((x ^ ((row0 >> 2) & 3)) << 4) + ((tq & 1) << 3),
          row1 * kRowBytes + 256 * lq + ((x ^ ((row1 >> 2) & 3)) << 4) + ((tq & 1) << 3), te};
}

// A value wave's result for one head column hv of row bq with one split: o_lat = o / l and
// lse = (m + log2 l) ln 2 are final.  The lane holds latents 128lq + 32mb + 8ii + 4hf + j.
__device__ __forceinline__ void store_value_rows(const AttnArgs& a, int bq, int hv, int lq, int hf, float m_fin,
                                                 float l_fin, const f32x16 (&o)[4]) {
  const float inv_l = 1.0f / l_fin;
  float* orow = a.o_lat + ((size_t)bq * a.H + hv) * kLatent + 128 * lq + 4 * hf;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
      *(f32x4*)(orow + 32 * mb + 8 * ii) = (f32x4){o[mb][4 * ii] * inv_l, o[mb][4 * ii + 1] * inv_l,
                                                  o[mb][4 * ii + 2] * inv_l, o[mb][4 * ii + 3] * inv_l};
  // __builtin_amdgcn_logf is the hardware base-2 logarithm
  if (a.lse != nullptr && hf == 0 && lq == 0)
    a.lse[(size_t)bq * a.H + hv] = (m_fin + __builtin_amdgcn_logf(l_fin)) * 0.69314718055994531f;
}

// A workgroup's split partial (several splits): the value waves stage the normalised fp16 rows
// (64 per query) in LDS, in the tile ring, idle once the loop is over; then every thread copies
// them out as 16-byte chunks, each wave instruction one contiguous KiB, since the 64 heads of a
// query are 64 consecutive rows of part_o.  Written straight from the accumulators, each store
// instruction would put 16 bytes into each of 32 rows.  Staged rows are 1 KiB apart, chunk c of
// row r at chunk position c ^ (r & 63): the staging writes of the 32 rows a wave holds then fall
// in different banks, and a row read back stays one KiB.
__device__ __forceinline__ void stage_value_rows(uint8_t* stage, int srow, int lq, int hf, float l_fin,
                                                 const f32x16 (&o)[4]) {
  const float inv_l = l_fin > 0.f ? 1.0f / l_fin : 0.f;
  uint8_t* rowp = stage + srow * kRowBytes + 8 * hf;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int chunk = 16 * lq + 4 * mb + ii;  // latents 8 chunk .. +7; this lane's four at + 4 hf
      *(f16x4*)(rowp + 16 * (chunk ^ (srow & 63))) =
          __builtin_convertvector((f32x4){o[mb][4 * ii] * inv_l, o[mb][4 * ii + 1] * inv_l,
                                          o[mb][4 * ii + 2] * inv_l, o[mb][4 * ii + 3] * inv_l}, f16x4);
    }
}
// every thread of the workgroup, after the staging writes and a barrier: staged rows srow0 ..
// srow0 + nrows - 1 (the group's heads, fewer than 64 in a last partial group) to part_o rows
// first .., and their (m, l) from m_row / l_row
__device__ __forceinline__ void copy_partial_block(const AttnArgs& a, size_t first, int nrows, const uint8_t* stage,
                                                   int srow0, const float* m_row, const float* l_row) {
  uint16_t* dst = a.part_o + first * kLatent;
  for (int c = threadIdx.x; c < nrows * 64; c += kThreads) {
    const int h = c >> 6, k = c & 63, r = srow0 + h;
    *(int4*)(dst + h * kLatent + 8 * k) = *(const int4*)(stage + r * kRowBytes + 16 * (k ^ (r & 63)));
  }
  if ((int)threadIdx.x < nrows)
    *(float2*)(a.part_ml + 2 * (first + threadIdx.x)) = float2{m_row[threadIdx.x], l_row[threadIdx.x]};
}

// LO: the absorbed query comes as two bf16 terms (q_abs + q_abs_lo) and each score takes both
// products into one fp32 accumulator.  NT: the tile copies are non-temporal (no other workgroup of
// the call reads these rows).
template <bool INDEXED, bool LO, bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void latent_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][64 * kPStride];  // P [head][pos] bf16
  __shared__ float abuf[2][64];                                            // rescale factor per head
  __shared__ float mlbuf[2][64];                                           // final (m, l) per head
  // indexed calls: each value wave's index slots for 16 tiles at a time (double-buffered), and a
  // byte per tile row telling the score waves whether its listed position is inside the cache
  __shared__ __attribute__((aligned(16))) int32_t ibuf[INDEXED ? 8 : 1][2][64];
  __shared__ __attribute__((aligned(16))) uint8_t vrow[INDEXED ? kRing : 1][kTile];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: keeps it in SGPRs
  const int wg = xcd_remap(blockIdx.x, a.total_wg);
  // logical order (b, head group, split, query): the queries of one split of one sequence are
  // adjacent, so they run on the same XCD and share the tile through its L2
  const int i = a.Q - 1 - wg % a.Q;  // later queries see more positions: they start first
  int rest = wg / a.Q;
  const int split = rest % a.num_splits;
  rest /= a.num_splits;
  const int hg = rest % a.HG;
  const int b = rest / a.HG;
  const int bq = b * a.Q + i;

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
  const uint32_t lane16 = (uint32_t)lane << 4;
  const uint32_t lds0 = lds_addr(&smem[0][0]);

  if (wave < 4) {
    // ======================= score waves =======================
    const int s = wave;
    const int c = lane & 15, G = lane >> 4;  // head 16s + c; k / row group G
    const int h = min(hg * 64 + 16 * s + c, a.H - 1);  // a partial group's missing heads reuse the last
    const float c2 = a.scale_log2;
    // absorbed query as the B operand: latents 32ks + 8G .. +7 (and its second term with LO)
    bf16x8 qf[16], ql[LO ? 16 : 1];
    {
      const size_t qoff = ((size_t)bq * a.H + h) * kLatent + 8 * G;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[ks] = *(const bf16x8*)(a.q_abs + qoff + 32 * ks);
      if constexpr (LO) {
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) ql[ks] = *(const bf16x8*)(a.q_abs_lo + qoff + 32 * ks);
      }
    }
    float m_run = -INFINITY;  // running maximum of scale*log2(e)*score (this lane's head)
    float l_run = 0.f;        // running sum of 2^(scale*log2(e)*score - m_run)
    // A operand: MFMA row m = lane & 15 of block blk reads tile row 16 blk + 4(m & 3) + (m >> 2)
    // (rows transposed within each 16, for which swz(row) = m: the sixteen lanes of a read then
    // fall in distinct LDS banks), chunk 4ks + G, stored at chunk ^ m =
    // 16(ks >> 2) + 4((ks & 3) ^ (m >> 2)) + (G ^ (m & 3)).  Result register jj of block blk
    // therefore holds tile position 16 blk + 4jj + G.
    const int qk_lane = (4 * (c & 3) + (c >> 2)) * kRowBytes + ((G ^ (c & 3)) << 4);
    const int qk_hi = c >> 2;
    wait_vmcnt<0>();
    __syncthreads();  // the first two tiles have landed (copied by the value waves)

    for (int t = 0; t <= ntiles; ++t) {
      // the previous step's P and rescale factors must be in LDS before the value waves pass
      // this barrier: the compiler places no LDS wait before a barrier reached along the loop's
      // back edge, so it is made explicit
      wait_lds_reads();
      __syncthreads();  // step t opens: tile t is in LDS; the value waves read P of step t-1
      if (t == ntiles) break;
      const uint8_t* rb = smem[t % kRing] + qk_lane;
      const int hi = opaque(qk_hi);
      auto rd = [&](int n) {  // n = 2 ks + block
        const int ks = n >> 1;
        return *(const bf16x8*)(rb + 16 * kRowBytes * (n & 1) + 256 * (ks >> 2) + (((ks & 3) ^ hi) << 6));
      };
      f32x4 sc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      // reads in flight ahead of the MFMA that consumes them (with LO each read feeds two MFMAs,
      // and the second query term leaves registers for two)
      constexpr int kAhead = LO ? 2 : 7;
      bf16x8 av[kAhead + 1];
#pragma unroll
      for (int n = 0; n < kAhead; ++n) av[n] = rd(n);
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        if (n + kAhead < 32) av[(n + kAhead) % (kAhead + 1)] = rd(n + kAhead);
        __builtin_amdgcn_sched_barrier(0);
        sc[n & 1] = mfma16(av[n % (kAhead + 1)], qf[n >> 1], sc[n & 1]);
        if constexpr (LO) sc[n & 1] = mfma16(av[n % (kAhead + 1)], ql[n >> 1], sc[n & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // lane holds positions 16 blk + 4jj + G of head c; mask those past the visible set
      float v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) v[k] = sc[k >> 2][k & 3];
      {
        const int base = s_begin + t * kTile;
        const int nvalid = s_end - base;
        uint32_t valid = nvalid >= kTile ? 0xffffffffu : ((1u << nvalid) - 1u);
        if constexpr (INDEXED) {
          // row validity posted by the value waves when they copied this tile (two steps ago): lane
          // l reads row l & 31's byte, and the wave's ballot is the tile's mask (bit r = row r)
          const bool ok = vrow[t % kRing][lane & 31] != 0;
          valid &= (uint32_t)__builtin_amdgcn_ballot_w64(ok);
        }
        if (valid != 0xffffffffu) {
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (!((valid >> (16 * (k >> 2) + 4 * (k & 3) + G)) & 1u)) v[k] = -INFINITY;
        }
      }
      float p[8];
      const float alpha = softmax_step(v, tile_max(v, c2), c2, m_run, l_run, p);
      store_p_row(pbuf[t & 1] + (16 * s + c) * kPStride + 8 * G, p);  // P row of head 16s + c
      if (G == 0) abuf[t & 1][16 * s + c] = alpha;
    }
    if (G == 0) {
      mlbuf[0][16 * s + c] = m_run;
      mlbuf[1][16 * s + c] = l_run;
    }
    __syncthreads();  // (m, l) are posted
  } else {
    // ======================= value waves =======================
    const int v = wave - 4;
    const int vh = v >> 2, lq = v & 3;  // heads 32vh .., latents 128lq ..
    const int hl = lane & 31, hf = lane >> 5;
    // tile copies: rows 4v .. 4v+3 of a tile
    // Indexed calls: the index slots of this wave's rows (4v .. 4v+3 of every tile) for tiles
    // 16k .. 16k+15 are copied straight into the wave's own LDS block k & 1 (lane l: tile 16k +
    // l / 4, row 4v + l % 4; slots past the split repeat its last slot).  The copy is counted by
    // the same vmcnt waits as the tile copies, so reading a slot never waits on memory.
    auto load_idx_block = [&](int k) {
      const int tile = 16 * k + (lane >> 2);
      const int slot = min(s_begin + tile * kTile + kRowsPerVWave * v + (lane & 3), s_end - 1);
      const uint32_t ls = __builtin_amdgcn_readfirstlane(lds_addr(&ibuf[INDEXED ? v : 0][k & 1][0]));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" : : "s"(ls), "v"(idx_row + slot)
                   : "memory", "m0");
#pragma clang diagnostic pop
    };
    // the wave's four listed positions of tile t, read from its index block in one 16-byte read
    auto tile_slots = [&](int t) {
      if constexpr (INDEXED) {
        const int4 q = *(const int4*)&ibuf[v][(t >> 4) & 1][4 * (t & 15)];
        return int4{__builtin_amdgcn_readfirstlane(q.x), __builtin_amdgcn_readfirstlane(q.y),
                    __builtin_amdgcn_readfirstlane(q.z), __builtin_amdgcn_readfirstlane(q.w)};
      } else {
        return int4{0, 0, 0, 0};
      }
    };
    int4 slots = {0, 0, 0, 0};
    auto issue_row = [&](int t, int rr) {
      const int r = kRowsPerVWave * v + rr;
      const uint32_t dst = lds0 + (t % kRing) * kTileBytes + r * kRowBytes;
      if constexpr (INDEXED) {
        int p = rr == 0 ? slots.x : rr == 1 ? slots.y : rr == 2 ? slots.z : slots.w;
        const bool ok = p >= 0 && p < L;
        if (lane == 0) vrow[t % kRing][r] = ok;
        p = ok ? p : 0;
        row_to_lds<NT>(seq + (size_t)p * kRowBytes, dst, lane16, (uint32_t)(swz(r) << 4));
      } else {
        const int first = s_begin + t * kTile;
        const int row = min(r, s_end - 1 - first);
        row_to_lds_at<NT>(seq + (size_t)first * kRowBytes, (uint32_t)(row * kRowBytes), dst, lane16,
                          (uint32_t)(swz(r) << 4));
      }
    };
    // Every row read is a visible row: rows past the split repeat its last row and indexed
    // slots naming a position outside the cache read row 0; the score waves mask both out.
    if constexpr (INDEXED) {
      if (ntiles > 0) {
        load_idx_block(0);
        wait_vmcnt<0>();
      }
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (t < ntiles) {
        slots = tile_slots(t);
#pragma unroll
        for (int rr = 0; rr < kRowsPerVWave; ++rr) issue_row(t, rr);
      }

    // transpose reads for the A operand
    const TrOffsets tro = transpose_offsets(lane, lq);
    const int tb0 = tro.tb0, tb1 = tro.tb1, te = tro.te;
    const int hv = hg * 64 + 32 * vh + hl;  // this lane's head (output column)

    f32x16 o[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int k = 0; k < 16; ++k) o[mb][k] = 0.f;
    wait_vmcnt<0>();
    __syncthreads();  // the first two tiles have landed

    for (int t = 0; t <= ntiles; ++t) {
      // tile t (copied in step t-2) must have landed before step t opens; tile t+1 may stay in flight
      if (t < ntiles) {
        if (t + 1 < ntiles) wait_vmcnt<kRowsPerVWave>();
        else wait_vmcnt<0>();
      }
      // the previous step's row-validity bytes must be in LDS before the score waves pass the
      // barrier (the compiler places no LDS wait before a barrier reached along the back edge)
      if constexpr (INDEXED) wait_lds_reads();
      __syncthreads();  // step t opens
      const int cp = t + 2;  // tile copied in this step, into the stage of tile t-2
      // the next block of index slots, needed from step 16k + 14 on, is copied in step 16k, before
      // this step's tile copies: the wait that opens step 16k + 1 has it in LDS
      if constexpr (INDEXED)
        if ((t & 15) == 0 && 16 * (t / 16 + 1) < ntiles) load_idx_block(t / 16 + 1);
      if (cp < ntiles) slots = tile_slots(cp);
      if (t == 0) {
        if (cp < ntiles)
#pragma unroll
          for (int rr = 0; rr < kRowsPerVWave; ++rr) issue_row(cp, rr);
        continue;
      }
      const int tv_ = t - 1;  // tile whose values this step accumulates
      const float alpha = abuf[tv_ & 1][32 * vh + hl];
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) o[mb] *= alpha;
      }
      bf16x8 pf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pf[ks] = *(const bf16x8*)(pbuf[tv_ & 1] + (32 * vh + hl) * kPStride + 32 * ks + 16 * hf);
      const uint8_t* tile = smem[tv_ % kRing];
      const int fh = opaque(te);
      const uint8_t* t0 = tile + tb0;
      const uint8_t* t1 = tile + tb1;
      constexpr int kAhead = 3;  // MFMAs whose reads are in flight ahead of the current one
      s16x4 tv[kAhead + 1][2];
      auto load = [&](int n, int slot) {  // n = 4 ks + mb
        const int sh = 64 * ((n & 3) ^ fh) + 16 * kRowBytes * (n >> 2);
        tv[slot][0] = lds_read_tr16(t0 + sh);
        tv[slot][1] = lds_read_tr16(t1 + sh);
      };
#pragma unroll
      for (int n = 0; n < kAhead; ++n) load(n, n);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        if (n + kAhead < 8) load(n + kAhead, (n + kAhead) % (kAhead + 1));
        if ((n & 1) == 0 && cp < ntiles) issue_row(cp, n >> 1);
        __builtin_amdgcn_sched_barrier(0);
        o[n & 3] = mfma32(concat_bf16(tv[n % (kAhead + 1)][0], tv[n % (kAhead + 1)][1]), pf[n >> 2], o[n & 3]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();  // (m, l) are posted; every read of the tile ring is done
    if (a.num_splits == 1) {
      if (hv < a.H) store_value_rows(a, bq, hv, lq, hf, mlbuf[0][32 * vh + hl], mlbuf[1][32 * vh + hl], o);
    } else {
      stage_value_rows(&smem[0][0], 32 * vh + hl, lq, hf, mlbuf[1][32 * vh + hl], o);
    }
  }
  if (a.num_splits > 1) {
    __syncthreads();  // the partial is staged
    copy_partial_block(a, ((size_t)split * a.B * a.Q + bq) * a.H + (size_t)hg * 64, min(64, a.H - 64 * hg),
                       &smem[0][0], 0, mlbuf[0], mlbuf[1]);
  }
}

// Query-pair form of the dense split kernel, used when a sequence has an even number of queries.
// One workgroup = one (sequence b, pair of adjacent queries i0 = i1 + 1, group of 64 heads,
// split).  The kernel also accepts an odd count, the first query then alone in its pair, but
// that workgroup costs a pair's step for one query's work, so the launcher (queries_per_wg)
// keeps odd counts on the single-query form.  The two queries differ
// only in their last visible position, so one run of tiles serves both, and every LDS read of a
// tile now feeds two products instead of one:
//   score wave s holds the absorbed queries of heads 16s .. 16s+15 for both queries (128 VGPRs)
//     and issues two MFMA 16x16x32 per tile read; the softmax runs per query, and P is posted
//     as 128 rows (query, head)
//   value wave 4+v (v = 4qq + lq) owns query qq of the pair, all 64 heads and latents
//     128lq .. 128lq+127: each transposed tile read feeds two MFMA 32x32x16 (the two 32-head
//     halves), sixteen per step
// Per step about 264 KiB of LDS traffic serves two queries, against 244 KiB for one in the
// single-query form.  The later query's extra position is masked out of the earlier one's scores
// in the last tile; a split that holds only that position gives the earlier query an empty
// partial (m = -inf, l = 0, o = 0), which the merge handles.  Each query's products, softmax and
// sums are those of the single-query form in the same order, so the two forms give the same bits.
// NT as for latent_attn_kernel.
template <bool NT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 3)))
void latent_attn_pair_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kRing][kTileBytes];
  __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][128 * kPStride];  // P [query][head][pos] bf16
  __shared__ float abuf[2][128];                                            // rescale factor per row
  __shared__ float mlbuf[2][128];                                           // final (m, l) per row

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wg = xcd_remap(blockIdx.x, a.total_wg);
  // logical order (b, head group, split, pair): the pairs of one split of one sequence are
  // adjacent, so they run on the same XCD and share the tile through its L2
  const int np = (a.Q + 1) >> 1;
  const int pr = wg % np;
  int rest = wg / np;
  const int split = rest % a.num_splits;
  rest /= a.num_splits;
  const int hg = rest % a.HG;
  const int b = rest / a.HG;
  const int i0 = a.Q - 1 - 2 * pr;  // later pairs see more positions: they start first
  const int i1 = i0 - 1;            // -1: no second query

  const int L = min(a.cache_len[b], a.max_cache_len);
  const int n0 = max(L - a.Q + i0 + 1, 0);  // positions 0 .. cache_len - Q + i0
  const int n1 = i1 >= 0 ? max(n0 - 1, 0) : 0;
  const int s_begin = split * a.split_len;
  const int s_end = min(s_begin + a.split_len, n0);
  const int s_end1 = min(s_begin + a.split_len, n1);
  const int ntiles = s_end > s_begin ? (s_end - s_begin + kTile - 1) / kTile : 0;
  const uint8_t* seq = a.cache + (size_t)b * a.cache_bstride_bytes;
  const uint32_t lane16 = (uint32_t)lane << 4;
  const uint32_t lds0 = lds_addr(&smem[0][0]);

  if (wave < 4) {
    // ======================= score waves =======================
    const int s = wave;
    const int c = lane & 15, G = lane >> 4;  // head 16s + c; k / row group G
    const int h = min(hg * 64 + 16 * s + c, a.H - 1);  // a partial group's missing heads reuse the last
    const float c2 = a.scale_log2;
    // absorbed queries as B operands: latents 32ks + 8G .. +7 (a lone query is loaded twice)
    bf16x8 qf[2][16];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int iq = (qq == 0 || i1 < 0) ? i0 : i1;
      const uint16_t* qrow = a.q_abs + ((size_t)(b * a.Q + iq) * a.H + h) * kLatent + 8 * G;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qf[qq][ks] = *(const bf16x8*)(qrow + 32 * ks);
    }
    // running maximum and sum per (query, head) live in mlbuf between steps (no room in VGPRs)
    if (G == 0) {
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        mlbuf[0][64 * qq + 16 * s + c] = -INFINITY;
        mlbuf[1][64 * qq + 16 * s + c] = 0.f;
      }
    }
    wait_vmcnt<0>();
    __syncthreads();  // the first two tiles have landed (copied by the value waves)

    for (int t = 0; t <= ntiles; ++t) {
      wait_lds_reads();
      __syncthreads();  // step t opens: tile t is in LDS; the value waves read P of step t-1
      if (t == ntiles) break;
      // the query registers leave no room to keep addresses across steps: each step derives them
      // from the lane index again (A operand addressing as in the single-query form)
      const int ln = opaque(lane);
      const int cl = ln & 15, Gl = ln >> 4;
      const uint8_t* rb = smem[t % kRing] + (4 * (cl & 3) + (cl >> 2)) * kRowBytes + ((Gl ^ (cl & 3)) << 4);
      const int hi = cl >> 2;
      auto rd = [&](int n) {  // n = 2 ks + block
        const int ks = n >> 1;
        return *(const bf16x8*)(rb + 16 * kRowBytes * (n & 1) + 256 * (ks >> 2) + (((ks & 3) ^ hi) << 6));
      };
      f32x4 sc[2][2] = {{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}, {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}}};
      constexpr int kAhead = 2;
      bf16x8 av[kAhead + 1];
      // the score waves' products issue first, so that their softmax tail overlaps the value
      // waves' products instead of following them
      __builtin_amdgcn_s_setprio(3);
#pragma unroll
      for (int n = 0; n < kAhead; ++n) av[n] = rd(n);
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        if (n + kAhead < 32) av[(n + kAhead) % (kAhead + 1)] = rd(n + kAhead);
        __builtin_amdgcn_sched_barrier(0);
        sc[0][n & 1] = mfma16(av[n % (kAhead + 1)], qf[0][n >> 1], sc[0][n & 1]);
        sc[1][n & 1] = mfma16(av[n % (kAhead + 1)], qf[1][n >> 1], sc[1][n & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      const int base = s_begin + t * kTile;
#pragma unroll
      for (int qq = 0; qq < 2; ++qq) {
        // lane holds positions 16 blk + 4jj + G of head c; mask those past the query's visible set
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = sc[qq][k >> 2][k & 3];
        const int nvalid = (qq == 0 ? s_end : s_end1) - base;
        const uint32_t valid = nvalid >= kTile ? 0xffffffffu : nvalid <= 0 ? 0u : ((1u << nvalid) - 1u);
        if (valid != 0xffffffffu) {
          // shifted once (no per-register bit masks to keep live), by the row group taken from
          // the lane index here rather than kept live across the products
          const uint32_t vg = valid >> (opaque(lane) >> 4);
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (!((vg >> (16 * (k >> 2) + 4 * (k & 3))) & 1u)) v[k] = -INFINITY;
        }
        const float tmax = tile_max(v, c2);
        const int lp = opaque(lane);
        const int row = 64 * qq + 16 * s + (lp & 15);  // P / rescale / (m, l) row of this lane
        float m_run = mlbuf[0][row], l_run = mlbuf[1][row];
        float p[8];
        const float alpha = softmax_step(v, tmax, c2, m_run, l_run, p);
        if (lp < 16) {
          mlbuf[0][row] = m_run;
          mlbuf[1][row] = l_run;
        }
        store_p_row(pbuf[t & 1] + row * kPStride + 8 * (lp >> 4), p);
        if (lp < 16) abuf[t & 1][row] = alpha;
      }
    }
    __syncthreads();  // (m, l) are posted
  } else {
    // ======================= value waves =======================
    const int v = wave - 4;
    const int qq = v >> 2, lq = v & 3;  // query qq of the pair, latents 128lq ..
    const int hl = lane & 31, hf = lane >> 5;
    // tile copies: rows 4v .. 4v+3 of a tile; rows past the split repeat its last row
    auto issue_row = [&](int t, int rr) {
      const int r = kRowsPerVWave * v + rr;
      const uint32_t dst = lds0 + (t % kRing) * kTileBytes + r * kRowBytes;
      const int first = s_begin + t * kTile;
      const int row = min(r, s_end - 1 - first);
      row_to_lds_at<NT>(seq + (size_t)first * kRowBytes, (uint32_t)(row * kRowBytes), dst, lane16,
                        (uint32_t)(swz(r) << 4));
    };
#pragma unroll
    for (int t = 0; t < 2; ++t)
      if (t < ntiles)
#pragma unroll
        for (int rr = 0; rr < kRowsPerVWave; ++rr) issue_row(t, rr);

    // transpose reads for the A operand, as in the single-query form
    const TrOffsets tro = transpose_offsets(lane, lq);
    const int tb0 = tro.tb0, tb1 = tro.tb1, te = tro.te;
    const int prow0 = 64 * qq + hl;  // P / rescale row of head half 0 (half 1: +32)

    f32x16 o[2][4];  // [head half][latent block]
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int k = 0; k < 16; ++k) o[nb][mb][k] = 0.f;
    wait_vmcnt<0>();
    __syncthreads();  // the first two tiles have landed

    for (int t = 0; t <= ntiles; ++t) {
      if (t < ntiles) {
        if (t + 1 < ntiles) wait_vmcnt<kRowsPerVWave>();
        else wait_vmcnt<0>();
      }
      __syncthreads();  // step t opens
      const int cp = t + 2;  // tile copied in this step, into the stage of tile t-2
      if (t == 0) {
        if (cp < ntiles)
#pragma unroll
          for (int rr = 0; rr < kRowsPerVWave; ++rr) issue_row(cp, rr);
        continue;
      }
      const int tv_ = t - 1;  // tile whose values this step accumulates
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float alpha = abuf[tv_ & 1][prow0 + 32 * nb];
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) o[nb][mb] *= alpha;
        }
      }
      // P of the first k-step now, of the second once its last product has been issued
      const uint8_t* pb = pbuf[tv_ & 1] + prow0 * kPStride + 16 * hf;
      bf16x8 pf[2];  // [head half]
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) pf[nb] = *(const bf16x8*)(pb + 32 * nb * kPStride);
      const uint8_t* tile = smem[tv_ % kRing];
      const int fh = opaque(te);
      const uint8_t* t0 = tile + tb0;
      const uint8_t* t1 = tile + tb1;
      constexpr int kAhead = 1;
      s16x4 tv[kAhead + 1][2];
      auto load = [&](int n, int slot) {  // n = 4 ks + mb
        const int sh = 64 * ((n & 3) ^ fh) + 16 * kRowBytes * (n >> 2);
        tv[slot][0] = lds_read_tr16(t0 + sh);
        tv[slot][1] = lds_read_tr16(t1 + sh);
      };
#pragma unroll
      for (int n = 0; n < kAhead; ++n) load(n, n);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        if (n + kAhead < 8) load(n + kAhead, (n + kAhead) % (kAhead + 1));
        if ((n & 1) == 0 && cp < ntiles) issue_row(cp, n >> 1);
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 av = concat_bf16(tv[n % (kAhead + 1)][0], tv[n % (kAhead + 1)][1]);
        o[0][n & 3] = mfma32(av, pf[0], o[0][n & 3]);
        o[1][n & 3] = mfma32(av, pf[1], o[1][n & 3]);
        __builtin_amdgcn_sched_barrier(0);
        if (n == 3)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) pf[nb] = *(const bf16x8*)(pb + 32 * nb * kPStride + 32);
      }
    }
    __syncthreads();  // (m, l) are posted; every read of the tile ring is done
    const int iq = qq == 0 ? i0 : i1;
    if (iq >= 0) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        if (a.num_splits == 1) {
          if (hg * 64 + 32 * nb + hl < a.H)
            store_value_rows(a, b * a.Q + iq, hg * 64 + 32 * nb + hl, lq, hf, mlbuf[0][prow0 + 32 * nb],
                             mlbuf[1][prow0 + 32 * nb], o[nb]);
        } else
          stage_value_rows(&smem[0][0], prow0 + 32 * nb, lq, hf, mlbuf[1][prow0 + 32 * nb], o[nb]);
      }
    }
  }
  if (a.num_splits > 1) {
    __syncthreads();  // the partials are staged: rows 64 qq + head of query qq of the pair
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      const int iq = qq == 0 ? i0 : i1;
      if (iq >= 0)
        copy_partial_block(a, ((size_t)split * a.B * a.Q + b * a.Q + iq) * a.H + (size_t)hg * 64,
                           min(64, a.H - 64 * hg), &smem[0][0], 64 * qq, mlbuf[0] + 64 * qq, mlbuf[1] + 64 * qq);
    }
  }
}

// Merge of the split partials (up to eight splits): four (b, i, head) rows per workgroup of 256
// threads, 64 threads per row, thread t owning latents 8t .. 8t+7 (16-byte loads, 32-byte stores).
// NS split slots loaded (merge_slots).
constexpr int kCombineRows = 4;
template <int NS>
__global__ __launch_bounds__(64 * kCombineRows) void combine_kernel(AttnArgs a) {
  const size_t rows = (size_t)a.B * a.Q * a.H;
  const size_t row = (size_t)blockIdx.x * kCombineRows + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int t = threadIdx.x & 63;
  // at most eight splits: one group, merged as merge_splits8 does (merge_one_group8_blocks)
  MergeGroup g[2];
  merge_load8<NS>(g, a.part_o + row * kLatent + 8 * t, a.part_ml + 2 * row, rows * kLatent, 2 * rows, a.num_splits,
                  0);
  const f32x4 v[2][8] = {{g[0].v[0], g[0].v[1], g[0].v[2], g[0].v[3], g[0].v[4], g[0].v[5], g[0].v[6], g[0].v[7]},
                         {g[1].v[0], g[1].v[1], g[1].v[2], g[1].v[3], g[1].v[4], g[1].v[5], g[1].v[6], g[1].v[7]}};
  float lse2;
  f32x4 o[2];
  merge_one_group8_blocks<2>(g[0].mm, g[0].ll, v, a.num_splits, &lse2, o);
  // the merged rows are the call's output, written once and not read again here: non-temporal
  // stores (16 MiB of o_lat at 32 x 4 indexed: 66.4 -> 64.6 us for the call)
  float* dst = a.o_lat + row * kLatent + 8 * t;
  __builtin_nontemporal_store(o[0], (f32x4*)dst);
  __builtin_nontemporal_store(o[1], (f32x4*)(dst + 4));
  if (a.lse != nullptr && t == 0) a.lse[row] = lse2 * 0.69314718055994531f;
}

// Merge of more than eight splits: G = min(8, groups of eight splits) thread groups of 64 per
// (b, i, head), thread t owning latents 8t .. 8t+7.  Thread group q reduces group r0 + q of a round
// of G groups, all the round's loads in flight together, and thread group 0 folds the round's
// results in group order (the order merge_splits8 uses, so the bits are the same): one memory round
// trip per G groups instead of one per group.
__global__ __launch_bounds__(512) void combine_wide_kernel(AttnArgs a) {
  __shared__ f32x4 gacc[8][2][64];
  __shared__ float gM[8][64], gL[8][64];  // the same for both blocks of four latents
  const size_t row = blockIdx.x;
  const int t = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int G = blockDim.x >> 6;  // thread groups, 2 .. 8
  const size_t rows = (size_t)a.B * a.Q * a.H;
  const int S = a.num_splits;
  const int ngroups = (S + 7) / 8;
  const uint16_t* po = a.part_o + row * kLatent + 8 * t;
  const float* pml = a.part_ml + 2 * row;
  float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.f, 0.f};
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int r0 = 0; r0 < ngroups; r0 += G) {
    const int g = r0 + q;
    MergePartial p[2];
    bool ok = false;
    if (g < ngroups) {
      MergeGroup grp[2];
      merge_load8(grp, po, pml, rows * kLatent, 2 * rows, S, 8 * g);
      ok = merge_group(grp[0], S, 8 * g, p[0]);
      merge_group(grp[1], S, 8 * g, p[1]);  // same weights: ok alike
    }
    gM[q][t] = ok ? p[0].M : -INFINITY;
    gL[q][t] = ok ? p[0].L : 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) gacc[q][h][t] = ok ? p[h].acc : f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (q == 0)
      for (int k = 0; k < G && r0 + k < ngroups; ++k)
        if (gM[k][t] != -INFINITY)
#pragma unroll
          for (int h = 0; h < 2; ++h) merge_fold(M[h], L[h], acc[h], MergePartial{gM[k][t], gL[k][t], gacc[k][h][t]});
    __syncthreads();  // the round's slots are rewritten by the next round
  }
  if (q == 0) {
    float* dst = a.o_lat + row * kLatent + 8 * t;  // output: non-temporal, as in combine_kernel
    __builtin_nontemporal_store(acc[0] * (1.0f / L[0]), (f32x4*)dst);
    __builtin_nontemporal_store(acc[1] * (1.0f / L[1]), (f32x4*)(dst + 4));
    // __builtin_amdgcn_logf is the hardware base-2 logarithm
    if (a.lse != nullptr && t == 0) a.lse[row] = (M[0] + __builtin_amdgcn_logf(L[0])) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_latent_attn(const AttnArgs& a, bool indexed, hipStream_t stream) {
  void* args[] = {const_cast<AttnArgs*>(&a)};
  const dim3 grid(a.total_wg), block(kThreads);
  const void* k;
  if (a.stream_once) {
    if (a.q_abs_lo != nullptr)
      k = indexed ? (const void*)&latent_attn_kernel<true, true, true>
                  : (const void*)&latent_attn_kernel<false, true, true>;
    else
      k = indexed                            ? (const void*)&latent_attn_kernel<true, false, true>
          : queries_per_wg(false, a.Q) == 2 ? (const void*)&latent_attn_pair_kernel<true>
                                            : (const void*)&latent_attn_kernel<false, false, true>;
  } else {
    if (a.q_abs_lo != nullptr)
      k = indexed ? (const void*)&latent_attn_kernel<true, true, false>
                  : (const void*)&latent_attn_kernel<false, true, false>;
    else
      k = indexed                            ? (const void*)&latent_attn_kernel<true, false, false>
          : queries_per_wg(false, a.Q) == 2 ? (const void*)&latent_attn_pair_kernel<false>
                                            : (const void*)&latent_attn_kernel<false, false, false>;
  }
  return hipLaunchKernel(k, grid, block, args, 0, stream);
}

hipError_t launch_combine(const AttnArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<AttnArgs*>(&a)};
  const dim3 grid(a.B * a.Q * a.H);
  if (a.num_splits > 8) {
    const int groups = (a.num_splits + 7) / 8;
    const dim3 block(64 * (groups < 8 ? groups : 8));
    return hipLaunchKernel((const void*)&combine_wide_kernel, grid, block, args, 0, stream);
  }
  const dim3 cgrid((unsigned)(((size_t)a.B * a.Q * a.H + kCombineRows - 1) / kCombineRows));
  const int ns = merge_slots(a.num_splits);
  const void* k = ns == 2 ? (const void*)&combine_kernel<2>
                  : ns == 4 ? (const void*)&combine_kernel<4>
                            : (const void*)&combine_kernel<8>;
  return hipLaunchKernel(k, cgrid, dim3(64 * kCombineRows), args, 0, stream);
}

}  // namespace mla
