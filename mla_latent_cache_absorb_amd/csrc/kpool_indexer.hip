// k-pooled sparse-attention indexer for gfx950: builds the position lists that indexed latent
// attention consumes (colibri "GLM-5.3-Flash engine (c/glm53.c)", "Architecture notes", "DSA
// with k-pooling"; page "Module 08 -- Vision, MTP, and Hybrid Serving State", section 3 for the
// pool-completion causality rule).
//
//   kpool_kernel   pooled[b][p][c] = sum_s w[s][c] k[b][p*pool + s][c], w[.][c] = softmax over the
//                  pool's positions of the gate logits g[b][p*pool + s][c] (fp32)
//   score_kernel   scores[b][i][p] = q[b][i] . pooled[b][p] (fp32, channels in order)
//   select_kernel  per query at t = cache_len - Q + i: the topk / pool best pools among the
//                  complete ones (last position <= t), ties to the lower pool, in ascending order,
//                  expanded to positions, then the incomplete tail floor((t+1)/pool)*pool .. t;
//                  unused slots -1
// The selection is integer work decided on the fp32 scores: a radix select over order-preserving
// 32-bit keys finds the k-th largest score, equal keys are taken lowest pool first.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kSelThreads = 256;

__global__ __launch_bounds__(256) void kpool_kernel(KpoolArgs a) {
  const int b = blockIdx.y;
  const int L = min(a.cache_len[b], a.max_cache_len);
  const int np = min(L / a.pool, a.max_pools);
  const int p0 = a.pool_begin ? max(a.pool_begin[b], 0) : 0;
  const int per_block = 256 / a.d;  // pools handled at once (d threads each)
  const int c = threadIdx.x % a.d;
  const uint16_t* kb = a.k + (size_t)b * a.batch_stride;
  const uint16_t* gb = a.g + (size_t)b * a.batch_stride;
  for (int p = p0 + blockIdx.x * per_block + (int)threadIdx.x / a.d; p < np; p += gridDim.x * per_block) {
    const size_t base = (size_t)p * a.pool * a.d + c;
    float gm = -INFINITY;
    for (int s = 0; s < a.pool; ++s) gm = fmaxf(gm, bf16_bits_to_f32(gb[base + (size_t)s * a.d]));
    float sum = 0.f, acc = 0.f;
    for (int s = 0; s < a.pool; ++s) {
      const float e = __expf(bf16_bits_to_f32(gb[base + (size_t)s * a.d]) - gm);
      sum += e;
      acc = __builtin_fmaf(e, bf16_bits_to_f32(kb[base + (size_t)s * a.d]), acc);
    }
    a.pooled[((size_t)b * a.max_pools + p) * a.d + c] = acc / sum;
  }
}

// One thread per pool, all queries of the sequence at once (Q <= kMaxIndexerQ); the queries
// sit in LDS as fp32, the pool's key is read once as 16-byte vectors.
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  __shared__ float qs[kMaxIndexerQ * kMaxIndexerDim];
  const int b = blockIdx.y;
  for (int e = threadIdx.x; e < a.Q * a.d; e += 256)
    qs[e] = bf16_bits_to_f32(a.q[(size_t)b * a.Q * a.d + e]);
  __syncthreads();
  const int L = min(a.cache_len[b], a.max_cache_len);
  const int np = min(L / a.pool, a.max_pools);
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= np) return;
  const f32x4* row = (const f32x4*)(a.pooled + ((size_t)b * a.max_pools + p) * a.d);
  float acc[kMaxIndexerQ];
#pragma unroll
  for (int i = 0; i < kMaxIndexerQ; ++i) acc[i] = 0.f;
  for (int c4 = 0; c4 < a.d / 4; ++c4) {
    const f32x4 v = row[c4];
#pragma unroll
    for (int i = 0; i < kMaxIndexerQ; ++i) {
      if (i < a.Q) {
        const float* qq = qs + i * a.d + 4 * c4;
        acc[i] = __builtin_fmaf(qq[0], v[0], acc[i]);
        acc[i] = __builtin_fmaf(qq[1], v[1], acc[i]);
        acc[i] = __builtin_fmaf(qq[2], v[2], acc[i]);
        acc[i] = __builtin_fmaf(qq[3], v[3], acc[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxIndexerQ; ++i)
    if (i < a.Q) a.scores[((size_t)b * a.Q + i) * a.max_pools + p] = acc[i];
}

// order-preserving unsigned key of an fp32 value (larger float, larger key)
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// number of set bits of a wave ballot below this lane
__device__ __forceinline__ int rank_in_wave(uint64_t ballot, int lane) {
  return __builtin_popcountll(ballot & ((1ull << lane) - 1ull));
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ uint32_t keys[kMaxIndexerPools];
  __shared__ int hist[256];
  __shared__ int wsum[kSelThreads / 64][2];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_remaining;

  const int bq = blockIdx.x;
  const int b = bq / a.Q, i = bq % a.Q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = min(a.cache_len[b], a.max_cache_len);
  const int t = L - a.Q + i;  // this query's position
  const int np = t >= 0 ? min((t + 1) / a.pool, min(L / a.pool, a.max_pools)) : 0;
  const int n_sel = a.topk / a.pool;
  const float* sc = a.scores + (size_t)bq * a.max_pools;
  for (int p = tid; p < np; p += kSelThreads) keys[p] = order_key(sc[p]);

  // the threshold key: the n_sel-th largest, found eight bits at a time from the top
  uint32_t kth = 0;
  int need_eq = 0;  // keys equal to kth that are taken (lowest pools first)
  const bool all = np <= n_sel;
  if (!all) {
    if (tid == 0) {
      s_prefix = 0;
      s_mask = 0;
      s_remaining = n_sel;
    }
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0;
      __syncthreads();
      const uint32_t prefix = s_prefix, mask = s_mask;
      for (int p = tid; p < np; p += kSelThreads) {
        const uint32_t k = keys[p];
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
      }
      __syncthreads();
      if (tid == 0) {
        int rem = s_remaining, cum = 0, digit = 0;
        for (int dgt = 255; dgt >= 0; --dgt) {
          if (cum + hist[dgt] >= rem) {
            digit = dgt;
            break;
          }
          cum += hist[dgt];
        }
        s_remaining = rem - cum;
        s_prefix = prefix | ((uint32_t)digit << shift);
        s_mask = mask | (255u << shift);
      }
      __syncthreads();
    }
    kth = s_prefix;
    need_eq = s_remaining;
  }

  // walk the pools in index order, 256 at a time: selected = above the threshold, or equal to
  // it within the first need_eq equal ones; each selected pool's rank places its positions
  int32_t* out = a.idx + (size_t)bq * a.K_max;
  int eq_seen = 0, taken = 0;
  for (int base = 0; base < np; base += kSelThreads) {
    const int p = base + tid;
    const bool valid = p < np;
    const uint32_t k = valid ? keys[p] : 0u;
    const bool eq = valid && !all && k == kth;
    const uint64_t beq = __builtin_amdgcn_ballot_w64(eq);
    if (lane == 0) wsum[wave][0] = __builtin_popcountll(beq);
    __syncthreads();
    int eq_off = eq_seen;
    for (int w = 0; w < wave; ++w) eq_off += wsum[w][0];
    const int eq_rank = eq_off + rank_in_wave(beq, lane);
    const bool sel = valid && (all || k > kth || (eq && eq_rank < need_eq));
    const uint64_t bsel = __builtin_amdgcn_ballot_w64(sel);
    if (lane == 0) wsum[wave][1] = __builtin_popcountll(bsel);
    __syncthreads();
    int sel_off = taken, eq_tot = 0, sel_tot = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) {
      if (w < wave) sel_off += wsum[w][1];
      eq_tot += wsum[w][0];
      sel_tot += wsum[w][1];
    }
    if (sel) {
      const int r = sel_off + rank_in_wave(bsel, lane);
      for (int u = 0; u < a.pool; ++u) out[r * a.pool + u] = p * a.pool + u;
    }
    eq_seen += eq_tot;
    taken += sel_tot;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  // the incomplete tail pool, then padding
  const int n_tail = (a.tail && t >= 0) ? t + 1 - np * a.pool : 0;
  const int len = taken * a.pool + n_tail;
  for (int j = tid; j < n_tail; j += kSelThreads) out[taken * a.pool + j] = np * a.pool + j;
  for (int j = len + tid; j < a.K_max; j += kSelThreads) out[j] = -1;
  if (tid == 0) a.idx_len[bq] = len;
}

}  // namespace

hipError_t launch_kpool(const KpoolArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<KpoolArgs*>(&a)};
  const int per_block = 256 / a.d;
  const int blocks = (a.max_pools + per_block - 1) / per_block;
  const dim3 grid(blocks < 4096 ? blocks : 4096, a.B), block(256);
  return hipLaunchKernel((const void*)&kpool_kernel, grid, block, args, 0, stream);
}

hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<ScoreArgs*>(&a)};
  const dim3 grid((a.max_pools + 255) / 256, a.B), block(256);
  return hipLaunchKernel((const void*)&score_kernel, grid, block, args, 0, stream);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<SelectArgs*>(&a)};
  const dim3 grid(a.B * a.Q), block(kSelThreads);
  return hipLaunchKernel((const void*)&select_kernel, grid, block, args, 0, stream);
}

}  // namespace mla
