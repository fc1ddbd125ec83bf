// k-pooled sparse-attention indexer for gfx950: builds the position lists that indexed latent
// attention consumes (colibri "GLM-5.3-Flash engine (c/glm53.c)", "Architecture notes", "DSA
// with k-pooling"; page "Module 08 -- Vision, MTP, and Hybrid Serving State", section 3 for the
// pool-completion causality rule).
//
//   kpool_kernel   pooled[b][p][c] = sum_s w[s][c] k[b][p*pool + s][c], w[.][c] = softmax over the
//                  pool's positions of the gate logits g[b][p*pool + s][c] (fp32)
//   score_kernel   scores[b][i][p] = q[b][i] . pooled[b][p] (fp32, a fixed order of the channels)
//   select_kernel  per query at t = cache_len - Q + i: the topk / pool best pools among the
//                  complete ones (last position <= t), ties to the lower pool, in ascending order,
//                  expanded to positions, then the incomplete tail floor((t+1)/pool)*pool .. t;
//                  unused slots -1
// The selection is integer work decided on the fp32 scores: a radix select over order-preserving
// 32-bit keys finds the k-th largest score, equal keys are taken lowest pool first.
// Keys and gate logits are read as 16-byte vectors: rows start 16-byte aligned (d is a multiple
// of 8, batch_stride a multiple of 8 elements).
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelPerThread = kMaxIndexerPools / kSelThreads;  // pools owned by one thread
constexpr int kHistBins = 2048;
constexpr int kKpoolBlocks = 4096;    // pooled-key workgroups in all, striding over the pools
constexpr int kScoreLanes = 8;        // lanes that share one pool's key
constexpr int kScoreBatch = 2;        // pools per lane group in flight together
constexpr int kScorePoolsPerBlock = 64;

static_assert(kSelPerThread <= 32 && 64 % kSelPerThread == 0, "the selection keeps one 32-bit mask per thread");

// Eight channels per thread (16-byte loads of keys and gate logits): d / 8 threads per pool.
// Per channel: gm = max_s g, e_s = exp(g_s - gm), pooled = (sum_s e_s k_s) / (sum_s e_s).
// Pools of up to PR positions (PR = 4 or 8) keep their gate logits in registers between the two
// passes and issue every load of the pool at once; longer pools (PR = 0) read the logits twice.

__device__ __forceinline__ void kpool_store(float* dst, const float (&acc)[8], const float (&sum)[8]) {
  const f32x4 lo = {acc[0] / sum[0], acc[1] / sum[1], acc[2] / sum[2], acc[3] / sum[3]};
  const f32x4 hi = {acc[4] / sum[4], acc[5] / sum[5], acc[6] / sum[6], acc[7] / sum[7]};
  *(f32x4*)dst = lo;
  *(f32x4*)(dst + 4) = hi;
}

template <int PR>
__global__ __launch_bounds__(256) void kpool_kernel(KpoolArgs a) {
  const int b = blockIdx.y;
  const int L = min(a.cache_len[b], a.max_cache_len);
  const int np = min(L / a.pool, a.max_pools);
  const int p0 = a.pool_begin ? max(a.pool_begin[b], 0) : 0;
  const int tpp = a.d >> 3;                 // threads per pool
  const int per_block = 256 / tpp;
  const int c0 = 8 * ((int)threadIdx.x % tpp);
  const int stride = gridDim.x * per_block;
  const uint16_t* kb = a.k + (size_t)b * a.batch_stride + c0;
  const uint16_t* gb = a.g + (size_t)b * a.batch_stride + c0;
  // pools of up to four positions: two pools per thread per pass, every load of both in flight
  constexpr int U = PR == 4 ? 2 : 1;
  for (int p = p0 + blockIdx.x * per_block + (int)threadIdx.x / tpp; p < np; p += stride * U) {
    if constexpr (PR > 0) {
      s16x8 gv[U][PR], kv[U][PR];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pu = p + u * stride;
        const size_t base = (size_t)pu * a.pool * a.d;
#pragma unroll
        for (int s = 0; s < PR; ++s) {
          if (s < a.pool && pu < np) {
            gv[u][s] = *(const s16x8*)(gb + base + (size_t)s * a.d);
            kv[u][s] = *(const s16x8*)(kb + base + (size_t)s * a.d);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pu = p + u * stride;
        if (pu >= np) break;
        float gm[8], sum[8], acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gm[e] = -INFINITY;
          sum[e] = acc[e] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < PR; ++s)
          if (s < a.pool)
#pragma unroll
            for (int e = 0; e < 8; ++e) gm[e] = fmaxf(gm[e], bf16_bits_to_f32((uint16_t)gv[u][s][e]));
#pragma unroll
        for (int s = 0; s < PR; ++s) {
          if (s < a.pool) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float w = __expf(bf16_bits_to_f32((uint16_t)gv[u][s][e]) - gm[e]);
              sum[e] += w;
              acc[e] = __builtin_fmaf(w, bf16_bits_to_f32((uint16_t)kv[u][s][e]), acc[e]);
            }
          }
        }
        kpool_store(a.pooled + ((size_t)b * a.max_pools + pu) * a.d + c0, acc, sum);
      }
    } else {
      const size_t base = (size_t)p * a.pool * a.d;
      float gm[8], sum[8], acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        gm[e] = -INFINITY;
        sum[e] = acc[e] = 0.f;
      }
      for (int s = 0; s < a.pool; ++s) {
        const s16x8 g1 = *(const s16x8*)(gb + base + (size_t)s * a.d);
#pragma unroll
        for (int e = 0; e < 8; ++e) gm[e] = fmaxf(gm[e], bf16_bits_to_f32((uint16_t)g1[e]));
      }
      for (int s = 0; s < a.pool; ++s) {
        const s16x8 g1 = *(const s16x8*)(gb + base + (size_t)s * a.d);
        const s16x8 k1 = *(const s16x8*)(kb + base + (size_t)s * a.d);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float w = __expf(bf16_bits_to_f32((uint16_t)g1[e]) - gm[e]);
          sum[e] += w;
          acc[e] = __builtin_fmaf(w, bf16_bits_to_f32((uint16_t)k1[e]), acc[e]);
        }
      }
      kpool_store(a.pooled + ((size_t)b * a.max_pools + p) * a.d + c0, acc, sum);
    }
  }
}

// Eight lanes per pool: lane i of a pool's group reads 16-byte chunks 8j + i of the fp32 key,
// so each load instruction reads whole 128-byte lines of eight consecutive pools.  The lane
// sums its channels for every query (queries in LDS as fp32), the group adds its eight
// partial sums (butterfly over lanes xor 1, 2, 4), and lane i < Q writes query i's score.
// NCH: 16-byte chunks per lane (d / 32).  QR > 0: every query (Q <= QR) is copied from LDS to
// registers once, so the inner loop reads no LDS; QR = 0 reads the queries from LDS per pool.
// A workgroup takes 64 pools, two per lane group, whose loads are issued before the queries are
// staged: the block's one memory round trip covers both.  Small blocks keep every CU's share of
// the pooled keys in flight at once (256 pools per block with the queries staged first ran 20%
// slower; loading the queries per lane from global memory instead of through LDS, slower still).
template <int NCH, int QR>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
  __shared__ f32x4 qs[kMaxIndexerQ * kMaxIndexerDim / 4];
  const int b = blockIdx.y;
  const int L = min(a.cache_len[b], a.max_cache_len);
  const int np = min(L / a.pool, a.max_pools);
  const int pb = blockIdx.x * kScorePoolsPerBlock;
  if (pb >= np) return;  // uniform over the block
  const int d4 = a.d >> 2;
  const int i = threadIdx.x & (kScoreLanes - 1);
  const int pend = min(pb + kScorePoolsPerBlock, np);
  constexpr int kStride = kScoreBatch * (256 / kScoreLanes);
  // a lane group takes kScoreBatch pools 32 apart at once, so all their loads are in flight together
  f32x4 v[kScoreBatch][NCH];
  auto load = [&](int p0) {
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u) {
      const int p = min(p0 + u * (256 / kScoreLanes), pend - 1);
      const f32x4* row = (const f32x4*)(a.pooled + ((size_t)b * a.max_pools + p) * a.d);
#pragma unroll
      for (int j = 0; j < NCH; ++j) v[u][j] = row[kScoreLanes * j + i];
    }
  };
  int p0 = pb + (int)threadIdx.x / kScoreLanes;
  load(p0);  // the first pools are in flight while the queries are staged
  for (int e = threadIdx.x; e < a.Q * d4; e += 256) {
    const uint16_t* src = a.q + ((size_t)b * a.Q * a.d) + 4 * e;
    qs[e] = f32x4{bf16_bits_to_f32(src[0]), bf16_bits_to_f32(src[1]), bf16_bits_to_f32(src[2]),
                  bf16_bits_to_f32(src[3])};
  }
  __syncthreads();
  constexpr int kQ = QR > 0 ? QR : kMaxIndexerQ;  // queries the loops run over
  f32x4 qreg[QR > 0 ? NCH : 1][QR > 0 ? QR : 1];
  if constexpr (QR > 0) {
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
      for (int q = 0; q < QR; ++q) qreg[j][q] = q < a.Q ? qs[q * d4 + kScoreLanes * j + i] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  for (;;) {  // lane groups past the block's last pool compute on clamped rows and store nothing
#pragma unroll
    for (int u = 0; u < kScoreBatch; ++u) {
      const int p = p0 + u * (256 / kScoreLanes);
      float acc[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) acc[q] = 0.f;
#pragma unroll
      for (int j = 0; j < NCH; ++j) {
        const int c = kScoreLanes * j + i;
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          if (q < a.Q) {
            f32x4 w;
            if constexpr (QR > 0)
              w = qreg[j][q];
            else
              w = qs[q * d4 + c];
            acc[q] = __builtin_fmaf(w[0], v[u][j][0], acc[q]);
            acc[q] = __builtin_fmaf(w[1], v[u][j][1], acc[q]);
            acc[q] = __builtin_fmaf(w[2], v[u][j][2], acc[q]);
            acc[q] = __builtin_fmaf(w[3], v[u][j][3], acc[q]);
          }
        }
      }
      float mine = 0.f;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (q < a.Q) {
          float x = acc[q];
          x += __shfl_xor(x, 1);
          x += __shfl_xor(x, 2);
          x += __shfl_xor(x, 4);
          if (q == i) mine = x;
        }
      }
      if (i < a.Q && p < pend) a.scores[((size_t)b * a.Q + i) * a.max_pools + p] = mine;
    }
    p0 += kStride;
    if (p0 >= pend) break;
    load(p0);
  }
}

// order-preserving unsigned key of an fp32 value (larger float, larger key)
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of v over the block's threads; `total` receives the block sum.
// Every thread of the block must call it (it holds two barriers).
__device__ int block_exclusive_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int s = wsum[w];
    if (w < wave) before += s;
    total += s;
  }
  __syncthreads();  // wsum is rewritten by the next scan
  return before + x - v;
}

// One workgroup per (sequence, query).  The selectable pools' scores become order keys in LDS;
// thread t owns pools 16t .. 16t+15 and visits them rotated by t/4 (slot j -> pool 16t + ((j +
// t/4) & 15)), which puts the 64 lanes of a wave in 64 different banks.
//   1. A radix select over the keys, 11 + 11 + 10 bits from the top, finds the n_sel-th largest
//      key kth and how many keys equal to it are taken (need_eq).
//   2. Each thread marks its pools above kth and its keys equal to kth; a block scan over the
//      equal counts gives the lowest-index-first share of need_eq to each thread, a second scan
//      over the selected counts gives each thread its place in the output, and the thread writes
//      its selected pools' positions in ascending order.
__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  __shared__ uint32_t keys[kMaxIndexerPools];
  __shared__ int hist[kHistBins];
  __shared__ int wsum[kSelThreads / 64];
  __shared__ int s_digit, s_remaining;

  const int bq = blockIdx.x;
  const int b = bq / a.Q, i = bq % a.Q;
  const int tid = threadIdx.x;
  const int L = min(a.cache_len[b], a.max_cache_len);
  const int t = L - a.Q + i;  // this query's position
  const int np = t >= 0 ? min((t + 1) / a.pool, min(L / a.pool, a.max_pools)) : 0;
  const int n_sel = a.topk / a.pool;
  const float* sc = a.scores + (size_t)bq * a.max_pools;
  // every load of the row in flight at once (up to 64 per thread), then the LDS stores
  {
    float v[kSelPerThread];
#pragma unroll
    for (int u = 0; u < kSelPerThread; ++u) {
      const int p = u * kSelThreads + tid;
      v[u] = p < np ? sc[p] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kSelPerThread; ++u) {
      const int p = u * kSelThreads + tid;
      if (p < np) keys[p] = order_key(v[u]);
    }
  }
  __syncthreads();

  const bool all = np <= n_sel;
  const int own = kSelPerThread * tid;
  uint32_t kth = 0;
  int need_eq = 0;
  if (!all) {
    uint32_t prefix = 0, mask = 0;
    int rem = n_sel;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const int nb = pass == 2 ? 1024 : 2048;
      for (int e = tid; e < nb; e += kSelThreads) hist[e] = 0;
      __syncthreads();
      for (int j = 0; j < kSelPerThread; ++j) {
        const int p = own + ((j + ((tid * kSelPerThread) >> 6)) & (kSelPerThread - 1));
        if (p < np) {
          const uint32_t k = keys[p];
          if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & (nb - 1)], 1);
        }
      }
      __syncthreads();
      // thread t sums bins nb-1-(per*t) .. nb-per-(per*t) (the top bins first)
      const int per = nb / kSelThreads;
      int c = 0;
      for (int e = 0; e < per; ++e) c += hist[nb - 1 - (per * tid + e)];
      int total;
      const int before = block_exclusive_scan(c, wsum, total);
      if (before < rem && rem <= before + c) {
        int cum = before;
        for (int e = 0; e < per; ++e) {
          const int bin = nb - 1 - (per * tid + e);
          const int h = hist[bin];
          if (cum + h >= rem) {
            s_digit = bin;
            s_remaining = rem - cum;
            break;
          }
          cum += h;
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      mask |= (uint32_t)(nb - 1) << shift;
      rem = s_remaining;
      __syncthreads();  // s_digit and hist are rewritten by the next pass
    }
    kth = prefix;
    need_eq = rem;
  }

  uint32_t above = 0, eq = 0;
  for (int j = 0; j < kSelPerThread; ++j) {
    const int jj = (j + ((tid * kSelPerThread) >> 6)) & (kSelPerThread - 1);
    const int p = own + jj;
    if (p < np) {
      const uint32_t k = keys[p];
      if (all || k > kth)
        above |= 1u << jj;
      else if (k == kth)
        eq |= 1u << jj;
    }
  }
  int total;
  const int n_eq = __builtin_popcount(eq);
  const int eq_before = block_exclusive_scan(n_eq, wsum, total);
  const int take = min(max(need_eq - eq_before, 0), n_eq);
  uint32_t kept = 0, rest = eq;
  for (int e = 0; e < take; ++e) {
    kept |= rest & (~rest + 1u);  // lowest set bit
    rest &= rest - 1u;
  }
  uint32_t sel = above | kept;
  int taken;
  int r = block_exclusive_scan(__builtin_popcount(sel), wsum, taken);
  int32_t* out = a.idx + (size_t)bq * a.K_max;
  while (sel) {
    const int jj = __builtin_ctz(sel);
    sel &= sel - 1u;
    const int p = own + jj;
    for (int u = 0; u < a.pool; ++u) out[r * a.pool + u] = p * a.pool + u;
    ++r;
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
  // about 4096 workgroups in all (16 per CU), each striding over its sequence's pools: enough
  // to stream a full build, and few enough that an incremental build of a handful of new pools
  // is not dominated by launching empty workgroups
  const int per_block = 256 / (a.d / 8);
  const int blocks = (a.max_pools + per_block - 1) / per_block;
  const int per_seq = a.B >= kKpoolBlocks ? 1 : kKpoolBlocks / a.B;
  const dim3 grid(blocks < per_seq ? blocks : per_seq, a.B), block(256);
  const void* fn = a.pool <= 4 ? (const void*)&kpool_kernel<4>
                   : a.pool <= 8 ? (const void*)&kpool_kernel<8> : (const void*)&kpool_kernel<0>;
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<ScoreArgs*>(&a)};
  const dim3 grid((a.max_pools + kScorePoolsPerBlock - 1) / kScorePoolsPerBlock, a.B), block(256);
  // queries in registers when they fit in 64 VGPRs (Q * d <= 512)
  const void* fn = a.d == 64   ? (const void*)&score_kernel<2, 8>
                   : a.d == 128 ? (a.Q <= 4 ? (const void*)&score_kernel<4, 4> : (const void*)&score_kernel<4, 0>)
                                : (a.Q <= 2 ? (const void*)&score_kernel<8, 2> : (const void*)&score_kernel<8, 0>);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t launch_select(const SelectArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<SelectArgs*>(&a)};
  const dim3 grid(a.B * a.Q), block(kSelThreads);
  return hipLaunchKernel((const void*)&select_kernel, grid, block, args, 0, stream);
}

}  // namespace mla
