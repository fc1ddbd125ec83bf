// The naive (expanded) form of MLA attention for gfx950, the other side of the prefill / decode
// comparison of page "Module 05 -- MLA: Compressing Per-Token History", section 5: expand every
// cached token's per-head key and value, k_{j,h} = U_h^K c_j and v_{j,h} = U_h^V c_j (section 1),
// then run ordinary causal multi-head attention on them (section 4: a query sees j <= t).
//
// expand_kv_kernel   one GEMM per operand: [positions x 512] latents times the [H*D x 512]
//                    weights (U_h stored [D][R] per head, so row h*D + d is U_h[d][:]), fp32
//                    accumulation, nearest-even bf16 out; 256 x 256 tiles, three stages of 32
//                    latents in flight.  Keys are written position-major,
//                    K[b][j][h][d]; values head-major and transposed, V^T[b][h][d][j], so that the
//                    attention's value product reads them along positions.
// naive_attn_kernel  flash attention with head dimension 256: per (sequence, head, 128 queries),
//                    eight waves of 16 queries each over 64-key tiles staged in LDS.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

// ---------------------------------------------------------------------------------- expansion
// A workgroup computes a 256 x 256 tile (channels h * D + d by positions) over the 512 latents in
// 16 stages of 32, eight waves of 64 channels x 128 positions (2 x 4 MFMA 32x32x16 blocks).  The
// stages pass through a ring of four LDS buffers, three in flight, so the products of one stage
// run while the next ones are on their way (with one stage in flight the workgroup waited on
// memory for every stage).
constexpr int kExpTile = 256;                    // channels and positions per workgroup
constexpr int kExpK = 32;                        // latents per stage
constexpr int kExpStages = kLatent / kExpK;      // 16
constexpr int kExpRing = 4;                      // stage buffers; three stages in flight
constexpr int kExpRowBytes = kExpK * 2;          // 64 bytes: 4 chunks of 16
constexpr int kExpTileBytes = kExpTile * kExpRowBytes;  // 16 KiB per operand
constexpr int kExpCopies = 2 * kExpTileBytes / 1024 / 8;  // copy instructions per wave per stage (4)
constexpr int kExpOutRows = kExpTile / 2;        // output rows staged per half
constexpr int kExpOutStride = 2 * kExpTile + 16;  // bytes per staged output row
static_assert(kExpOutRows * kExpOutStride <= kExpRing * 2 * kExpTileBytes, "output staged in the ring");

// chunk c of tile row r sits at slot c ^ ((r >> 2) & 3): the sixteen rows read by one quarter of
// an MFMA operand read (64-byte rows, four per 256 bytes) then fall in sixteen different 16-byte
// bank groups
__device__ __forceinline__ int row64_swz(int r) { return (r >> 2) & 3; }

// VT = false: keys, K[b][position][h * D + d], each output row a position.  VT = true: values
// transposed, V^T[b][h * D + d][position], each output row a channel.
template <bool VT>
__global__ __launch_bounds__(512) void expand_kv_kernel(ExpandArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kExpRing][2][kExpTileBytes];  // [stage][W, latents]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kExpTile;          // weight rows (h*D + d)
  const int m0 = blockIdx.y * kExpTile;          // positions
  const int b = blockIdx.z;
  const int L = min(a.cache_len[b], a.max_cache_len);
  if (m0 >= L) return;  // uniform over the block
  const uint16_t* w = (VT ? a.w_v : a.w_k) + (size_t)n0 * kLatent;
  const uint8_t* c = a.cache + (size_t)b * a.cache_bstride_bytes;

  // one copy instruction moves 16 rows x 64 bytes of one operand; wave v moves rows 32v .. 32v+31
  // of both (lane l: row 16j + l / 4, slot l % 4, holding chunk (l % 4) ^ swz(row))
  auto issue = [&](int st) {
    const int kb = st * kExpRowBytes;
    uint8_t* buf = &lds[st % kExpRing][0][0];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * wave + u;
      const int r = 16 * j + (lane >> 2);
      const int chunk = (lane & 3) ^ row64_swz(r);
      copy16_to_lds((const uint8_t*)(w + (size_t)r * kLatent) + kb + 16 * chunk, lds_addr(buf + 1024 * j));
      const int pr = min(m0 + r, L - 1);
      copy16_to_lds(c + (size_t)pr * kRowBytes + kb + 16 * chunk, lds_addr(buf + kExpTileBytes + 1024 * j));
    }
  };
  static_assert(kExpCopies == 4, "two rows of copies per operand per wave");

  const int wn = wave & 3, wm = wave >> 2;       // this wave: channels 64wn .., positions 128wm ..
  const int r32 = lane & 31, kg = lane >> 5;
  f32x16 acc[2][4];                              // [channel block][position block]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[x][y][e] = 0.f;

#pragma unroll
  for (int st = 0; st < kExpRing - 1; ++st) issue(st);
  for (int st = 0; st < kExpStages; ++st) {
    // stage st has landed; the stages after it may stay in flight
    if (st + 2 < kExpStages) wait_vmcnt<2 * kExpCopies>();
    else if (st + 1 < kExpStages) wait_vmcnt<kExpCopies>();
    else wait_vmcnt<0>();
    __syncthreads();  // stage st is in LDS for every wave; every wave is done with stage st - 1
    if (st + kExpRing - 1 < kExpStages) issue(st + kExpRing - 1);  // into the buffer of stage st - 1
    const uint8_t* wt = &lds[st % kExpRing][0][0];
    const uint8_t* ct = &lds[st % kExpRing][1][0];
#pragma unroll
    for (int s = 0; s < kExpK / 16; ++s) {  // k-steps of 16 latents: chunk 2s + kg
      const int chunk = 2 * s + kg;
      bf16x8 fw[2], fc[4];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int rw = 64 * wn + 32 * x + r32;
        fw[x] = *(const bf16x8*)(wt + rw * kExpRowBytes + 16 * (chunk ^ row64_swz(rw)));
      }
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int rc = 128 * wm + 32 * y + r32;
        fc[y] = *(const bf16x8*)(ct + rc * kExpRowBytes + 16 * (chunk ^ row64_swz(rc)));
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          if constexpr (VT)
            acc[x][y] = mfma32(fc[y], fw[x], acc[x][y]);  // [positions][channels]
          else
            acc[x][y] = mfma32(fw[x], fc[y], acc[x][y]);  // [channels][positions]
        }
    }
  }

  // The tile leaves through LDS, half of its output rows at a time.  Every output row (a position
  // of the keys, a channel of the transposed values) holds 256 values, 512 contiguous bytes in
  // memory, written by 32 lanes with 16-byte stores; written straight from the accumulators, each
  // store would put 8 bytes into each of 32 rows 16-32 KiB apart.  Staged rows are kExpOutStride
  // bytes apart, so that the 8-byte writes of consecutive rows spread over the banks.
  uint8_t* stage = &lds[0][0][0];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    __syncthreads();  // every wave is done reading the ring, or the previous half is written out
    // D lane layout: column lane & 31, rows 8i + 4kg + j.  VT: output rows are channels 64wn +
    // 32x + r32, the lane's four values positions 128wm + 32y + 8i + 4kg ..; otherwise output rows
    // are positions 128wm + 32y + r32 and the values channels 64wn + 32x + 8i + 4kg ..
    const bool mine = VT ? (wn >> 1) == half : wm == half;
    if (mine) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t lo = (uint32_t)f32_to_bf16_bits(acc[x][y][4 * i]) |
                                ((uint32_t)f32_to_bf16_bits(acc[x][y][4 * i + 1]) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_bits(acc[x][y][4 * i + 2]) |
                                ((uint32_t)f32_to_bf16_bits(acc[x][y][4 * i + 3]) << 16);
            const int row = VT ? 64 * wn + 32 * x + r32 : 128 * wm + 32 * y + r32;
            const int col = VT ? 128 * wm + 32 * y + 8 * i + 4 * kg : 64 * wn + 32 * x + 8 * i + 4 * kg;
            *(uint2*)(stage + (row - kExpOutRows * half) * kExpOutStride + 2 * col) = uint2{lo, hi};
          }
    }
    __syncthreads();
    for (int q = threadIdx.x; q < kExpOutRows * 32; q += 512) {
      const int row = q >> 5, ch = q & 31;
      const int orow = kExpOutRows * half + row;
      uint4 v = *(const uint4*)(stage + row * kExpOutStride + 16 * ch);
      if constexpr (VT) {
        // channel n0 + orow (= h * D + d), positions m .. m+7; positions from L up to the next
        // multiple of 64 get zeros: the attention reads whole 64-position spans and multiplies
        // them by zero weights, which must not meet a NaN
        const int m = m0 + 8 * ch;
        const int pad_end = min((L + 63) & ~63, a.vt_len);
        uint16_t* dst = a.v_out + (size_t)b * a.vt_bstride + (size_t)(n0 + orow) * a.vt_len + m;
        if (m + 7 < L) {
          *(uint4*)dst = v;
        } else if (m < pad_end) {
          uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (m + e >= L) wd[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          *(uint4*)dst = uint4{wd[0], wd[1], wd[2], wd[3]};
        }
      } else {
        const int m = m0 + orow;
        if (m < L) *(uint4*)(a.k_out + (size_t)b * a.k_bstride + (size_t)m * a.HD + n0 + 8 * ch) = v;
      }
    }
  }
}

// ------------------------------------------------------------------------------ attention
// chunk c of a 128-byte tile row r sits at slot c ^ ((r >> 1) & 7): sixteen consecutive rows at
// one chunk (an MFMA operand read) then fall in sixteen different 16-byte bank groups
__device__ __forceinline__ int row128_swz(int r) { return (r >> 1) & 7; }

constexpr int kNaWaves = 8;
constexpr int kNaQ = 16 * kNaWaves;        // queries per workgroup
constexpr int kNaKeys = 64;                // keys per tile
constexpr int kNaKRow = kHeadDim * 2;      // 512-byte key rows
constexpr int kNaVRow = kNaKeys * 2;       // 128-byte rows of the transposed value tile
constexpr int kNaStage = kNaKeys * kNaKRow;  // 32 KiB, and the same for the value tile
constexpr int kNaPStride = 72;             // bf16 per P row (64 + 8 pad: conflict-free)
constexpr float kNaRescale = 8.f;          // lazy rescale threshold, log2 units

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// max / sum over the four lanes l, l^16, l^32, l^48 (one query column of a 16x16 result)
__device__ __forceinline__ float col_max(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  u = __builtin_bit_cast(unsigned, x);
  auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)t[0]), __builtin_bit_cast(float, (unsigned)t[1]));
}
__device__ __forceinline__ float col_sum(float x) {
  unsigned u = __builtin_bit_cast(unsigned, x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
  u = __builtin_bit_cast(unsigned, x);
  auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)t[0]) + __builtin_bit_cast(float, (unsigned)t[1]);
}

__global__ __launch_bounds__(64 * kNaWaves) void naive_attn_kernel(NaiveArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t kt[2][kNaStage];   // keys [64][256], swizzled
  __shared__ __attribute__((aligned(1024))) uint8_t vt[2][kNaStage];   // values^T [256][64], swizzled
  __shared__ __attribute__((aligned(16))) uint16_t pb[kNaWaves][16 * kNaPStride];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i0 = blockIdx.x * kNaQ;
  const int h = blockIdx.y, b = blockIdx.z;
  const int L = min(a.cache_len[b], a.max_cache_len);
  const int ql = lane & 15, g = lane >> 4;
  const int qi = i0 + 16 * wave + ql;              // this lane's query column
  const int t = L - a.Q + qi;                      // its position
  const int t_last = L - a.Q + min(i0 + kNaQ - 1, a.Q - 1);
  const int ntiles = t_last >= 0 ? t_last / kNaKeys + 1 : 0;

  const uint8_t* kbase = (const uint8_t*)(a.k + (size_t)b * a.k_bstride + (size_t)h * kHeadDim);
  const uint8_t* vbase = (const uint8_t*)(a.vt + (size_t)b * a.vt_bstride + (size_t)h * kHeadDim * a.vt_len);
  // copies: key tile = 32 instructions of two 512-byte rows, value tile = 32 of eight 128-byte
  // rows; wave w issues instructions 4w .. 4w+3 of each
  auto issue = [&](int tile, int buf) {
    const int key0 = tile * kNaKeys;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = wave * 4 + u;
      {
        const int r = 2 * j + (lane >> 5);
        const int key = min(key0 + r, L - 1);
        const int chunk = (lane & 31) ^ (r & 15);
        copy16_to_lds(kbase + (size_t)key * a.HD * 2 + 16 * chunk, lds_addr(&kt[buf][1024 * j]));
      }
      {
        const int r = 8 * j + (lane >> 3);  // head dimension row of V^T
        const int chunk = (lane & 7) ^ row128_swz(r);
        // positions key0 .. key0+63 (vt_len is a multiple of 64, so the span is inside the row;
        // positions from the length to the next multiple of 64 hold zeros, written by the expansion)
        copy16_to_lds(vbase + ((size_t)r * a.vt_len + key0) * 2 + 16 * chunk, lds_addr(&vt[buf][1024 * j]));
      }
    }
  };

  // queries as the B operand of S^T = K Q^T: lane (column q, group g) holds d = 32s + 8g .. +7
  bf16x8 qf[8];
  {
    const int qc = min(qi, a.Q - 1);
    const uint16_t* src = a.q + (((size_t)b * a.Q + qc) * a.H + h) * kHeadDim + 8 * g;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *(const bf16x8*)(src + 32 * s);
  }
  f32x4 o[16];
#pragma unroll
  for (int db = 0; db < 16; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  uint16_t* pw = pb[wave];

  if (ntiles > 0) issue(0, 0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int buf = tile & 1;
    wait_vmcnt<0>();
    __syncthreads();
    if (tile + 1 < ntiles) issue(tile + 1, buf ^ 1);
    const int key0 = tile * kNaKeys;
    // S^T[64 keys x 16 queries]: lane holds keys 16kb + 4g + j of column q
    f32x4 sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * kb + ql;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 kf = *(const bf16x8*)&kt[buf][r * kNaKRow + 16 * ((4 * s + g) ^ (r & 15))];
        sc[kb] = mfma16(kf, qf[s], sc[kb]);
      }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = key0 + 16 * kb + 4 * g + j;
        const float v = (key <= t && key < L) ? sc[kb][j] * a.scale_log2 : -INFINITY;
        sc[kb][j] = v;
        mt = fmaxf(mt, v);
      }
    mt = col_max(mt);
    // lazy rescale: move the running maximum only when the tile's exceeds it by 2^8
    const bool grow = mt > m_run + kNaRescale;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mt : m_run;
      const float alpha = grow ? exp2f(m_run - m_new) : 1.f;  // 0 on the first tile (m_run = -inf)
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 16; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    // P = exp2(s - m), bf16, to this wave's LDS rows (query q, keys 16kb + 4g .. +3)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        p[j] = exp2f(sc[kb][j] - m_run);
        l_run += p[j];
      }
      const uint32_t lo = (uint32_t)f32_to_bf16_bits(p[0]) | ((uint32_t)f32_to_bf16_bits(p[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(p[2]) | ((uint32_t)f32_to_bf16_bits(p[3]) << 16);
      *(uint2*)&pw[ql * kNaPStride + 16 * kb + 4 * g] = uint2{lo, hi};
    }
    // P^T as the B operand: lane (q, g) holds keys 32ks + 8g .. +7 of its query
    bf16x8 pf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) pf[ks] = *(const bf16x8*)&pw[ql * kNaPStride + 32 * ks + 8 * g];
    // O^T[256 d x 16 q] += V^T[256 x 64] P^T[64 x 16]; A operand: row d = 16db + ql, keys 32ks + 8g
#pragma unroll
    for (int db = 0; db < 16; ++db) {
      const int r = 16 * db + ql;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 vf = *(const bf16x8*)&vt[buf][r * kNaVRow + 16 * ((4 * ks + g) ^ row128_swz(r))];
        o[db] = mfma16(vf, pf[ks], o[db]);
      }
    }
  }

  const float l_all = col_sum(l_run);
  if (qi < a.Q) {
    const float inv = 1.f / l_all;
    float* dst = a.out + (((size_t)b * a.Q + qi) * a.H + h) * kHeadDim + 4 * g;
#pragma unroll
    for (int db = 0; db < 16; ++db) *(f32x4*)(dst + 16 * db) = o[db] * inv;
    if (a.lse && g == 0) a.lse[((size_t)b * a.Q + qi) * a.H + h] = (m_run + __log2f(l_all)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_expand_kv(const ExpandArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<ExpandArgs*>(&a)};
  const dim3 grid(a.HD / kExpTile, (a.max_cache_len + kExpTile - 1) / kExpTile, a.B), block(512);
  hipError_t e = hipLaunchKernel((const void*)&expand_kv_kernel<false>, grid, block, args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)&expand_kv_kernel<true>, grid, block, args, 0, stream);
}

hipError_t launch_naive_attn(const NaiveArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<NaiveArgs*>(&a)};
  const dim3 grid((a.Q + kNaQ - 1) / kNaQ, a.H, a.B), block(64 * kNaWaves);
  return hipLaunchKernel((const void*)&naive_attn_kernel, grid, block, args, 0, stream);
}

}  // namespace mla
