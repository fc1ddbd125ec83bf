// Latent down-projection with cache append for gfx950 (page "Module 05 -- MLA: Compressing
// Per-Token History", section 1: each token is projected down to one shared latent and that
// latent is what the cache keeps; page "Module 08 -- Vision, MTP, and Hybrid Serving State",
// section 1: hidden width 4096).
//
//   c[n][r] = sum_k W[r][k] h[n][k]   (fp32), stored as bf16 (nearest, ties to even) at
//   cache[b][cache_len[b] - Q + i][r] for token n = b*Q + i.
//
// A workgroup owns 16 latent channels (one 16 x 4096 slab of W, 128 KiB) and sixteen waves; wave
// w holds the slab's K-slice 256w .. 256w+255 in 32 VGPRs for the whole kernel, so W is read from
// memory once per workgroup however many tokens it projects.  For each tile of 16 tokens every
// wave multiplies its K-slice (8 MFMA 16x16x32, k in natural order) and the sixteen partial tiles
// are summed through LDS in wave order: the result of a token depends only on its own hidden
// state and W, never on the batch it came in.
//
// Operands reach registers through a private 8 KiB LDS stage per wave: each copy instruction
// moves two 512-byte row slices (1 KiB, whole 128-byte lines) straight from memory into LDS, with
// 16-byte chunk c of row r stored at slot c ^ r, so that the MFMA-layout reads (16 rows at one
// chunk) fall in sixteen different bank groups.
#include "mla_device.h"
#include "mla_internal.h"

namespace mla {

namespace {

constexpr int kDownCols = 16;              // latent channels per workgroup
constexpr int kDownWaves = 16;
constexpr int kDownThreads = 64 * kDownWaves;
constexpr int kSlice = kHidden / kDownWaves;  // K per wave
constexpr int kSteps = kSlice / 32;           // MFMA 16x16x32 per tile
constexpr int kSliceBytes = kSlice * 2;       // one row's slice: 32 chunks of 16 bytes
constexpr int kStageBytes = 16 * kSliceBytes;

static_assert(kSlice == 256 && kSteps == 8, "lane k-ranges assume a 256-wide slice");

__device__ __forceinline__ f32x4 mfma16x16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Stage 16 rows' K-slices (row r at `rows + r * kHidden` elements) into this wave's LDS stage.
// Copy j moves rows 2j and 2j+1: lane l takes row 2j + (l >> 5) and fills slot l & 31 with chunk
// (l & 31) ^ row.  Rows at or past nrows_valid are read from the last valid row.
__device__ __forceinline__ void stage_rows(const uint16_t* rows, int nrows_valid, uint32_t st, int lane) {
  const int slot = lane & 31, half = lane >> 5;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 2 * j + half;
    const int rc = r < nrows_valid ? r : nrows_valid - 1;
    const uint8_t* src = (const uint8_t*)(rows + (size_t)rc * kHidden) + 16 * (slot ^ r);
    copy16_to_lds(src, st + 1024 * j);
  }
}

// operand fragment for MFMA step s: row m, chunk 4s + g (k = 32s + 8g .. +7 of the slice)
__device__ __forceinline__ bf16x8 stage_read(const uint8_t* stage, int m, int g, int s) {
  return *(const bf16x8*)(stage + m * kSliceBytes + 16 * ((4 * s + g) ^ m));
}

__global__ __launch_bounds__(kDownThreads) void latent_down_kernel(DownArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[kDownWaves][kStageBytes];  // 128 KiB
  __shared__ f32x4 red[kDownWaves][kDownCols][4];  // [wave][channel][tokens / 4]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int m = lane & 15, g = lane >> 4;
  const int r0 = blockIdx.x * kDownCols;
  const uint8_t* my = stage[wave];
  const uint32_t st = lds_addr(my);

  bf16x8 wb[kSteps];
  stage_rows(a.w + (size_t)r0 * kHidden + wave * kSlice, 16, st, lane);
  wait_vmcnt<0>();
#pragma unroll
  for (int s = 0; s < kSteps; ++s) wb[s] = stage_read(my, m, g, s);

  const int rows = a.B * a.Q;
  const int ntiles = (rows + 15) / 16;
  for (int tile = blockIdx.y; tile < ntiles; tile += gridDim.y) {
    wait_lds_reads();  // the stage is rewritten below
    stage_rows(a.h + (size_t)tile * 16 * kHidden + wave * kSlice, min(16, rows - tile * 16), st, lane);
    wait_vmcnt<0>();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) acc = mfma16x16(stage_read(my, m, g, s), wb[s], acc);
    // lane holds channel r0 + m of tokens 16 tile + 4g + j
    red[wave][m][g] = acc;
    __syncthreads();
    if (threadIdx.x < 16 * kDownCols) {
      const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
      const float* part = (const float*)&red[0][col][0] + row;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kDownWaves; ++w) sum += part[w * kDownCols * 16];
      const int nn = tile * 16 + row;
      if (nn < rows) {
        const int b = nn / a.Q, i = nn - b * a.Q;
        const int pos = min(a.cache_len[b], a.max_cache_len) - a.Q + i;
        if (pos >= 0) a.cache[(size_t)b * a.cache_bstride + (size_t)pos * kLatent + r0 + col] = f32_to_bf16_bits(sum);
      }
    }
    __syncthreads();  // red is rewritten by the next tile
  }
}

// ---------------------------------------------------------------------- long passes (prefill)
// A tiled product for passes of many tokens: a workgroup owns 64 tokens x 128 channels, four
// waves of 32 channels x 64 tokens, and streams the hidden dimension through LDS 64 at a time
// (a ring of four stages, three in flight while one is multiplied: with one stage in flight the
// copies' latency set the pace; one copy instruction per 8 rows x 128 bytes, chunk c of row r at
// slot c ^ ((r >> 1) & 7)).  The sum keeps latent_down_kernel's order exactly: per K-slice of 256 a
// partial from zero over the same eight MFMA 16x16x32 k-steps, the partials added to the total in
// slice order, so a token gets the same bits in either kernel.  The operands are swapped (W rows
// as A, tokens as B), so each lane holds four consecutive channels of one token and stores them
// as one 8-byte write.
constexpr int kGemmM = 64;                          // tokens per workgroup
constexpr int kGemmN = 128;                         // channels per workgroup
constexpr int kGemmK = 64;                          // hidden per stage
constexpr int kGemmRowBytes = kGemmK * 2;           // 128 bytes: 8 chunks of 16
constexpr int kGemmStages = kHidden / kGemmK;       // 64
constexpr int kStagesPerSlice = kSlice / kGemmK;    // 4
constexpr int kGemmRing = 4;                        // stages held in LDS: three in flight, one in use
constexpr int kGemmCopies = 6;                      // copy instructions per wave per stage
static_assert(kSlice % kGemmK == 0 && kGemmK % 32 == 0, "a stage holds whole k-steps of one slice");

__device__ __forceinline__ int gemm_swz(int r) { return (r >> 1) & 7; }

__global__ __launch_bounds__(256) void down_gemm_kernel(DownArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t ldsW[kGemmRing][kGemmN * kGemmRowBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t ldsH[kGemmRing][kGemmM * kGemmRowBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * kGemmN;  // channels
  const int m0 = blockIdx.y * kGemmM;  // tokens
  const int rows = a.B * a.Q;

  auto issue = [&](int st, int buf) {
    const int kb = st * kGemmRowBytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {  // W: 16 copies of 8 rows, four per wave
      const int j = wave * 4 + u;
      const int r = 8 * j + (lane >> 3);
      const int chunk = (lane & 7) ^ gemm_swz(r);
      copy16_to_lds((const uint8_t*)(a.w + (size_t)(n0 + r) * kHidden) + kb + 16 * chunk, lds_addr(&ldsW[buf][1024 * j]));
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {  // tokens: 8 copies of 8 rows, two per wave; rows past the pass repeat its last
      const int j = wave * 2 + u;
      const int r = 8 * j + (lane >> 3);
      const int chunk = (lane & 7) ^ gemm_swz(r);
      const int tok = min(m0 + r, rows - 1);
      copy16_to_lds((const uint8_t*)(a.h + (size_t)tok * kHidden) + kb + 16 * chunk, lds_addr(&ldsH[buf][1024 * j]));
    }
  };

  const int ql = lane & 15, g = lane >> 4;
  f32x4 total[2][4], part[2][4];  // [channel block x][token block y]
#pragma unroll
  for (int x = 0; x < 2; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) total[x][y] = part[x][y] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int st = 0; st < kGemmRing - 1; ++st) issue(st, st);
  for (int st = 0; st < kGemmStages; ++st) {
    const int buf = st % kGemmRing;
    // stage st has landed once at most the stages issued after it are in flight
    if (st + 2 < kGemmStages) wait_vmcnt<2 * kGemmCopies>();
    else if (st + 1 < kGemmStages) wait_vmcnt<kGemmCopies>();
    else wait_vmcnt<0>();
    __syncthreads();  // stage st landed for every wave; every wave is done reading stage st - 1
    // into the buffer of stage st - 1, which every wave finished reading before the barrier
    if (st + kGemmRing - 1 < kGemmStages) issue(st + kGemmRing - 1, (st + kGemmRing - 1) % kGemmRing);
    if (st % kStagesPerSlice == 0) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) part[x][y] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < kGemmK / 32; ++ks) {  // k = 32ks + 8g + e within the stage
      const int chunk = 4 * ks + g;
      bf16x8 fw[2], fh[4];
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int r = 32 * wave + 16 * x + ql;
        fw[x] = *(const bf16x8*)&ldsW[buf][r * kGemmRowBytes + 16 * (chunk ^ gemm_swz(r))];
      }
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int r = 16 * y + ql;
        fh[y] = *(const bf16x8*)&ldsH[buf][r * kGemmRowBytes + 16 * (chunk ^ gemm_swz(r))];
      }
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) part[x][y] = mfma16x16(fw[x], fh[y], part[x][y]);
    }
    if (st % kStagesPerSlice == kStagesPerSlice - 1) {  // a slice is complete: add it in slice order
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) total[x][y] += part[x][y];
    }
  }
  // lane holds channels n0 + 32 wave + 16x + 4g .. +3 of token m0 + 16y + ql
#pragma unroll
  for (int y = 0; y < 4; ++y) {
    const int nn = m0 + 16 * y + ql;
    if (nn >= rows) continue;
    const int b = nn / a.Q, i = nn - b * a.Q;
    const int pos = min(a.cache_len[b], a.max_cache_len) - a.Q + i;
    if (pos < 0) continue;
    uint16_t* dst = a.cache + (size_t)b * a.cache_bstride + (size_t)pos * kLatent + n0 + 32 * wave + 4 * g;
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const uint32_t lo = (uint32_t)f32_to_bf16_bits(total[x][y][0]) | ((uint32_t)f32_to_bf16_bits(total[x][y][1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_bits(total[x][y][2]) | ((uint32_t)f32_to_bf16_bits(total[x][y][3]) << 16);
      *(uint2*)(dst + 16 * x) = uint2{lo, hi};
    }
  }
}

}  // namespace

int down_row_groups(int rows) {
  const int ntiles = (rows + 15) / 16;
  return ntiles < 32 ? ntiles : 32;
}

hipError_t launch_latent_down(const DownArgs& a, hipStream_t stream) {
  void* args[] = {const_cast<DownArgs*>(&a)};
  const int rows = a.B * a.Q;
  if (rows >= kDownGemmMinRows) {
    const dim3 grid(kLatent / kGemmN, (rows + kGemmM - 1) / kGemmM), block(256);
    return hipLaunchKernel((const void*)&down_gemm_kernel, grid, block, args, 0, stream);
  }
  const dim3 grid(kLatent / kDownCols, down_row_groups(a.B * a.Q)), block(kDownThreads);
  return hipLaunchKernel((const void*)&latent_down_kernel, grid, block, args, 0, stream);
}

}  // namespace mla
