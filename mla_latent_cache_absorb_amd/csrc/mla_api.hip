// C ABI of libmla_absorb (declared in include/mla_absorb.h): argument validation, device
// checks, split sizing and kernel launches.  Every call validates on the host first and
// enqueues nothing on error; it never allocates, synchronises or keeps per-call state.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "mla_absorb.h"
#include "mla_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// per device: 0 = unknown, 1 = gfx950, -1 = other; compute-unit count
std::atomic<int> g_dev_ok[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];

int check_device(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  int ok = g_dev_ok[dev].load(std::memory_order_acquire);
  if (ok == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_dev_ok[dev].store(ok, std::memory_order_release);
  }
  if (ok != 1) return MLA_ERR_DEVICE;
  if (cus) *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
  return MLA_OK;
}

// The split count.  Independent work units are (sequence, query unit, 64-head group), a
// query unit being one query, or two adjacent queries of one sequence in dense calls with an
// even Q (mla::query_units); the positions of each unit are cut into `s` contiguous splits of
// whole tiles, one workgroup per CU.  The estimate charges the rounds of resident workgroups
// times the tiles of one split, plus the partial results each extra split writes and the
// merge reads back (priced as four 32 KiB tiles each way per query; measured sweeps of the
// split count agree with this weight) and a fixed cost for the merge launch.
int32_t choose_splits(int64_t units, int32_t max_positions, int cus) {
  const int64_t tiles = (max_positions + mla::kTilePositions - 1) / mla::kTilePositions;
  const int64_t slots = cus > 0 ? cus : 256;
  const int64_t smax = tiles < mla::kMaxSplits ? tiles : mla::kMaxSplits;
  int32_t best = 1;
  double best_cost = 1e300;
  for (int64_t s = 1; s <= smax; ++s) {
    const int64_t per = (tiles + s - 1) / s;
    if ((s - 1) * per >= tiles) continue;  // would leave an empty split
    const int64_t rounds = (units * s + slots - 1) / slots;
    double cost = (double)rounds * (double)per;
    if (s > 1) cost += (double)(units * s * 8) / (double)slots + 3.0;
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = (int32_t)s;
    }
  }
  return best;
}

// positions per split (whole tiles) for a split count
int32_t split_length(int32_t max_positions, int32_t s) {
  const int32_t tiles = (max_positions + mla::kTilePositions - 1) / mla::kTilePositions;
  const int32_t per = (tiles + s - 1) / s;
  return per * mla::kTilePositions;
}

bool supported(int32_t H, int32_t D, int32_t R) { return R == 512 && D == 256 && H > 0 && H % 16 == 0; }

// head groups of the attention kernels: 64 heads each, the last one possibly partial
int32_t head_groups(int32_t H) { return (H + 63) / 64; }

// the choice depends on the workgroup count per split (one per sequence, 64-head group and query,
// or pair of queries for dense calls with two or more) and the tiles only
int resolve_splits(int32_t B, int32_t Q, int32_t H, int32_t max_positions, int32_t num_splits, int cus,
                   bool indexed) {
  if (B < 1 || Q < 1 || H < 16 || H % 16 != 0 || max_positions < 1) return MLA_ERR_SHAPE;
  if (num_splits < 0) return MLA_ERR_ARG;
  const int32_t tiles = (max_positions + mla::kTilePositions - 1) / mla::kTilePositions;
  int32_t s;
  if (num_splits == 0) {
    s = choose_splits((int64_t)B * mla::query_units(indexed, Q) * head_groups(H), max_positions, cus);
  } else {
    s = num_splits > mla::kMaxSplits ? mla::kMaxSplits : num_splits;
    if (s > tiles) s = tiles;
  }
  // drop splits that would be empty once the positions are cut into whole tiles
  const int32_t len = split_length(max_positions, s);
  return (max_positions + len - 1) / len;
}

// split partials: fp16 normalised latents, then fp32 (m, l) per row
size_t workspace_bytes_for(int32_t B, int32_t Q, int32_t H, int32_t s) {
  if (s <= 1) return 0;
  const size_t rows = (size_t)s * B * Q * H;
  return rows * 512 * sizeof(uint16_t) + rows * 2 * sizeof(float);
}

// with the up-projection fused: the partials, or for one split the accumulated latents
size_t fused_workspace_bytes_for(int32_t B, int32_t Q, int32_t H, int32_t s) {
  return s > 1 ? workspace_bytes_for(B, Q, H, s) : (size_t)B * Q * H * 512 * sizeof(float);
}

// ---- fixed scratch of the no-allocation entry point (mla_latent_attn_up_v_noalloc)
// The array's name is a host-side stand-in in host code, not a device address: host code uses only
// the per-device address hipGetSymbolAddress returns (each GPU holds its own copy of the array).
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// the current device's copy of `scratch`, resolved once per device with that device current
int scratch_for_current_device(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return MLA_OK;
}

int device_cus_or_default() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices) {
    cus = g_dev_cus[dev].load(std::memory_order_relaxed);
    if (cus == 0 && hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      g_dev_cus[dev].store(cus, std::memory_order_relaxed);
  }
  return cus > 0 ? cus : 256;
}

int attn_common(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache, int64_t cache_batch_stride,
                const int32_t* cache_len,
                const int32_t* idx, const int32_t* idx_len, int32_t K_max, bool indexed, int32_t B, int32_t Q,
                int32_t H, int32_t R, int32_t max_cache_len, float scale, int32_t num_splits, float* o_lat,
                float* lse, void* workspace, size_t workspace_bytes, void* stream, const uint16_t* w_v = nullptr,
                float* out = nullptr, bool fixed_scratch = false) {
  // w_v != null: the up-projection follows, fused with the split merge, and writes `out`;
  // fixed_scratch: the partials go to the library's own scratch (workspace arguments ignored)
  const bool fused = w_v != nullptr;
  if (!q_abs || !cache || !cache_len || (fused ? !out : !o_lat)) return MLA_ERR_NULL;
  if (indexed && (!idx || !idx_len)) return MLA_ERR_NULL;
  if (!supported(H, 256, R) || B < 1 || Q < 1 || max_cache_len < 1) return MLA_ERR_SHAPE;
  if (max_cache_len < Q) return MLA_ERR_ARG;
  if (cache_batch_stride < (int64_t)max_cache_len * R) return MLA_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return MLA_ERR_ARG;
  if (indexed && K_max < 1) return MLA_ERR_ARG;
  if (num_splits < 0) return MLA_ERR_ARG;
  int cus = 0;
  const int dst = check_device(&cus);
  if (dst != MLA_OK) return dst;
  const int32_t max_positions = indexed ? K_max : max_cache_len;
  const int s = resolve_splits(B, Q, H, max_positions, num_splits, cus, indexed);
  if (s < 1) return s;
  const size_t need = fused ? fused_workspace_bytes_for(B, Q, H, s) : workspace_bytes_for(B, Q, H, s);
  if (fixed_scratch) {
    if (need > kScratchBytes) return MLA_ERR_SCRATCH;
    const int sst = scratch_for_current_device(&workspace);
    if (sst != MLA_OK) return sst;
    workspace_bytes = kScratchBytes;
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return MLA_ERR_WORKSPACE;
  // a two-term query runs every query in a workgroup of its own (same split count)
  const int64_t units = q_abs_lo != nullptr ? Q : mla::query_units(indexed, Q);
  const int64_t total = (int64_t)B * units * head_groups(H) * s;
  if (total > 0x7fffffff || (int64_t)B * Q * H > 0x7fffffff) return MLA_ERR_SHAPE;

  mla::AttnArgs a;
  a.q_abs = q_abs;
  a.q_abs_lo = q_abs_lo;
  a.cache = (const uint8_t*)cache;
  a.cache_bstride_bytes = cache_batch_stride * 2;
  a.cache_len = cache_len;
  a.idx = idx;
  a.idx_len = idx_len;
  a.K_max = indexed ? K_max : 0;
  a.B = B;
  a.Q = Q;
  a.H = H;
  a.HG = head_groups(H);
  a.max_cache_len = max_cache_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_splits = s;
  a.split_len = split_length(max_positions, s);
  a.total_wg = (int32_t)total;
  // one workgroup per (sequence, split): no other workgroup reads its rows, so they are streamed
  // non-temporally; with several queries or head groups per sequence the rows are shared in L2
  a.stream_once = units * head_groups(H) == 1;
  a.o_lat = fused ? (s > 1 ? nullptr : (float*)workspace) : o_lat;
  a.lse = lse;
  const size_t rows = (size_t)s * B * Q * H;
  a.part_o = s > 1 ? (uint16_t*)workspace : nullptr;
  a.part_ml = s > 1 ? (float*)((uint8_t*)workspace + rows * 512 * sizeof(uint16_t)) : nullptr;

  hipStream_t st = (hipStream_t)stream;
  if (mla::launch_latent_attn(a, indexed, st) != hipSuccess) return MLA_ERR_HIP;
  if (!fused) {
    if (s > 1 && mla::launch_combine(a, st) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
  }
  if (s == 1) return mla::launch_up_v(a.o_lat, w_v, out, B * Q, H, cus, st) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  mla::MergeUpArgs m{};
  m.part_o = a.part_o;
  m.part_ml = a.part_ml;
  m.num_splits = s;
  m.rows = B * Q;
  m.H = H;
  m.w_v = w_v;
  m.out = out;
  m.lse = lse;
  return mla::launch_merge_up_v(m, cus, st) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_NULL: return "a required pointer is NULL";
    case MLA_ERR_SHAPE: return "unsupported shape (need R == 512, D == 256, H a positive multiple of 16, sizes >= 1)";
    case MLA_ERR_ARG: return "argument out of range";
    case MLA_ERR_WORKSPACE: return "workspace too small";
    case MLA_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case MLA_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case MLA_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point holds (64 MiB)";
    default: return "unknown status";
  }
}

int mla_absorb_q(const uint16_t* q, const uint16_t* w_k, uint16_t* q_abs, uint16_t* q_abs_lo, int32_t rows,
                 int32_t H, int32_t D, int32_t R, float prescale, void* stream) {
  if (!q || !w_k || !q_abs) return MLA_ERR_NULL;
  if (!supported(H, D, R) || rows < 1 || (int64_t)rows * H > 0x7fffffff) return MLA_ERR_SHAPE;
  if (!isfinite(prescale)) return MLA_ERR_ARG;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  if (mla::launch_absorb_q(q, w_k, q_abs, q_abs_lo, rows, H, prescale, (hipStream_t)stream) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int32_t mla_latent_attn_num_splits(int32_t B, int32_t Q, int32_t H, int32_t max_positions, int32_t num_splits,
                                   int32_t indexed) {
  return resolve_splits(B, Q, H, max_positions, num_splits, device_cus_or_default(), indexed != 0);
}

size_t mla_latent_attn_workspace_size(int32_t B, int32_t Q, int32_t H, int32_t R, int32_t max_positions,
                                      int32_t num_splits, int32_t indexed) {
  if (R != 512) return 0;
  const int s = resolve_splits(B, Q, H, max_positions, num_splits, device_cus_or_default(), indexed != 0);
  if (s < 1) return 0;
  return workspace_bytes_for(B, Q, H, s);
}

int mla_latent_attn(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache, int64_t cache_batch_stride,
                    const int32_t* cache_len, int32_t B, int32_t Q, int32_t H, int32_t R, int32_t max_cache_len,
                    float scale, int32_t num_splits, float* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return attn_common(q_abs, q_abs_lo, cache, cache_batch_stride, cache_len, nullptr, nullptr, 0, false, B, Q, H, R,
                     max_cache_len, scale, num_splits, o_lat, lse, workspace, workspace_bytes, stream);
}

int mla_latent_attn_indexed(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache,
                            int64_t cache_batch_stride, const int32_t* cache_len, const int32_t* idx,
                            const int32_t* idx_len, int32_t K_max, int32_t B, int32_t Q, int32_t H, int32_t R,
                            int32_t max_cache_len, float scale, int32_t num_splits, float* o_lat, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return attn_common(q_abs, q_abs_lo, cache, cache_batch_stride, cache_len, idx, idx_len, K_max, true, B, Q, H, R,
                     max_cache_len, scale, num_splits, o_lat, lse, workspace, workspace_bytes, stream);
}

size_t mla_latent_attn_up_v_workspace_size(int32_t B, int32_t Q, int32_t H, int32_t R, int32_t max_positions,
                                           int32_t num_splits, int32_t indexed) {
  if (R != 512) return 0;
  const int s = resolve_splits(B, Q, H, max_positions, num_splits, device_cus_or_default(), indexed != 0);
  if (s < 1 || B < 1 || Q < 1 || H < 1) return 0;
  return fused_workspace_bytes_for(B, Q, H, s);
}

int mla_latent_attn_up_v(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache,
                         int64_t cache_batch_stride, const int32_t* cache_len, const int32_t* idx, const int32_t* idx_len, int32_t K_max,
                         int32_t B, int32_t Q, int32_t H, int32_t R, int32_t max_cache_len, float scale,
                         int32_t num_splits, const uint16_t* w_v, int32_t D, float* out, float* lse, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (!w_v) return MLA_ERR_NULL;
  if ((idx == nullptr) != (idx_len == nullptr)) return MLA_ERR_NULL;
  if (!supported(H, D, R)) return MLA_ERR_SHAPE;
  return attn_common(q_abs, q_abs_lo, cache, cache_batch_stride, cache_len, idx, idx_len, K_max, idx != nullptr, B,
                     Q, H, R, max_cache_len, scale, num_splits, nullptr, lse, workspace, workspace_bytes, stream, w_v, out);
}

int mla_latent_attn_up_v_noalloc(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache,
                                 int64_t cache_batch_stride, const int32_t* cache_len, const int32_t* idx, const int32_t* idx_len,
                                 int32_t K_max, int32_t B, int32_t Q, int32_t H, int32_t R, int32_t max_cache_len,
                                 float scale, int32_t num_splits, const uint16_t* w_v, int32_t D, float* out,
                                 float* lse, void* stream) {
  if (!w_v) return MLA_ERR_NULL;
  if ((idx == nullptr) != (idx_len == nullptr)) return MLA_ERR_NULL;
  if (!supported(H, D, R)) return MLA_ERR_SHAPE;
  return attn_common(q_abs, q_abs_lo, cache, cache_batch_stride, cache_len, idx, idx_len, K_max, idx != nullptr, B,
                     Q, H, R, max_cache_len, scale, num_splits, nullptr, lse, nullptr, 0, stream, w_v, out, true);
}

int mla_stream_read(const void* src, size_t bytes, uint32_t never, uint32_t* sink, void* stream) {
  if (!src || !sink) return MLA_ERR_NULL;
  if (bytes < mla::kStreamChunkBytes || bytes % mla::kStreamChunkBytes != 0) return MLA_ERR_SHAPE;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  return mla::launch_stream_read(src, bytes, never, sink, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_check_attn_inputs(const int32_t* cache_len, const int32_t* idx, const int32_t* idx_len, int32_t B,
                          int32_t Q, int32_t K_max, int32_t max_cache_len, int32_t* flags, void* stream) {
  static_assert(mla::kBadCacheLenShort == MLA_BAD_CACHE_LEN_SHORT && mla::kBadCacheLenLong == MLA_BAD_CACHE_LEN_LONG &&
                    mla::kBadIdxLen == MLA_BAD_IDX_LEN && mla::kBadIdxRange == MLA_BAD_IDX_RANGE &&
                    mla::kBadIdxOrder == MLA_BAD_IDX_ORDER && mla::kBadIdxCausal == MLA_BAD_IDX_CAUSAL,
                "flag bits");
  if (!cache_len || !flags) return MLA_ERR_NULL;
  if ((idx == nullptr) != (idx_len == nullptr)) return MLA_ERR_NULL;
  if (B < 1 || Q < 1 || max_cache_len < 1) return MLA_ERR_SHAPE;
  if (idx != nullptr && K_max < 1) return MLA_ERR_ARG;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  mla::CheckArgs a{cache_len, idx, idx_len, B, Q, idx ? K_max : 0, max_cache_len, flags};
  return mla::launch_check_inputs(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_kpool_keys(const uint16_t* k, const uint16_t* g, int64_t batch_stride, const int32_t* cache_len,
                   const int32_t* pool_begin, int32_t B, int32_t max_cache_len, int32_t d, int32_t pool,
                   float* pooled, int32_t max_pools, void* stream) {
  if (!k || !g || !cache_len || !pooled) return MLA_ERR_NULL;
  if (B < 1 || max_cache_len < 1 || pool < 1 || max_pools < 1) return MLA_ERR_SHAPE;
  if (!(d == 64 || d == 128 || d == 256)) return MLA_ERR_SHAPE;
  if (batch_stride < (int64_t)max_cache_len * d || batch_stride % 8 != 0) return MLA_ERR_ARG;
  if (max_pools < max_cache_len / pool) return MLA_ERR_ARG;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  mla::KpoolArgs a{k, g, batch_stride, cache_len, pool_begin, B, max_cache_len, d, pool, max_pools, pooled};
  return mla::launch_kpool(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_indexer_scores(const uint16_t* q, const float* pooled, const int32_t* cache_len, int32_t B, int32_t Q,
                       int32_t d, int32_t pool, int32_t max_pools, int32_t max_cache_len, float* scores,
                       void* stream) {
  if (!q || !pooled || !cache_len || !scores) return MLA_ERR_NULL;
  if (B < 1 || Q < 1 || Q > mla::kMaxIndexerQ || pool < 1 || max_pools < 1 || max_cache_len < 1)
    return MLA_ERR_SHAPE;
  if (!(d == 64 || d == 128 || d == 256)) return MLA_ERR_SHAPE;
  if (max_pools < max_cache_len / pool) return MLA_ERR_ARG;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  mla::ScoreArgs a{q, pooled, cache_len, B, Q, d, pool, max_pools, max_cache_len, scores};
  return mla::launch_scores(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_indexer_select(const float* scores, const int32_t* cache_len, int32_t B, int32_t Q, int32_t pool,
                       int32_t max_pools, int32_t max_cache_len, int32_t topk, int32_t tail, int32_t* idx,
                       int32_t* idx_len, int32_t K_max, void* stream) {
  if (!scores || !cache_len || !idx || !idx_len) return MLA_ERR_NULL;
  if (B < 1 || Q < 1 || pool < 1 || max_pools < 1 || max_cache_len < 1) return MLA_ERR_SHAPE;
  if (max_pools > mla::kMaxIndexerPools || max_pools < max_cache_len / pool) return MLA_ERR_ARG;
  if (topk < pool || topk % pool != 0) return MLA_ERR_ARG;
  if (K_max < topk + (tail ? pool - 1 : 0)) return MLA_ERR_ARG;
  if ((int64_t)B * Q > 0x7fffffff) return MLA_ERR_SHAPE;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  mla::SelectArgs a{scores, cache_len, B, Q, pool, max_pools, max_cache_len, topk, tail ? 1 : 0, K_max, idx, idx_len};
  return mla::launch_select(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_latent_append(const uint16_t* h, const uint16_t* w_dkv, uint16_t* cache, int64_t cache_batch_stride,
                      const int32_t* cache_len, int32_t B, int32_t Q, int32_t hidden, int32_t R,
                      int32_t max_cache_len, void* stream) {
  if (!h || !w_dkv || !cache || !cache_len) return MLA_ERR_NULL;
  if (hidden != mla::kHidden || R != 512 || B < 1 || Q < 1 || (int64_t)B * Q > 0x7fffffff)
    return MLA_ERR_SHAPE;
  if (max_cache_len < Q || cache_batch_stride < (int64_t)max_cache_len * R) return MLA_ERR_ARG;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  mla::DownArgs a{h, w_dkv, cache, cache_batch_stride, cache_len, B, Q, max_cache_len};
  if (mla::launch_latent_down(a, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_expand_kv(const uint16_t* cache, int64_t cache_batch_stride, const int32_t* cache_len, const uint16_t* w_k,
                  const uint16_t* w_v, int32_t B, int32_t H, int32_t D, int32_t R, int32_t max_cache_len,
                  uint16_t* k_out, uint16_t* vt_out, int32_t vt_len, void* stream) {
  if (!cache || !cache_len || !w_k || !w_v || !k_out || !vt_out) return MLA_ERR_NULL;
  if (!supported(H, D, R) || B < 1 || max_cache_len < 1) return MLA_ERR_SHAPE;
  if (cache_batch_stride < (int64_t)max_cache_len * R || vt_len < max_cache_len || vt_len % 64 != 0)
    return MLA_ERR_ARG;
  if ((max_cache_len + 127) / 128 > 65535 || B > 65535) return MLA_ERR_SHAPE;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  const int32_t HD = H * D;
  mla::ExpandArgs a{(const uint8_t*)cache, cache_batch_stride * 2, cache_len, w_k, w_v,
                    k_out, (int64_t)max_cache_len * HD, vt_out, (int64_t)HD * vt_len, vt_len,
                    B, HD, max_cache_len};
  return mla::launch_expand_kv(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_naive_attn(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int32_t vt_len, const int32_t* cache_len,
                   int32_t B, int32_t Q, int32_t H, int32_t D, int32_t max_cache_len, float scale, float* out,
                   float* lse, void* stream) {
  if (!q || !k || !vt || !cache_len || !out) return MLA_ERR_NULL;
  if (!supported(H, D, 512) || B < 1 || Q < 1 || max_cache_len < 1) return MLA_ERR_SHAPE;
  if ((int64_t)B * Q * H > 0x7fffffff || B > 65535 || H > 65535) return MLA_ERR_SHAPE;
  if (max_cache_len < Q || vt_len < max_cache_len || vt_len % 64 != 0) return MLA_ERR_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return MLA_ERR_ARG;
  const int dst = check_device(nullptr);
  if (dst != MLA_OK) return dst;
  const int32_t HD = H * D;
  mla::NaiveArgs a{q, k, (int64_t)max_cache_len * HD, vt, (int64_t)HD * vt_len, vt_len, cache_len,
                   B, Q, H, HD, max_cache_len, scale * 1.4426950408889634f, out, lse};
  return mla::launch_naive_attn(a, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

int mla_up_v(const float* o_lat, const uint16_t* w_v, float* out, int32_t rows, int32_t H, int32_t D, int32_t R,
             void* stream) {
  if (!o_lat || !w_v || !out) return MLA_ERR_NULL;
  if (!supported(H, D, R) || rows < 1 || (int64_t)rows * H > 0x7fffffff) return MLA_ERR_SHAPE;
  int cus = 0;
  const int dst = check_device(&cus);
  if (dst != MLA_OK) return dst;
  if (mla::launch_up_v(o_lat, w_v, out, rows, H, cus, (hipStream_t)stream) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

}  // extern "C"
