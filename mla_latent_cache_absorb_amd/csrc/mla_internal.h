// Host-side launch interface between the C ABI (mla_api.cpp) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kTilePositions = 32;    // latent rows per LDS tile
constexpr int kMaxSplits = 1024;

struct AttnArgs {
  const uint16_t* q_abs;          // [B][Q][H][R] bf16
  const uint16_t* q_abs_lo;       // [B][Q][H][R] bf16 second term of the absorbed query, or null
  const uint8_t* cache;           // latent rows (bytes)
  int64_t cache_bstride_bytes;    // bytes between sequences
  const int32_t* cache_len;       // [B]
  const int32_t* idx;             // [B][Q][K_max] (indexed only)
  const int32_t* idx_len;         // [B][Q]        (indexed only)
  int32_t K_max;
  int32_t B, Q, H, HG;            // HG = ceil(H / 64) head groups (H a multiple of 16)
  int32_t max_cache_len;
  float scale_log2;               // softmax scale * log2(e)
  int32_t num_splits, split_len;  // split_len: positions (or index slots) per split, multiple of the tile
  int32_t total_wg;
  int32_t stream_once;            // 1: every cache row is read by one workgroup only (launches the
                                  // split kernel instance whose tile copies are non-temporal)
  float* o_lat;                   // [B][Q][H][R] fp32 (written directly when num_splits == 1)
  float* lse;                     // [B][Q][H] or null
  uint16_t* part_o;               // [S][B*Q][H][R] fp16 bits: the split's normalised partial o / l
  float* part_ml;                 // [S][B*Q][H][2] fp32 (running max in log2 units, sum)
};

// queries one workgroup of the split kernel takes: dense calls with an even number of queries
// per sequence pair adjacent queries, so one run of tiles serves both (with an odd count the lone
// query's workgroup would cost a pair's time for one query's work).  Split counts are planned
// with this form; a call given the second query term runs every query alone (the pair form has
// no registers for a second term) with the same split count.
inline int queries_per_wg(bool indexed, int32_t Q) { return !indexed && Q % 2 == 0 ? 2 : 1; }
// workgroups per (sequence, head group, split)
inline int32_t query_units(bool indexed, int32_t Q) { return queries_per_wg(indexed, Q) == 2 ? (Q + 1) / 2 : Q; }

hipError_t launch_latent_attn(const AttnArgs& a, bool indexed, hipStream_t stream);
hipError_t launch_combine(const AttnArgs& a, hipStream_t stream);
// ---- k-pooled indexer
constexpr int kMaxIndexerPools = 16384;  // selectable pools per query (one LDS key each)
constexpr int kMaxIndexerQ = 8;          // queries per sequence scored together
constexpr int kMaxIndexerDim = 256;      // indexer key width

struct KpoolArgs {
  const uint16_t* k;          // [B][.][d] bf16 indexer keys, batch_stride elements apart
  const uint16_t* g;          // [B][.][d] bf16 gate logits, same layout
  int64_t batch_stride;
  const int32_t* cache_len;   // [B]
  const int32_t* pool_begin;  // [B] first pool to (re)build, or null for 0
  int32_t B, max_cache_len, d, pool, max_pools;
  float* pooled;              // [B][max_pools][d]
};

struct ScoreArgs {
  const uint16_t* q;          // [B][Q][d] bf16
  const float* pooled;        // [B][max_pools][d]
  const int32_t* cache_len;
  int32_t B, Q, d, pool, max_pools, max_cache_len;
  float* scores;              // [B][Q][max_pools]
};

struct SelectArgs {
  const float* scores;        // [B][Q][max_pools]
  const int32_t* cache_len;
  int32_t B, Q, pool, max_pools, max_cache_len, topk, tail, K_max;
  int32_t* idx;               // [B][Q][K_max]
  int32_t* idx_len;           // [B][Q]
};

hipError_t launch_kpool(const KpoolArgs& a, hipStream_t stream);
hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, hipStream_t stream);

// ---- latent down-projection with cache append
constexpr int kHidden = 4096;   // hidden width projected down to the latent
struct DownArgs {
  const uint16_t* h;          // [B*Q][kHidden] bf16 hidden states of the new tokens
  const uint16_t* w;          // [kLatent][kHidden] bf16 projection
  uint16_t* cache;            // latent rows, cache_bstride elements between sequences
  int64_t cache_bstride;
  const int32_t* cache_len;   // [B] lengths after the append
  int32_t B, Q, max_cache_len;
};
int down_row_groups(int rows);
constexpr int kDownGemmMinRows = 2048;  // passes of this many tokens or more use the tiled product
hipError_t launch_latent_down(const DownArgs& a, hipStream_t stream);

// ---- the naive (expanded) form
struct ExpandArgs {
  const uint8_t* cache;          // latent rows (bytes)
  int64_t cache_bstride_bytes;
  const int32_t* cache_len;      // [B]
  const uint16_t* w_k;           // [H*D][R]
  const uint16_t* w_v;           // [H*D][R]
  uint16_t* k_out;               // [B][max_cache_len][H*D]
  int64_t k_bstride;             // elements
  uint16_t* v_out;               // [B][H*D][vt_len] (values transposed)
  int64_t vt_bstride;            // elements
  int32_t vt_len;                // positions per transposed row, a multiple of 64
  int32_t B, HD, max_cache_len;
};
struct NaiveArgs {
  const uint16_t* q;             // [B][Q][H][D] bf16
  const uint16_t* k;             // as ExpandArgs::k_out
  int64_t k_bstride;
  const uint16_t* vt;            // as ExpandArgs::v_out
  int64_t vt_bstride;
  int32_t vt_len;
  const int32_t* cache_len;
  int32_t B, Q, H, HD, max_cache_len;
  float scale_log2;              // softmax scale * log2(e)
  float* out;                    // [B][Q][H][D] fp32
  float* lse;                    // [B][Q][H] or null
};
hipError_t launch_expand_kv(const ExpandArgs& a, hipStream_t stream);
hipError_t launch_naive_attn(const NaiveArgs& a, hipStream_t stream);

hipError_t launch_absorb_q(const uint16_t* q, const uint16_t* w_k, uint16_t* q_abs, uint16_t* q_abs_lo, int rows,
                           int H, float prescale, hipStream_t stream);
hipError_t launch_up_v(const float* o_lat, const uint16_t* w_v, float* out, int rows, int H, int cus,
                       hipStream_t stream);

// the up-projection's arguments: the latents given (o_lat), or split-K partials merged straight
// into it (o_lat null)
struct MergeUpArgs {
  const float* o_lat;      // [rows][H][R] fp32, or null
  const uint16_t* part_o;  // [S][rows][H][R] fp16 bits: normalised partials o / l
  const float* part_ml;    // [S][rows][H][2] fp32 (running max in log2 units, sum)
  int32_t num_splits;
  int32_t rows, H;         // rows = B * Q
  const uint16_t* w_v;     // [H][D][R] bf16
  float* out;              // [rows][H][D] fp32
  float* lse;              // [rows][H] fp32 or null
  int32_t rows_per_pass, passes, groups, total_wg;  // set by the launcher
};
hipError_t launch_merge_up_v(MergeUpArgs a, int cus, hipStream_t stream);

// ---- device-side precondition check (bits of the flag word, as in the public header)
constexpr int kBadCacheLenShort = 1, kBadCacheLenLong = 2, kBadIdxLen = 4, kBadIdxRange = 8, kBadIdxOrder = 16,
              kBadIdxCausal = 32;
struct CheckArgs {
  const int32_t* cache_len;  // [B]
  const int32_t* idx;        // [B][Q][K_max] or null (dense)
  const int32_t* idx_len;    // [B][Q] (with idx)
  int32_t B, Q, K_max, max_cache_len;
  int32_t* flags;            // one int32, written
};
hipError_t launch_check_inputs(const CheckArgs& a, hipStream_t stream);

// ---- streaming-read measurement
constexpr size_t kStreamChunkBytes = 32768;  // bytes one workgroup reads per turn (256 lanes x 8 x 16 B)
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t never, uint32_t* sink, hipStream_t stream);

}  // namespace mla
