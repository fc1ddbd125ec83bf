/*
 * mla_absorb.h -- C ABI of libmla_absorb.so: absorbed Multi-head Latent Attention over a
 * 512-wide bf16 latent KV cache, hand-written HIP kernels for AMD MI355X (gfx950).
 *
 * The operation (page "Module 05 -- MLA: Compressing Per-Token History", sections 1-4;
 * colibri "GLM-5.3-Flash engine", section "MLA is absorbed"):
 *   each cached token j is one latent c_j (width R = 512); head h rebuilds
 *   k_{j,h} = U_h^K c_j and v_{j,h} = U_h^V c_j (U = D x R, D = 256).  Attention never
 *   rebuilds them.  The three calls below are the three steps of the absorbed form:
 *     1. mla_absorb_q     q~_h = (U_h^K)^T q_h, once per query and head;
 *     2. mla_latent_attn  s_j = scale * q~_h . c_j over the visible positions, softmax,
 *                         and the weighted sum kept in latent space, o_lat,h = sum_j a_j c_j;
 *        mla_latent_attn_indexed: the same over an explicit list of positions per query
 *                         (the consumer of a sparse selection such as DSA k-pooling, colibri
 *                         "DSA with k-pooling");
 *     3. mla_up_v         out_h = U_h^V o_lat,h, the one expansion at the end.
 *   Composed, they equal ordinary softmax attention on the expanded keys and values
 *   (exactly: only the order of the products changes, colibri "MLA is absorbed"); the scores
 *   equal the expanded scores, with the same scale.
 *
 * Conventions shared by every call
 *   - All tensor arguments are DEVICE pointers owned by the caller (the library never
 *     allocates, frees or keeps them), row-major and contiguous unless a stride is given,
 *     16-byte aligned.  bf16 values are passed as uint16_t bit patterns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only enqueues work
 *     on it: it never synchronises, never allocates and keeps no state between calls, so
 *     calls on different streams may run concurrently.
 *   - Supported shapes: R == 512, D == 256, H a positive multiple of 16 (the checkpoint
 *     has H = 64; the attention kernels take heads in groups of 64, the last group of other
 *     counts partial).  Other shapes return MLA_ERR_SHAPE.
 *   - On any error the call returns a negative status BEFORE enqueuing anything, so no
 *     output is written.  MLA_ERR_HIP means a launch failed after validation.
 *   - The current HIP device must be a gfx950 GPU (MLA_ERR_DEVICE otherwise).
 *
 * Query positions (page "Module 08 -- Vision, MTP, and Hybrid Serving State", section 2:
 * the full model verifies the drafted tokens in one forward pass; page "Module 05",
 * section 4: a query sees only j <= t):
 *   a pass over Q new positions of sequence b appends their latents to the cache first;
 *   query i (0 <= i < Q) then sits at position t = cache_len[b] - Q + i and, in the dense
 *   call, sees every position j <= t.  Q = 1 is single-token decode; Q = 1 + k verifies k
 *   drafted tokens.  Rolling back rejected drafts is a smaller cache_len (the latent cache
 *   is truncatable by position, page "Module 08", section 3).
 */
#ifndef MLA_ABSORB_H
#define MLA_ABSORB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = -1,      /* a required pointer is NULL */
  MLA_ERR_SHAPE = -2,     /* unsupported H, D or R, or a non-positive size */
  MLA_ERR_ARG = -3,       /* another argument out of range (stride, num_splits, K_max, scale) */
  MLA_ERR_WORKSPACE = -4, /* workspace smaller than mla_latent_attn_workspace_size() */
  MLA_ERR_HIP = -5,       /* a HIP runtime call or kernel launch failed */
  MLA_ERR_DEVICE = -6,    /* the current device is not a gfx950 GPU */
  MLA_ERR_SCRATCH = -7    /* the call needs more than the fixed scratch of the no-allocation entry
                             point (MLA_NOALLOC_SCRATCH_BYTES) */
};

/* Human-readable text for a status code (static storage; never NULL). */
const char* mla_status_string(int status);

/*
 * Query absorption (page "Module 05", section 3: q~_h = (U_h^K)^T q_h, computed once per
 * query and head, independent of the cached token it is scored against).
 *   q      [rows][H][D] bf16   the queries (rows = batch * q_len)
 *   w_k    [H][D][R]    bf16   U_h^K for every head, as stored in the checkpoint (D x R per head)
 *   q_abs  [rows][H][R] bf16   output: prescale * (U_h^K)^T q_h, accumulated in fp32 and
 *                              rounded to nearest-even bf16
 *   q_abs_lo [rows][H][R] bf16 output (may be NULL): the second term of the same value, the
 *                              nearest-even bf16 of (x - q_abs) for the fp32 result x, so that
 *                              q_abs + q_abs_lo carries x to within 2^-17 |x|.  Pass it to the
 *                              attention calls when scores need more than bf16's 8 bits of the
 *                              absorbed query (latents with large outliers, as in a stress case
 *                              with 1% of positions scaled x8, where one term moves a few outputs
 *                              by about 1% of the output's largest value)
 *   prescale                   1.0f, or a power of two such as the softmax scale 1/16 (then
 *                              pass scale = 1 to the attention call); must be finite
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (rows < 1 or unsupported dims), MLA_ERR_ARG
 * (non-finite prescale), MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_absorb_q(const uint16_t* q, const uint16_t* w_k, uint16_t* q_abs, uint16_t* q_abs_lo, int32_t rows,
                 int32_t H, int32_t D, int32_t R, float prescale, void* stream);

/*
 * Number of position splits a latent-attention call will use (split-K over the positions,
 * each split a partial softmax merged by log-sum-exp).
 *   max_positions  dense: the max_cache_len bound; indexed: K_max
 *   num_splits     0 = choose automatically for the current device; otherwise the request,
 *                  clamped to [1, 1024] and to the number of 32-position tiles, then lowered
 *                  so that no split is empty once the positions are cut into equal runs of
 *                  whole tiles (e.g. 8 tiles asked for 5 splits use 4 splits of 2 tiles)
 *   indexed        0 for mla_latent_attn, 1 for mla_latent_attn_indexed.  Both are priced
 *                  the same way: rounds of one workgroup per CU times the tiles of a split,
 *                  plus the partials each extra split writes and the merge reads back.  A
 *                  workgroup takes one query per sequence and 64-head group, except in dense
 *                  calls with an even Q, where it takes two adjacent queries; the two calls
 *                  can therefore choose different counts for the same sizes
 * Returns the split count (>= 1), or a negative status for bad sizes.
 */
int32_t mla_latent_attn_num_splits(int32_t B, int32_t Q, int32_t H, int32_t max_positions,
                                   int32_t num_splits, int32_t indexed);

/*
 * Workspace bytes a latent-attention call needs (0 when it uses one split): the split
 * partials, [splits][B*Q][H][R] fp16 (each split's weighted sum of latents divided by its own
 * softmax sum) plus [splits][B*Q][H][2] fp32 (running maximum, sum).  Same
 * arguments as mla_latent_attn_num_splits plus R.  Returns 0 on bad sizes as well; the
 * attention calls reject a workspace that is too small.
 */
size_t mla_latent_attn_workspace_size(int32_t B, int32_t Q, int32_t H, int32_t R,
                                      int32_t max_positions, int32_t num_splits, int32_t indexed);

/*
 * Dense latent attention (page "Module 05", section 3: scores read the cached latent
 * directly through the absorbed query; the value sum accumulates in latent space and is
 * expanded later; the scale is that of the original q.k).
 *   q_abs      [B][Q][H][R] bf16   absorbed queries (mla_absorb_q)
 *   q_abs_lo   [B][Q][H][R] bf16   second query term (mla_absorb_q), or NULL.  Given, every
 *                                  score is c_j . q_abs + c_j . q_abs_lo, both products summed in
 *                                  one fp32 accumulator; each query then runs in a workgroup of its
 *                                  own (about 10% slower for Q = 1; dense calls with an even Q lose
 *                                  the query pairing), with the split count of the one-term call
 *   cache      bf16 latent rows: row j of sequence b starts at cache + b*cache_batch_stride
 *              + j*R; cache_batch_stride (elements) >= max_cache_len * R
 *   cache_len  [B] int32 (device)  positions held by each sequence, including the Q new ones
 *   max_cache_len                  host-side bound on every cache_len[b] (>= Q)
 *   scale                          softmax scale on q.k (1/16 for 256-wide heads); finite, > 0
 *   num_splits                     0 = auto (see mla_latent_attn_num_splits)
 *   o_lat      [B][Q][H][R] fp32   output: sum_j a_j c_j, a = softmax_j(scale * q~ . c_j)
 *   lse        [B][Q][H] fp32      output (may be NULL): ln sum_j exp(scale * q~ . c_j)
 *   workspace, workspace_bytes     caller-owned device scratch of at least
 *                                  mla_latent_attn_workspace_size() bytes (may be NULL if 0)
 * Device-side preconditions (not checked on the host): Q <= cache_len[b] <= max_cache_len.
 * Cache rows at or past min(cache_len[b], max_cache_len) are never read.  A query whose
 * visible set is empty (cache_len[b] < Q) gets o_lat = NaN and lse = -inf.
 * Results are deterministic for a fixed num_splits (no atomics in any reduction), and for the
 * same split count and query terms equal bit for bit those of mla_latent_attn_indexed given
 * every causal position.  With several splits each split's normalised partial is kept in fp16 between the
 * two kernels (2^-11 relative; a convex combination of cached latents, so the cache's values
 * must stay below 65,504 in magnitude); maxima, sums and lse stay fp32.
 */
int mla_latent_attn(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache,
                    int64_t cache_batch_stride, const int32_t* cache_len, int32_t B, int32_t Q, int32_t H,
                    int32_t R, int32_t max_cache_len, float scale, int32_t num_splits, float* o_lat,
                    float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Indexed latent attention: as mla_latent_attn, but query i of sequence b attends exactly
 * to the positions idx[b][i][0 .. idx_len[b][i]-1] (the rows a sparse selector such as DSA
 * k-pooling picked, plus the causal tail of the pass; colibri "DSA with k-pooling").
 *   idx      [B][Q][K_max] int32 (device)  positions, sorted ascending, unique, causal
 *   idx_len  [B][Q] int32 (device)         entries used per query, 1 <= idx_len <= K_max
 *   K_max                                  slots per query in idx (>= 1)
 * Index slots at or past idx_len are never read.  A position outside
 * [0, min(cache_len[b], max_cache_len)) is skipped without being read (memory safety; the
 * result for such input is not the attention over the listed positions).  A query with no
 * usable position gets o_lat = NaN and lse = -inf.  Workspace: pass K_max as max_positions
 * to mla_latent_attn_workspace_size.
 */
int mla_latent_attn_indexed(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache,
                            int64_t cache_batch_stride, const int32_t* cache_len, const int32_t* idx,
                            const int32_t* idx_len, int32_t K_max, int32_t B, int32_t Q, int32_t H,
                            int32_t R, int32_t max_cache_len, float scale, int32_t num_splits,
                            float* o_lat, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * k-pooled sparse-attention indexer: the three steps that turn indexer keys into the position
 * lists mla_latent_attn_indexed consumes (colibri "GLM-5.3-Flash engine", "Architecture notes",
 * "DSA with k-pooling": keys are grouped into pools, a pool's key is a per-channel softmax
 * mixture of its members, only complete and causally visible pools are selectable, the
 * incomplete tail is appended, ties go to the lower index; page "Module 08", section 3: after a
 * rollback the selection is rebuilt under the same pool-completion rule, which a smaller
 * cache_len gives).  Pool p holds positions p*pool .. p*pool + pool - 1 of its sequence.
 *
 * mla_kpool_keys: pooled[b][p][c] = sum_s w[s][c] * k[b][p*pool + s][c] with
 * w[.][c] = softmax over s of g[b][p*pool + s][c] (fp32), for every complete pool
 * p < min(cache_len[b], max_cache_len) / pool at or after pool_begin[b].
 *   k, g         bf16 rows of d values; row j of sequence b at (k|g) + b*batch_stride + j*d;
 *                batch_stride (elements) >= max_cache_len * d and a multiple of 8 (rows are read as
 *                16-byte vectors); rows past cache_len are never read
 *   cache_len    [B] int32 (device)
 *   pool_begin   [B] int32 (device) first pool to build (pools before it are left as they are,
 *                so an append after new positions only builds the pools they complete), or
 *                NULL for 0
 *   d            64, 128 or 256;  pool >= 1;  max_pools >= max_cache_len / pool
 *   pooled       [B][max_pools][d] fp32 output (caller-owned)
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ARG, MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_kpool_keys(const uint16_t* k, const uint16_t* g, int64_t batch_stride, const int32_t* cache_len,
                   const int32_t* pool_begin, int32_t B, int32_t max_cache_len, int32_t d, int32_t pool,
                   float* pooled, int32_t max_pools, void* stream);

/*
 * mla_indexer_scores: scores[b][i][p] = q[b][i] . pooled[b][p] (fp32, the channels summed in
 * one fixed order), for every complete pool of sequence b.
 *   q        [B][Q][d] bf16 indexer queries; 1 <= Q <= 8
 *   pooled   [B][max_pools][d] fp32 from mla_kpool_keys
 *   scores   [B][Q][max_pools] fp32 output; entries of incomplete pools are not written
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (Q or d out of range), MLA_ERR_ARG, MLA_ERR_DEVICE,
 * MLA_ERR_HIP.
 */
int mla_indexer_scores(const uint16_t* q, const float* pooled, const int32_t* cache_len, int32_t B, int32_t Q,
                       int32_t d, int32_t pool, int32_t max_pools, int32_t max_cache_len, float* scores,
                       void* stream);

/*
 * mla_indexer_select: for query i of sequence b, at position t = cache_len[b] - Q + i, the
 * topk / pool highest-scoring pools whose last position is <= t (ties: the lower pool first;
 * all of them when there are fewer), in ascending order and expanded to their positions, then
 * (tail != 0) the positions floor((t+1)/pool)*pool .. t of the incomplete pool.
 *   scores   [B][Q][max_pools] fp32 (mla_indexer_scores); max_pools <= 16384
 *   topk     positions selected before the tail: a positive multiple of pool
 *   idx      [B][Q][K_max] int32 output, ascending positions, unused slots -1;
 *            K_max >= topk + pool - 1 with the tail (topk without)
 *   idx_len  [B][Q] int32 output: entries used
 * The selection is exact integer work on the fp32 scores and deterministic.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ARG, MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_indexer_select(const float* scores, const int32_t* cache_len, int32_t B, int32_t Q, int32_t pool,
                       int32_t max_pools, int32_t max_cache_len, int32_t topk, int32_t tail, int32_t* idx,
                       int32_t* idx_len, int32_t K_max, void* stream);

/*
 * Latent down-projection with cache append (page "Module 05", section 1: every token is
 * projected down to one shared latent c_t, and c_t is what the cache keeps; page "Module 08",
 * section 1: hidden width 4096; section 3: the latent cache is truncatable by position).
 *   h          [B][Q][hidden] bf16  hidden states of the pass's Q new tokens per sequence
 *   w_dkv      [R][hidden]    bf16  the projection; row r holds the weights of latent channel r
 *   cache      latent cache (as in mla_latent_attn); row j of sequence b at
 *              cache + b*cache_batch_stride + j*R; cache_batch_stride >= max_cache_len * R
 *   cache_len  [B] int32 (device): lengths AFTER the pass.  Token i of sequence b is written at
 *              position cache_len[b] - Q + i, where its query sits in the attention call, as
 *              bf16(sum_k w_dkv[r][k] h[b][i][k]) (fp32 accumulation, nearest-even rounding).
 *              Nothing else is written.  Device-side precondition: Q <= cache_len[b] <=
 *              max_cache_len (positions that would fall outside the cache are skipped).
 * Each row depends only on its own hidden state and w_dkv (a fixed summation order), so a token
 * projected in a verification pass and the same token projected alone give identical bits.
 * Rolling back rejected tokens is a smaller cache_len; their stale rows are never read.
 * Supported: hidden == 4096, R == 512.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ARG (stride or max_cache_len < Q),
 * MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_latent_append(const uint16_t* h, const uint16_t* w_dkv, uint16_t* cache, int64_t cache_batch_stride,
                      const int32_t* cache_len, int32_t B, int32_t Q, int32_t hidden, int32_t R,
                      int32_t max_cache_len, void* stream);

/*
 * The naive (expanded) form, for comparison with the absorbed one (page "Module 05", section 5:
 * prefill and decode may prefer different algebra; the naive form expands k_{j,h} and v_{j,h}
 * for every cached token and runs ordinary multi-head attention).  The two calls below compute
 * the same attention as mla_absorb_q + mla_latent_attn + mla_up_v, up to rounding: keys and values
 * are rounded to bf16 after expansion.
 *
 * mla_expand_kv: k_{j,h} = U_h^K c_j and v_{j,h} = U_h^V c_j for every position j < cache_len[b]
 * (fp32 accumulation, nearest-even bf16 out).
 *   cache, cache_batch_stride, cache_len, max_cache_len   as in mla_latent_attn
 *   w_k, w_v  [H][D][R] bf16, as in mla_absorb_q / mla_up_v
 *   k_out     [B][max_cache_len][H][D] bf16 output, position-major (rows past cache_len untouched)
 *   vt_out    [B][H][D][vt_len] bf16 output: values transposed, each (head, dim) row running over
 *             positions; vt_len >= max_cache_len and a multiple of 64.  Positions from cache_len[b]
 *             to the next multiple of 64 are written as zeros (mla_naive_attn reads whole
 *             64-position spans); later ones are untouched.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ARG (stride or vt_len), MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_expand_kv(const uint16_t* cache, int64_t cache_batch_stride, const int32_t* cache_len, const uint16_t* w_k,
                  const uint16_t* w_v, int32_t B, int32_t H, int32_t D, int32_t R, int32_t max_cache_len,
                  uint16_t* k_out, uint16_t* vt_out, int32_t vt_len, void* stream);

/*
 * mla_naive_attn: causal multi-head attention on the expanded keys and values of mla_expand_kv:
 * query i of sequence b (position t = cache_len[b] - Q + i) and head h sees k_{j,h}, v_{j,h} for
 * j <= t; s_j = scale * q . k_j, out = sum_j softmax(s)_j v_j (fp32), lse = ln sum_j exp(s_j).
 *   q      [B][Q][H][D] bf16 queries (not absorbed)
 *   k, vt  the outputs of mla_expand_kv for the same cache_len, max_cache_len and vt_len
 *   out    [B][Q][H][D] fp32;  lse  [B][Q][H] fp32 or NULL
 * Device-side precondition: Q <= cache_len[b] <= max_cache_len.
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_ARG (scale, vt_len, max_cache_len < Q),
 * MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_naive_attn(const uint16_t* q, const uint16_t* k, const uint16_t* vt, int32_t vt_len, const int32_t* cache_len,
                   int32_t B, int32_t Q, int32_t H, int32_t D, int32_t max_cache_len, float scale, float* out,
                   float* lse, void* stream);

/*
 * Value up-projection (page "Module 05", section 3: U_h^V factors out of the sum over
 * history, so the accumulated latent is expanded once, at the end).
 *   o_lat  [rows][H][R] fp32   accumulated latents (mla_latent_attn)
 *   w_v    [H][D][R]    bf16   U_h^V for every head, as stored in the checkpoint
 *   out    [rows][H][D] fp32   output: U_h^V o_lat,h (o_lat is split into two bf16 terms
 *                              before the bf16 matrix multiply, so it keeps ~16 mantissa bits)
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_up_v(const float* o_lat, const uint16_t* w_v, float* out, int32_t rows, int32_t H, int32_t D,
             int32_t R, void* stream);

/*
 * Latent attention and the value up-projection in one call (page "Module 05", section 3: the
 * value sum accumulates in latent space and U_h^V is applied once per query and head).  The
 * attention is mla_latent_attn, or mla_latent_attn_indexed when idx is given; the merge of its
 * split partials is fused into the up-projection, so the accumulated latents never travel
 * through device memory as a separate array.  The result has the same bits as mla_up_v applied
 * to the o_lat of the separate attention call with the same split count (same merge arithmetic in
 * the same order, same up-projection).
 *   q_abs, q_abs_lo, cache, cache_batch_stride, cache_len, B, Q, H, R, max_cache_len, scale,
 *   num_splits         as in mla_latent_attn
 *   idx, idx_len, K_max  as in mla_latent_attn_indexed, or idx = idx_len = NULL (K_max ignored)
 *                      for dense attention
 *   w_v    [H][D][R] bf16   U_h^V (D == 256)
 *   out    [B][Q][H][D] fp32 output
 *   lse    [B][Q][H] fp32   output (may be NULL)
 *   workspace, workspace_bytes  caller-owned device scratch of at least
 *                      mla_latent_attn_up_v_workspace_size() bytes (never 0: with one split it
 *                      holds the accumulated latents)
 * Errors: MLA_ERR_NULL (a required pointer, or only one of idx / idx_len), MLA_ERR_SHAPE,
 * MLA_ERR_ARG, MLA_ERR_WORKSPACE, MLA_ERR_DEVICE, MLA_ERR_HIP.  Device-side preconditions and
 * empty-query behaviour as in the attention calls (out = NaN for a query that sees nothing).
 */
size_t mla_latent_attn_up_v_workspace_size(int32_t B, int32_t Q, int32_t H, int32_t R,
                                           int32_t max_positions, int32_t num_splits, int32_t indexed);
int mla_latent_attn_up_v(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache,
                         int64_t cache_batch_stride, const int32_t* cache_len, const int32_t* idx,
                         const int32_t* idx_len, int32_t K_max, int32_t B, int32_t Q, int32_t H, int32_t R,
                         int32_t max_cache_len, float scale, int32_t num_splits, const uint16_t* w_v,
                         int32_t D, float* out, float* lse, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Debug check of the attention calls' device-side preconditions (the calls themselves do not
 * check device data: on bad data they stay within the cache and index rows but their result
 * is not the attention asked for).  Page "Module 05", section 4 (query t sees j <= t); page
 * "Module 08", section 2 (the Q new positions are the cache's last Q); colibri "DSA with
 * k-pooling" (a query's positions are a sorted selection of its prefix).
 *   cache_len  [B] int32 (device)
 *   idx, idx_len  as in mla_latent_attn_indexed, or both NULL to check a dense call
 *   B, Q, K_max, max_cache_len  as in the attention call (K_max ignored when idx is NULL)
 *   flags      one int32 (device), output: 0 when every precondition holds, else the OR of
 *              the MLA_BAD_* bits below.  Read it after the stream has reached this call.
 * Enqueues one single-workgroup kernel; allocates nothing, clears nothing beforehand (the
 * flag word is written whole), never synchronises.  Meant for debugging: it reads every listed
 * index slot.  Errors: MLA_ERR_NULL (cache_len, flags, or only one of idx / idx_len),
 * MLA_ERR_SHAPE (B, Q or max_cache_len < 1), MLA_ERR_ARG (K_max < 1 with idx),
 * MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
enum mla_bad_input {
  MLA_BAD_CACHE_LEN_SHORT = 1,  /* cache_len[b] < Q */
  MLA_BAD_CACHE_LEN_LONG = 2,   /* cache_len[b] > max_cache_len */
  MLA_BAD_IDX_LEN = 4,          /* idx_len[b][i] outside [1, K_max] */
  MLA_BAD_IDX_RANGE = 8,        /* a listed position outside [0, min(cache_len[b], max_cache_len)) */
  MLA_BAD_IDX_ORDER = 16,       /* listed positions not strictly ascending */
  MLA_BAD_IDX_CAUSAL = 32       /* a listed position past the query's own, cache_len[b] - Q + i */
};
int mla_check_attn_inputs(const int32_t* cache_len, const int32_t* idx, const int32_t* idx_len, int32_t B,
                          int32_t Q, int32_t K_max, int32_t max_cache_len, int32_t* flags, void* stream);

/*
 * Measurement helper, not a step of the attention path: reads `bytes` of device memory at src
 * once, in 32 KiB chunks spread over the GPU, as a plain streaming read.  Its rate is the
 * device's achievable streaming-read bandwidth, the ceiling beside the published peak against
 * which the attention kernels' cache streams are measured (page "Module 05", section 5: decode is
 * bandwidth-bound, and a workload's regime is measured rather than counted).
 *   src    device memory, 16-byte aligned, bytes readable
 *   bytes  a positive multiple of 32768
 *   never  a value the folded bytes (XOR of every 32-bit word each lane reads) will not equal
 *   sink   one uint32 (device): OR-ed with 1 only if some lane's folded value equals never, so
 *          that the loads cannot be dropped; practically never written
 * Errors: MLA_ERR_NULL, MLA_ERR_SHAPE (bytes), MLA_ERR_DEVICE, MLA_ERR_HIP.
 */
int mla_stream_read(const void* src, size_t bytes, uint32_t never, uint32_t* sink, void* stream);

/*
 * mla_latent_attn_up_v for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments, kernels,
 * split count and bits as mla_latent_attn_up_v, minus the workspace: the split partials live
 * in a scratch buffer of MLA_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * per GPU, until the process ends.  The call allocates nothing (no hipMalloc, no allocating
 * library routine); the caller passes every input and output.
 *   - The first call on a device resolves that device's buffer address (with that device
 *     current); make it outside graph capture.
 *   - A call whose workspace would exceed the buffer (mla_latent_attn_up_v_workspace_size() >
 *     MLA_NOALLOC_SCRATCH_BYTES) is refused with MLA_ERR_SCRATCH before anything is enqueued.
 *     The four full-size workloads of this library need at most about 63 MB.
 *   - Every call on one GPU shares that GPU's buffer and leaves the last call's partials in it
 *     (nothing in it needs clearing: each call writes every partial it reads).  Calls that
 *     overlap on one GPU, on different streams or from different threads, RACE and give wrong
 *     results: serialise them (one stream, or events between streams).
 * Errors: those of mla_latent_attn_up_v except MLA_ERR_WORKSPACE, plus MLA_ERR_SCRATCH.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int mla_latent_attn_up_v_noalloc(const uint16_t* q_abs, const uint16_t* q_abs_lo, const uint16_t* cache,
                                 int64_t cache_batch_stride, const int32_t* cache_len, const int32_t* idx,
                                 const int32_t* idx_len, int32_t K_max, int32_t B, int32_t Q, int32_t H,
                                 int32_t R, int32_t max_cache_len, float scale, int32_t num_splits,
                                 const uint16_t* w_v, int32_t D, float* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ABSORB_H */
