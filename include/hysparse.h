/*
 * hysparse.h -- C ABI of libhysparse: the HySparse2 Cross-Decoder hybrid-block
 * attention path (one full-attention layer that selects tokens, sparse layers
 * that reuse its cache and selection, and the KV Bridging projection that
 * fills the cache), for AMD Instinct MI355X (gfx950).
 *
 * Sources (web write-ups of the HySparse2 announcement, cited by site, page
 * title and section):
 *   ithome  -- IT之家 "小米公开 MiMo-V3 核心架构 HySparse2：面向长程多轮 Agent
 *              优化推理效率": KV-sharing overview (KV Bridging), section
 *              "KV Reuse：在同一 Hybrid Block 内，复用 KV 与选择结果", and the
 *              recent-window paragraphs after it.
 *   cnyes   -- 量子位 repost "MiMo-V2.6剛發佈，羅福莉就開始劇透MiMo-V3了", sections
 *              "預填充只走前半程" and "檢索精確到token".
 *   toolnavs-- "Xiaomi stellt HySparse2 vor", section "HySparse2 がやったこと".
 *   ai-bio  -- "小米 MiMo-V3 – 小米 MiMo 团队公布的下一代长上下文基础模型",
 *              sections "两级 KV 共享：KV 桥接与 KV 重用" and
 *              "token 级稀疏与近期 Token 强制窗口".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is DEVICE memory owned by the caller, row-major,
 *   unless the comment says "host".  The library never allocates, frees or
 *   keeps a pointer past the call; its scratch memory is the caller's
 *   workspace, sized by the *_workspace_size queries.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   work is enqueued on it; nothing is synchronised: the caller syncs.
 * - Validation is complete and synchronous, before anything is enqueued: on
 *   any error nothing is launched and no output or workspace byte is written.
 *   A launch failure returns HS_ERR_HIP; the text of the last error of the
 *   calling thread is available from hs_last_error().  Faults inside a kernel
 *   surface at the caller's next synchronisation, as HIP reports them.
 * - No C++ exception crosses this interface.  Calls are reentrant on
 *   different streams with disjoint workspaces and outputs.
 * - head_dim must be 128.  num_kv_heads must divide num_q_heads (MQA: 1).
 */
#ifndef HYSPARSE_H
#define HYSPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HS_ABI_VERSION 3

typedef enum {
  HS_OK = 0,
  HS_ERR_INVALID_ARGUMENT = 1,
  HS_ERR_UNSUPPORTED = 2,
  HS_ERR_WORKSPACE_TOO_SMALL = 3,
  HS_ERR_HIP = 4
} hs_status;

/* Element types.  HS_FP8_E4M3 is OCP E4M3FN (bias 7, max 448, no infinity,
 * S.1111.111 = NaN) with one float32 scale per cached row: value = decode(code)
 * * scale.  The pages say only that the cache is FP8 (ithome page, cost
 * analysis); the format and the per-token scale are this library's reading. */
typedef enum { HS_F32 = 0, HS_BF16 = 1, HS_FP8_E4M3 = 2 } hs_dtype;

/* One shared KV cache: the cache of one hybrid block's full-attention layer
 * (ithome page, "KV Reuse" section: the sparse layers of the block read this
 * same cache), or one KV Bridging target.
 *   k, v        device [capacity_rows, num_kv_heads, head_dim] of dtype
 *   k_scale,
 *   v_scale     device float [capacity_rows, num_kv_heads]; required for
 *               HS_FP8_E4M3, must be NULL otherwise
 *   batch       number of sequences B (rows of sequence b are
 *               [row_start[b], row_start[b] + seq_len[b]))
 *   d_row_start device int64 [batch]; h_row_start the same values on the host
 *   d_seq_len   device int32 [batch] L_b >= 1; h_seq_len the same on the host
 *               (host copies are used to validate bounds and plan launches)
 * The L_b rows of a sequence are the cache after the current step's tokens
 * were appended: the recent window is its last rows. */
typedef struct {
  hs_dtype dtype;
  int32_t head_dim;
  int32_t num_kv_heads;
  int32_t batch;
  int64_t capacity_rows;
  void *k;
  void *v;
  float *k_scale;
  float *v_scale;
  const int64_t *d_row_start;
  const int64_t *h_row_start;
  const int32_t *d_seq_len;
  const int32_t *h_seq_len;
} hs_kv_cache;

/* Attention / selection parameters.
 *   num_q_heads   H (query heads; heads h*G..h*G+G-1 share KV head h, G = H/n_kv)
 *   q_tokens      n_q query tokens per sequence in this step (no mask among them:
 *                 every query token attends to all L_b rows)
 *   top_k         global budget k (1024 in the pages), taken from outside the window
 *   window        recent window W (128 in the pages), always selected
 *   softmax_scale 0 => 1/sqrt(head_dim)
 *   select_block  0 (or 1): token-level selection, the HySparse2 mechanism;
 *                 64: the previous generation's block-level selection (dpshk
 *                 page, section 03: history chosen in 64-token blocks), kept
 *                 as a comparison variant.  Block b covers candidates
 *                 [64b, min(64b + 64, L - W')); its score is the float32 sum of
 *                 its tokens' scores added as a pairwise tree in index order;
 *                 when k' < L - W' the list takes floor(k'/64) whole blocks
 *                 (score descending, ties to the lower block), else every
 *                 candidate; global tokens ascending, then the window, then -1.
 *                 Other values: HS_ERR_UNSUPPORTED.  Only hs_full_attn_select
 *                 reads it.
 * ithome page, recent-window paragraph: the 128 most recent tokens are forced
 * into the selection and 1,024 global tokens come from outside that window. */
typedef struct {
  int32_t num_q_heads;
  int32_t q_tokens;
  int32_t top_k;
  int32_t window;
  float softmax_scale;
  int32_t select_block;
} hs_attn_params;

/* Workspace bytes hs_full_attn_select needs for these shapes: the largest over
 * the query types that are supported for them (0 when none is, or on invalid
 * arguments).  Uses the host lengths only.  The size queries do not change the
 * calling thread's last error. */
size_t hs_full_attn_select_workspace_size(const hs_kv_cache *kv, const hs_attn_params *p);

/* Workspace bytes hs_sparse_attn needs for these shapes (0 on invalid arguments). */
size_t hs_sparse_attn_workspace_size(const hs_kv_cache *kv, const hs_attn_params *p);

/* Workspace bytes hs_select_from_scores needs (0 on invalid arguments). */
size_t hs_select_workspace_size(int32_t batch, int32_t q_tokens, int32_t n_kv, int32_t max_len,
                                int32_t top_k, int32_t window);

/* KV Bridging (ithome page, KV-sharing overview; toolnavs page "HySparse2 が
 * やったこと"; ai-bio page "两级 KV 共享"): every target full-attention layer l
 * projects its own K and V from one source hidden state,
 *     K_l = X W_k[l],  V_l = X W_v[l]   (no bias, no norm, no rotary),
 * and stores them at rows [row_offset, row_offset + n_tokens) of its cache.
 *   hidden      device bf16 [n_tokens, d_model]
 *   w_k, w_v    HOST arrays of n_targets device pointers, each bf16
 *               [d_model, head_dim] row-major
 *   targets     HOST array of n_targets caches (dtype HS_BF16 or HS_FP8_E4M3,
 *               num_kv_heads 1, head_dim 128); only k, v, k_scale, v_scale,
 *               capacity_rows and dtype are used
 * bf16 targets store round-to-nearest-even of the float32 accumulator.  FP8
 * targets store, per row r (one token; K and V separately): a = max|r_i|,
 * scale = a / 448 (correctly rounded float32; 1 when that is 0),
 * code_i = e4m3_rne(r_i / scale) saturating at 448.
 * Rows outside [row_offset, row_offset + n_tokens) are not written.
 * Errors: HS_ERR_INVALID_ARGUMENT for null pointers, d_model not a positive
 * multiple of 64, row_offset < 0, row_offset + n_tokens > capacity_rows, a
 * dtype other than bf16/fp8, or scale pointers that do not match the dtype. */
hs_status hs_kv_bridge(const void *hidden, int64_t n_tokens, int32_t d_model, int32_t n_targets,
                       const void *const *w_k, const void *const *w_v,
                       const hs_kv_cache *const *targets, int64_t row_offset, void *stream);

/* Decode-time KV append through the bridge (ithome page, KV-sharing overview,
 * and the prefill early-exit paragraphs: once generation starts the Cross-
 * Decoder runs normally, so each new token's K/V for every target full layer
 * is projected from the matching Self-Decoder hidden state).  Computes exactly
 * what hs_kv_bridge computes for these n_tokens rows (same rounding and FP8
 * scaling), but token t is stored at cache row rows[t] of every target instead
 * of a contiguous range: for a decode step, rows[b] = row_start[b] + L_b of
 * sequence b (the caller then advances its lengths).
 *   hidden      device bf16 [n_tokens, d_model]
 *   w_k, w_v, targets   as for hs_kv_bridge
 *   d_rows      device int64 [n_tokens]: destination row of each token
 *   h_rows      host int64 [n_tokens]: the same rows, used only to validate
 *   workspace   device scratch of hs_kv_append_workspace_size() bytes (may be
 *               NULL when that is 0); the library keeps nothing in it
 * Up to 128 tokens the product is split over d_model (the weights dominate the
 * bytes) and summed in a fixed order, so values may differ from hs_kv_bridge's
 * in the last float32 bit before rounding; more tokens use the bridge kernel.
 * Errors: HS_ERR_INVALID_ARGUMENT as for hs_kv_bridge, and for a row outside
 * [0, capacity_rows) of any target or a row named twice (the writes would
 * race); HS_ERR_WORKSPACE_TOO_SMALL. */
size_t hs_kv_append_workspace_size(int64_t n_tokens, int32_t d_model, int32_t n_targets);
hs_status hs_kv_append(const void *hidden, int64_t n_tokens, int32_t d_model, int32_t n_targets,
                       const void *const *w_k, const void *const *w_v,
                       const hs_kv_cache *const *targets, const int64_t *d_rows, const int64_t *h_rows,
                       void *workspace, size_t workspace_bytes, void *stream);

/* Full-attention layer of a hybrid block, with token-level selection
 * (ithome page, "KV Reuse" section and recent-window paragraph; cnyes page
 * "檢索精確到token"; dpshk page section 03).  For every sequence b, query token t
 * and head h (KV head g = h / G):
 *     l_j = scale * <q[b,t,h], k[b,j,g]>  for all j < L_b (no mask),
 *     out[b,t,h] = sum_j softmax(l)_j v[b,j,g],  lse[b,t,h] = log sum_j exp(l_j).
 * Selection, per (b, t, g):
 *     s_j = sum over the G heads h of group g of exp(l_j(h) - lse(h)),
 *           for the global candidates j < L_b - W', W' = min(window, L_b);
 *     global set = the k' = max(0, min(top_k, L_b - window)) candidates with
 *           the largest s_j (float32 value order, ties to the lower j);
 *     sel_idx[b,t,g,:] = global set ascending, then L_b-W' .. L_b-1, then -1 padding;
 *     sel_count[b,t,g] = k' + W'.
 *   q         device [B, q_tokens, num_q_heads, head_dim], q_dtype HS_F32 or HS_BF16
 *   out       device float [B, q_tokens, num_q_heads, head_dim]
 *   lse       device float [B, q_tokens, num_q_heads] (natural log), or NULL
 *   sel_idx   device int32 [B, q_tokens, num_kv_heads, window + top_k]
 *   sel_count device int32 [B, q_tokens, num_kv_heads]
 *   scores_out device float [B, q_tokens, num_kv_heads, S] or NULL, with
 *             S = max_b (L_b - min(window, L_b)); when given, the float32 s_j
 *             used for selection are left there (entries past a list's own
 *             candidate count are unspecified)
 * Cache dtypes: HS_F32, HS_BF16, HS_FP8_E4M3.  Heads per KV head G = H / n_kv:
 * 8, 16, 32, 64, 128 or 256 (at most 128 with F32 queries or an F32 cache).
 * Alignment: q and out 16 bytes; lse, sel_idx, sel_count and scores_out 4 bytes.
 * Errors: HS_ERR_INVALID_ARGUMENT (null pointer, misaligned pointer, bad shape,
 * L_b < 1, rows outside capacity, scale pointers not matching the dtype,
 * top_k/window < 0), HS_ERR_WORKSPACE_TOO_SMALL, HS_ERR_UNSUPPORTED (head_dim !=
 * 128, another G, more than 65535 lists B * q_tokens * num_kv_heads).
 * Opt-in, E4M3 caches with more than 32 query rows per KV head: with the environment
 * variable HS_MANY_ROW_FP8_QK=1 (read at each call) the products q.k of out and lse use q
 * rounded to E4M3 per query row (scale = that row's amax / 448) on FP8 matrix units; the
 * selection scores still use the bf16 q, but with that lse.  This changes the results and
 * is off by default. */
hs_status hs_full_attn_select(const hs_kv_cache *kv, const hs_attn_params *p, const void *q,
                              hs_dtype q_dtype, float *out, float *lse, int32_t *sel_idx,
                              int32_t *sel_count, float *scores_out, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Sparse-attention layer of a hybrid block (ithome page, "KV Reuse" section:
 * it reads the full layer's cache and selection indices; recent-window
 * paragraphs: local and global rows are read in one pass, with no separate
 * sliding-window branch).  For every (b, t, h), with S = the sel_count[b,t,g]
 * first entries of sel_idx[b,t,g,:]:
 *     out[b,t,h] = sum_{j in S} softmax_S(l)_j v[b,j,g],  l_j = scale * <q, k_j>.
 *   q, out, sel_idx, sel_count: layouts as in hs_full_attn_select; every
 *   listed index must be in [0, L_b) (checked on the device: an index out of
 *   range is treated as absent).  A list with no row left (count <= 0, or every
 *   listed index absent) gets out = 0.  Any G.  Alignment: q and out 16 bytes,
 *   sel_idx and sel_count 4 bytes.  Errors as hs_full_attn_select. */
hs_status hs_sparse_attn(const hs_kv_cache *kv, const hs_attn_params *p, const void *q,
                         hs_dtype q_dtype, const int32_t *sel_idx, const int32_t *sel_count,
                         float *out, void *workspace, size_t workspace_bytes, void *stream);

/* hs_sparse_attn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (minus the workspace), same
 * launches and the same results as hs_sparse_attn.  Its scratch (the per-chunk
 * partials of the sparse layer) is a static device array of
 * HS_NOALLOC_SCRATCH_BYTES (8 MiB) that every GPU the library runs on holds
 * until the process ends; the call allocates nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (on different
 * streams, or from different host threads) race on it and must not be issued.
 * Nothing in it needs clearing between calls.  `stream` (NULL: the null stream)
 * must belong to the calling thread's current device.  Errors: as
 * hs_sparse_attn (no workspace errors), HS_ERR_INVALID_ARGUMENT for a stream of
 * another device, and HS_ERR_UNSUPPORTED when the shapes need more scratch than
 * the array holds (hs_sparse_attn_workspace_size() bounds what they need; lists
 * that fit one workgroup each need none). */
#define HS_NOALLOC_SCRATCH_BYTES (8u << 20)
hs_status hs_sparse_attn_noalloc(const hs_kv_cache *kv, const hs_attn_params *p, const void *q,
                                 hs_dtype q_dtype, const int32_t *sel_idx, const int32_t *sel_count,
                                 float *out, void *stream);

/* Sliding-window attention of the Self-Decoder side, which feeds KV Bridging
 * (ithome page, architecture overview: the Self-Decoder mixes full and
 * sliding-window attention over the current input; the pages give no window
 * size, so w = p->window is the caller's).  The q_tokens queries of sequence b
 * are the last q_tokens rows of its cache (a prefill chunk appended before the
 * call): query t sits at position pos = L_b - q_tokens + t and, for every head h
 * of KV head g,
 *     out[b,t,h] = sum_{j in B} softmax_B(l)_j v[b,j,g],  l_j = scale * <q, k_j>,
 *     B = { max(0, pos - w + 1) .. pos }.
 *   q   device [B, q_tokens, num_q_heads, head_dim], q_dtype HS_BF16
 *   out device float [B, q_tokens, num_q_heads, head_dim]
 * p->top_k and p->select_block are ignored.  No workspace.  Cache dtypes:
 * HS_BF16, HS_FP8_E4M3.  Errors: HS_ERR_INVALID_ARGUMENT (null pointer, bad
 * shape, window < 1, q_tokens > L_b for some b, L_b < 1, rows outside
 * capacity, scale pointers not matching the dtype), HS_ERR_UNSUPPORTED
 * (head_dim != 128, an F32 cache, F32 queries, batch * num_kv_heads > 65535).
 * Launch failures: HS_ERR_HIP. */
hs_status hs_swa_attn(const hs_kv_cache *kv, const hs_attn_params *p, const void *q,
                      hs_dtype q_dtype, float *out, void *stream);

/* hs_swa_attn with the output type chosen by the caller: out_dtype HS_F32 (the
 * same call as hs_swa_attn) or HS_BF16, where out holds each float32 result
 * rounded to bf16 (nearest, ties to even), half the output bytes.  out must be
 * 16-byte aligned either way.  Errors: as hs_swa_attn, and
 * HS_ERR_INVALID_ARGUMENT for another out_dtype. */
hs_status hs_swa_attn_out(const hs_kv_cache *kv, const hs_attn_params *p, const void *q,
                          hs_dtype q_dtype, void *out, hs_dtype out_dtype, void *stream);

/* One prefill chunk of a prompt on the Self-Decoder side, feeding the
 * Cross-Decoder (ithome page, prefill early-exit paragraphs: prefill runs only
 * the first half of the layers plus the bridging projections, which fill every
 * Cross-Decoder full layer's cache; toolnavs page "Prefill は半分で終わる").
 * Exactly hs_swa_attn_out(self_kv, swa_p, q, q_dtype, swa_out, swa_out_dtype,
 * stream) followed by
 * hs_kv_bridge(hidden, n_tokens, d_model, n_targets, w_k, w_v, targets,
 * row_offset, stream) on the same stream: the chunk's n_tokens queries attend
 * to their bands of the Self-Decoder cache (the chunk's rows appended at its
 * end before the call, so bands reach back into earlier chunks), and the
 * chunk's hidden states are projected into every target at rows
 * [row_offset, row_offset + n_tokens).  A prompt is prefilled by calling it on
 * consecutive chunks with growing self_kv lengths and row_offset advancing by
 * each chunk's size.  self_kv holds one sequence (batch 1) and
 * swa_p->q_tokens must equal n_tokens.  Every check of both steps runs before
 * either is launched; errors as the two calls. */
hs_status hs_prefill_chunk(const hs_kv_cache *self_kv, const hs_attn_params *swa_p, const void *q,
                           hs_dtype q_dtype, void *swa_out, hs_dtype swa_out_dtype,
                           const void *hidden, int64_t n_tokens, int32_t d_model, int32_t n_targets,
                           const void *const *w_k, const void *const *w_v,
                           const hs_kv_cache *const *targets, int64_t row_offset, void *stream);

/* The selection stage alone, on caller-given float32 scores (a test hook for
 * checking the selection bit for bit).  scores: device float
 * [batch, q_tokens, n_kv, max_len - min(window, max_len)] laid out as
 * scores_out above; lists with L_b = d_seq_len[b] use their first
 * L_b - min(window, L_b) entries.  Scores must be finite; the order is the
 * float order (-0 below +0), ties to the lower index.  select_block as in
 * hs_attn_params (0: tokens, 64: blocks).  Outputs as hs_full_attn_select.
 * scores, sel_idx and sel_count must be 4-byte aligned; at most 65535 lists
 * (HS_ERR_UNSUPPORTED beyond). */
hs_status hs_select_from_scores(const float *scores, const int32_t *d_seq_len,
                                const int32_t *h_seq_len, int32_t batch, int32_t q_tokens,
                                int32_t n_kv, int32_t max_len, int32_t top_k, int32_t window,
                                int32_t select_block, int32_t *sel_idx, int32_t *sel_count,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Kernel timing, a profiling aid (off by default).  While enabled, every
 * kernel the library enqueues is bracketed by a pair of HIP events recorded on
 * the same stream.  hs_timing_collect waits for the recorded events, writes up
 * to max records (kernel name, milliseconds) in launch order, returns how many
 * it wrote (-1 on a HIP error) and forgets all records.  The name pointers are
 * static strings.  The switch and the records belong to the calling thread (like
 * the last error): a thread collects only the launches it made itself. */
typedef struct {
  const char *name;
  float ms;
} hs_kernel_time;
void hs_timing_enable(int enable);
int hs_timing_collect(hs_kernel_time *out, int max);

/* Streaming read probe, a measurement aid: reads `bytes` (a multiple of 16) of
 * device memory at buf with 16-byte loads (non-temporal when non_temporal != 0,
 * the load the decode passes stream their cache with), grid workgroups of 512
 * threads, four loads in flight per thread.  Timed around the call it gives
 * the practical read ceiling (HBM for buffers larger than the 256 MB Infinity
 * Cache, the cache for repeated reads of smaller ones).  sink: 16 device bytes
 * that are never written for real data.  Errors: HS_ERR_INVALID_ARGUMENT. */
hs_status hs_read_probe(const void *buf, size_t bytes, int non_temporal, int32_t grid, void *sink,
                        void *stream);

/* Self-check of the FP8 storage conversion on the running device (for tests):
 * hs_kv_bridge (and hs_kv_append above 128 tokens, which runs the same
 * kernel) rounds to E4M3 with the hardware packed conversion; this compares it
 * with a bit-level round-to-nearest-even reference (the FP8 rule above
 * hs_kv_bridge) on every finite float32 y with |y| < 464, the range those
 * calls use.  counts: device, two 64-bit words,
 * set to (mismatches, values compared = 2 * 0x43E80000).  Errors:
 * HS_ERR_INVALID_ARGUMENT (NULL or misaligned counts). */
hs_status hs_e4m3_check(unsigned long long *counts, void *stream);

const char *hs_status_string(hs_status s);
/* Text of the calling thread's last error ("" if none). */
const char *hs_last_error(void);
int hs_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* HYSPARSE_H */
