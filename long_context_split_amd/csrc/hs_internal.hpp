// Internal argument blocks and launchers of libhysparse (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

enum KvType { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };       // cache storage type
enum ComputeType { CT_BF16 = 0, CT_F32 = 1 };              // MFMA input type

// attn_partial: one list = (b, g) in dense mode, (b, t, g) in gather mode.
struct AttnArgs {
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int64_t* row_start;
  const int32_t* seq_len;
  const void* q;
  int q_f32;
  int n_kv, H, G, n_q;
  int R;                 // query rows per list: n_q*G (dense) or G (gather)
  int n_lists;
  int chunk;             // tokens (dense) or list positions (gather) per work item
  int max_chunks;
  float scale_log2;      // softmax scale * log2(e)
  const int32_t* sel_idx;
  const int32_t* sel_count;
  int sel_cap;
  float* part_acc;       // [n_lists][max_chunks][R][128] unnormalised
  float* part_ml;        // [n_lists][max_chunks][R][2]  (max in log2 units, sum)
  int direct;            // one chunk per list: write out / lse / lse2 instead of partials
  float* out;            // [B, n_q, H, 128]
  float* lse;            // nullable, natural log
  float* lse2;           // nullable, log2 units
  int n_items;           // attn_wave dense: one-dimensional grid of (list, chunk) items (grid_item)
  int uniform_items;     //   items per list when every list has the same number, else 0
  uint32_t* zero_ptr;    // attn_wave: words cleared by the grid (nullable):
  int64_t zero_stride;   //   zero_lists runs of zero_words words, zero_stride apart
  int zero_words, zero_lists;
  int window;            // swa_attn: band width w (rows p - w + 1 .. p)
  // attn_wave dense, optional (score filter): per 32-token tile of every list, a CODE_TILE_BYTES
  // record at codes + (list * code_tiles + tile) * CODE_TILE_BYTES: 256 words [quad q][row h] whose
  // byte i is the code of token 32 tile + 4 q + i and row h, code = floor(8 (l2 - m) + 191) clamped
  // to [0, 255] with l2 the logit in log2 units and m the row's running reference in that tile, then
  // the 32 references m (float, rows 0..31)
  uint8_t* codes;
  int64_t code_tiles;    // tiles per list (ceil(max L / 32))
  uint32_t* zero2_ptr;   // attn_wave: a second run of words cleared by the grid (nullable)
  int64_t zero2_words;
  int qk_fp8;            // attn_rows on an E4M3 cache: Q K^T on FP8 MFMA (Q quantised per row)
  int out_bf16;          // swa_attn: out holds bf16 (round to nearest even) instead of float
};

constexpr int CODE_TILE_BYTES = 1152;      // 1024 bytes of codes + 32 float references
constexpr int CODE_OFFSET = 191;           // code = floor(8 x + CODE_OFFSET), x = l2 - m <= 8

struct MergeArgs {
  const float* part_acc;
  const float* part_ml;
  const int32_t* seq_len;
  const int32_t* sel_count;
  int sel_cap;
  int gather;
  int n_kv, H, G, n_q, R, n_lists, chunk, max_chunks;
  float* out;            // [B, n_q, H, 128]
  float* lse;            // nullable, natural log
  float* lse2;           // nullable, log2 units
};

struct ScoreArgs {
  const void* k;
  const float* k_scale;
  const int64_t* row_start;
  const int32_t* seq_len;
  const void* q;
  int q_f32;
  int n_kv, H, G, n_q, R, n_lists, window, chunk, max_chunks;
  float scale_log2;
  const float* lse2;     // [B, n_q, H]
  float* scores;         // [B, n_q, n_kv, s_stride]
  int64_t s_stride;
  int n_items;           // scores_wave: one-dimensional grid of (list, chunk) items (grid_item)
  int uniform_items;     //   items per list when every list has the same number, else 0
  uint32_t* hist;        // scores_wave: first-digit histograms of the selection (nullable),
  int64_t hist_stride;   //   2048 words per list, hist_stride words apart
  // scores_wave, optional: the full layer's chunk partials (as attn_wave writes them); when set,
  // the kernel derives LSE from them itself and its workgroups also merge O and write out / lse
  const float* part_acc;
  const float* part_ml;
  int dchunk, dmax_chunks;
  float* out;
  float* lse;            // nullable, natural log
  // scores_wave, candidate mode (cand_off > 0; one query token, hist set, chunk =
  // scores_cand_chunk()): list l has cand_nper(ncand_l, cand_total) workgroups, consecutive in the
  // grid (n_items = their sum; cand_uniform: every list has n_items / n_lists, found by division
  // instead of a scan), cand_region >= scores_cand_region(ncand_l, nper_l) for every list.  A
  // workgroup takes units of `chunk` tokens from its list's counter (SELECT_CLAIM_WORD) and appends
  // the (key, index) pairs of every score whose first digit is at or above the lowest digit the k'-th
  // key can still have (from the list's histogram as it fills) to its own region of the list's
  // candidate buffer (hist + cand_off words; region `slot` of cand_region pairs, its pair count
  // written at SELECT_RCOUNT_WORD + slot, the list's region count at SELECT_NREG_WORD); `scores`
  // may then be null (no dense scores)
  int64_t cand_off;
  int64_t cand_region;
  int top_k;
  int cand_uniform;
  int64_t cand_total;    // sum over the lists of their candidate counts
};

// Score filter (one query token per list, at most 32 query rows per KV head, after attn_wave wrote
// its codes): the bounds pass turns each candidate's codes into an upper and a lower bound of its
// selection score, histograms the lower bounds per list and keeps the first digit of each upper
// bound; the exact pass finds the highest digit d whose lower-bound bins hold k' tokens (so the
// k'-th score is at least the smallest value of digit d), recomputes the exact score of every
// token whose upper bound reaches that value, with the score pass's arithmetic, and appends the
// (key, index) pairs and their first-digit histogram for the candidate-mode selection.
struct FilterArgs {
  const void* k;
  const float* k_scale;
  const int64_t* row_start;
  const int32_t* seq_len;
  const void* q;
  int q_f32;
  int n_kv, H, G, R, n_lists, window, top_k;
  float scale_log2;
  const uint8_t* codes;  // as AttnArgs::codes
  int64_t code_tiles;
  uint16_t* udig;        // [lists][u_stride] first digit (float bits >> 20) of each upper bound
  int64_t u_stride;      //   a multiple of 32
  uint32_t* lhist;       // [lists][2048] first-digit histogram of the lower bounds (cleared before)
  float* lse2;           // [B, 1, H] log2 units: written by the bounds pass when it merges, else read
  // bounds pass: one-dimensional grid of (list, chunk) items, chunk a multiple of 2048 tokens
  int chunk, n_items, uniform_items;
  const float* part_acc; // nullable: fold the full layer's merge (as scores_wave does)
  const float* part_ml;
  int dchunk, dmax_chunks;
  float* out;
  float* lse;            // nullable
  // exact pass: cand_nper(ncand_l, cand_total) workgroups per list, consecutive; region `slot` of
  // cand_region pairs at sel_ws + list * sel_stride + cand_off (words)
  uint32_t* sel_ws;
  int64_t sel_stride, cand_off, cand_region, cand_total;
  int cand_uniform, n_wg2;
};
hipError_t launch_filter_bounds(const FilterArgs& a, hipStream_t st);
hipError_t launch_filter_exact(const FilterArgs& a, int kvt, hipStream_t st);
constexpr int FILTER_SPAN_ALIGN = 512;     // exact pass: token range of a workgroup, a multiple of this
constexpr int FILTER_BOUNDS_CHUNK = 2048;  // bounds pass: chunk granule

struct SelectArgs {
  const float* scores;   // [lists][s_stride]
  int64_t s_stride;
  const int32_t* seq_len;
  int n_q, n_kv, top_k, window, cap;
  int32_t* sel_idx;      // [lists][cap]
  int32_t* sel_count;    // [lists]
  uint32_t* ws;          // [lists][ws_stride] words (layout in hs_select.hip)
  int64_t ws_stride, cand_off;
  int chunk, max_chunks; // candidates per chunk workgroup, chunks per list
  int64_t cand_region;   // candidate mode: region stride (pairs); the region count per list is at SELECT_NREG_WORD
};

struct SelectPlan {
  int chunk, max_chunks;
  int64_t ws_stride, cand_off;   // words
};
// cand_pairs: candidate-mode capacity (pairs per list) when it exceeds s_stride
void select_plan(int64_t s_stride, SelectPlan& p, int64_t cand_pairs = 0);

struct BridgeArgs {
  const uint16_t* x;     // [T, D] bf16
  int64_t T;
  int Dm;
  int n_targets;
  const uint16_t* w[16]; // per output head block of 128 columns: (target, K|V)
  void* out[16];         // per block: cache k or v base pointer
  float* scale[16];      // per block: FP8 scale base pointer or null
  int fp8;
  int64_t row_offset;
  const int64_t* rows;   // nullable: cache row of each token (decode-time append); else row_offset + t
};

// Decode-time append (few tokens): split-K partials in a caller workspace, then a finish kernel.
struct AppendArgs {
  const uint16_t* x;     // [T, Dm] bf16
  int64_t T;
  int Dm;
  int n_blocks;          // 2 * n_targets head blocks (target, K|V) of 128 columns
  int n_slices, m_tiles;
  const uint16_t* w[16];
  void* out[16];
  float* scale[16];
  int fp8;
  const int64_t* rows;   // cache row of each token
  float* part;           // workspace: [n_slices][n_blocks][m_tiles][32][128] float32
};
void append_plan(int64_t n_tokens, int d_model, int n_targets, AppendArgs& a);
size_t append_workspace_bytes(const AppendArgs& a);
hipError_t launch_append(const AppendArgs& a, hipStream_t st);
constexpr int64_t APPEND_MAX_TOKENS = 128;   // above this hs_kv_append uses the bridge kernel

int rows_per_wave_group(int R);
int partial_tile_tokens(int nwr);

// nwr: query-row wave groups per workgroup, as planned by the host (1, 2, 4, 8; fp32 compute: 1 or 4)
hipError_t launch_attn_partial(const AttnArgs& a, int kvt, int ct, int nwr, bool gather, hipStream_t st);
// attn_wave: R <= 32 query rows per list, bf16 or FP8 caches, 8 independent waves per workgroup
hipError_t launch_attn_wave(const AttnArgs& a, int kvt, hipStream_t st);
// sparse layer, bf16 Q with a bf16 or FP8 cache, any G (blocks of 32 heads); chunk a multiple of 32
hipError_t launch_attn_gather(const AttnArgs& a, int kvt, hipStream_t st);
hipError_t launch_swa_attn(const AttnArgs& a, int kvt, hipStream_t st);
// Whether the ring form of sliding-window attention (bf16 caches; a.chunk > 0 query tokens per
// workgroup, a multiple of 8) holds the bands of a window this wide.
bool swa_ring_fits(int window);
hipError_t launch_attn_merge(const MergeArgs& m, hipStream_t st);
// attn_rows: dense pass 1 for R > 32 query rows per list, bf16 or FP8 caches, bf16 MFMA;
// nrg = query-row groups of 32 per workgroup (2, 4 or 8; rows beyond 32*nrg take more z blocks)
hipError_t launch_attn_rows(const AttnArgs& a, int kvt, int nrg, hipStream_t st);
// attn_rows_scores: selection scores for R > 32 rows (G = 16 or a multiple of 32), bf16 or FP8;
// a.hist (nullable) takes the first-digit histogram when a workgroup spans at most 4 query tokens
hipError_t launch_attn_rows_scores(const ScoreArgs& a, int kvt, int nrg, hipStream_t st);
int rows_groups(int R);
int rows_tile_tokens(int nrg);
hipError_t launch_attn_scores(const ScoreArgs& a, int kvt, int ct, int nwr, hipStream_t st);
// fused_prefix: the histogram words were cleared and the first-digit histogram built by the
// kernels before (attn_wave's zero hook, scores_wave); otherwise the select does both itself.
hipError_t launch_select(const SelectArgs& a, int n_lists, bool fused_prefix, hipStream_t st);
// block-level variant (64-token blocks); max_cand = the longest list's candidate count
hipError_t launch_select_blocks(const SelectArgs& a, int n_lists, int64_t max_cand, hipStream_t st);
int64_t select_blocks_max_candidates();
hipError_t launch_scores_wave(const ScoreArgs& a, int kvt, hipStream_t st);
// candidate mode of scores_wave: tokens per unit of work (ScoreArgs::chunk), units taken in order;
// the region size (pairs) each of nper workgroups per list needs for a list of s_stride candidates
int scores_cand_chunk();
int64_t scores_cand_region(int64_t s_stride, int nper);
constexpr int SELECT_ZERO_WORDS = 4100;   // per-list words the selection needs cleared
constexpr int SELECT_CCOUNT_WORD = 4096;  // per-list word: candidate pairs appended so far
constexpr int SELECT_RCOUNT_WORD = 2048;  // candidate mode: per-list pair counts of the regions (<= 256)
constexpr int SELECT_CLAIM_WORD = 4099;   // candidate mode: per-list counter of the units taken
constexpr int SELECT_NREG_WORD = 2304;    // candidate mode: per-list number of regions (score workgroups)
static_assert(SELECT_NREG_WORD >= SELECT_RCOUNT_WORD + 256 && SELECT_NREG_WORD < SELECT_CCOUNT_WORD, "free word");
// candidate mode: score workgroups of a list with ncand candidates out of `total` over all lists
// (about 256 workgroups in all, at least one per list); the host and the kernels use this same formula
__host__ __device__ inline int cand_nper(int64_t ncand, int64_t total) {
  const int64_t n = total > 0 ? 256 * ncand / total : 0;
  return n < 1 ? 1 : (int)n;
}
static_assert(SELECT_CLAIM_WORD < SELECT_ZERO_WORDS && SELECT_CLAIM_WORD != SELECT_CCOUNT_WORD, "cleared, unshared");
// candidate mode: the score pass appended the candidate pairs (ScoreArgs::cand_off); one workgroup
// per list, lists of at most SELECT_CAND_MAX_N candidates (an LDS bitmap over them)
constexpr int SELECT_CAND_MAX_N = 1 << 20;
hipError_t launch_select_cand(const SelectArgs& a, int n_lists, hipStream_t st);
hipError_t launch_bridge(const BridgeArgs& a, hipStream_t st);
// all float32 bit patterns: the bridge's E4M3 conversion against the software RNE (counts: device, 2 words)
hipError_t launch_e4m3_check(unsigned long long* counts, hipStream_t st);
// streaming read of bytes (a multiple of 16) with grid workgroups of 512 threads; sink: 16 bytes
hipError_t launch_read_probe(const void* buf, size_t bytes, int non_temporal, int grid, void* sink, hipStream_t st);

}  // namespace hs
