// libhysparse C ABI: argument validation, workspace planning and kernel launches.
// Every check runs before anything is enqueued; on an error nothing is launched
// and no output or workspace byte is written.  The library never synchronises
// and never allocates device memory.

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "hysparse.h"
#include "hs_internal.hpp"

namespace {

thread_local std::string g_last_error;

hs_status fail(hs_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
hs_status fail(hs_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

hs_status hip_fail(hipError_t e, const char* what) {
  return fail(HS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- optional kernel timing

// Per calling thread, like the last error: each thread enables, records and collects its own
// launches (its events are kept in its own pool for reuse).
thread_local bool g_timing = false;
struct TimeRec {
  const char* name;
  hipEvent_t a, b;
};
thread_local std::vector<TimeRec> g_recs;
thread_local std::vector<hipEvent_t> g_pool;

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs one launch; when timing is on, brackets it with events on its stream.
template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_timing) return launch();
  hipEvent_t a = pool_get(), b = pool_get();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e != hipSuccess) return e;
  e = launch();
  if (e != hipSuccess) return e;
  e = hipEventRecord(b, s);
  g_recs.push_back({name, a, b});
  return e;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Kernels put lists on the second grid dimension (at most 65535 blocks).
constexpr int64_t MAX_LISTS = 65535;

int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  if (!s || !*s) return dflt;
  return atoi(s);
}

// ---------------------------------------------------------------- shared validation

struct CacheInfo {
  int B, n_kv, maxL;
  int64_t total;
};

hs_status check_cache(const hs_kv_cache* kv, CacheInfo& ci, bool need_rows) {
  if (!kv) return fail(HS_ERR_INVALID_ARGUMENT, "kv is NULL");
  if (kv->head_dim != 128) return fail(HS_ERR_UNSUPPORTED, "head_dim %d (only 128 is supported)", kv->head_dim);
  // A C caller may store any int in the enum field; read it as one before it is known to be valid
  // (a C++ load of an hs_dtype outside its enumerators is undefined).
  int32_t dt;
  memcpy(&dt, &kv->dtype, sizeof dt);
  if (dt != HS_F32 && dt != HS_BF16 && dt != HS_FP8_E4M3)
    return fail(HS_ERR_INVALID_ARGUMENT, "unknown cache dtype %d", (int)dt);
  if (kv->num_kv_heads < 1) return fail(HS_ERR_INVALID_ARGUMENT, "num_kv_heads %d", kv->num_kv_heads);
  if (!kv->k || !kv->v) return fail(HS_ERR_INVALID_ARGUMENT, "cache k/v pointer is NULL");
  if (!aligned16(kv->k) || !aligned16(kv->v)) return fail(HS_ERR_INVALID_ARGUMENT, "cache k/v not 16-byte aligned");
  const bool fp8 = kv->dtype == HS_FP8_E4M3;
  if (fp8 != (kv->k_scale != nullptr) || fp8 != (kv->v_scale != nullptr))
    return fail(HS_ERR_INVALID_ARGUMENT, "scale pointers must be given exactly for FP8 caches");
  if (kv->capacity_rows < 1) return fail(HS_ERR_INVALID_ARGUMENT, "capacity_rows %lld", (long long)kv->capacity_rows);
  ci.n_kv = kv->num_kv_heads;
  ci.B = kv->batch;
  ci.maxL = 0;
  ci.total = 0;
  if (!need_rows) return HS_OK;
  if (kv->batch < 1) return fail(HS_ERR_INVALID_ARGUMENT, "batch %d", kv->batch);
  if (!kv->d_row_start || !kv->h_row_start || !kv->d_seq_len || !kv->h_seq_len)
    return fail(HS_ERR_INVALID_ARGUMENT, "row_start / seq_len pointer is NULL");
  for (int b = 0; b < kv->batch; ++b) {
    const int64_t L = kv->h_seq_len[b], r0 = kv->h_row_start[b];
    if (L < 1) return fail(HS_ERR_INVALID_ARGUMENT, "seq_len[%d] = %lld < 1", b, (long long)L);
    if (r0 < 0 || r0 + L > kv->capacity_rows)
      return fail(HS_ERR_INVALID_ARGUMENT, "rows of sequence %d [%lld, %lld) outside capacity %lld", b,
                  (long long)r0, (long long)(r0 + L), (long long)kv->capacity_rows);
    ci.maxL = std::max<int>(ci.maxL, (int)L);
    ci.total += L;
  }
  return HS_OK;
}

hs_status check_params(const hs_attn_params* p, int n_kv) {
  if (!p) return fail(HS_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->num_q_heads < 1 || p->num_q_heads % n_kv)
    return fail(HS_ERR_INVALID_ARGUMENT, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                p->num_q_heads, n_kv);
  if (p->q_tokens < 1) return fail(HS_ERR_INVALID_ARGUMENT, "q_tokens %d", p->q_tokens);
  if (p->top_k < 0 || p->window < 0 || (int64_t)p->top_k + p->window < 1)
    return fail(HS_ERR_INVALID_ARGUMENT, "top_k %d / window %d", p->top_k, p->window);
  if (!(p->softmax_scale >= 0.f) || !isfinite(p->softmax_scale))
    return fail(HS_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (p->select_block != 0 && p->select_block != 1 && p->select_block != 64)
    return fail(HS_ERR_UNSUPPORTED, "select_block %d (0, 1 or 64)", p->select_block);
  return HS_OK;
}

// block-level selection keeps a list's block keys in LDS
hs_status check_block_select(int select_block, int64_t max_cand) {
  if (select_block == 64 && max_cand > hs::select_blocks_max_candidates())
    return fail(HS_ERR_UNSUPPORTED, "block-level selection supports at most %lld candidates per list",
                (long long)hs::select_blocks_max_candidates());
  return HS_OK;
}

float scale_log2(const hs_attn_params* p) {
  const float s = p->softmax_scale > 0.f ? p->softmax_scale : 1.0f / sqrtf(128.0f);
  return s * 1.4426950408889634f;
}

int kv_type(hs_dtype d) { return d == HS_F32 ? hs::KV_F32 : d == HS_BF16 ? hs::KV_BF16 : hs::KV_FP8; }

// ---------------------------------------------------------------- plans

struct FullPlan {
  int wave;  // 1: at most 32 query rows per KV head on a bf16 / FP8 cache -> attn_wave kernel
  int rows;  // 1: more rows, bf16 / FP8 cache -> attn_rows kernel (nrg row groups per workgroup)
  int nrg;
  int ct, nwr, G, R, n_lists, chunk, max_chunks;
  int nwr_s, chunk_s, max_chunks_s;
  int64_t s_stride;
  // candidate mode (one query token, wave path): score workgroups (about one per CU; per list
  // hs::cand_nper of its candidate count), each filling its own region of cand_region pairs
  int cand, cand_wgs, cand_uniform;
  int64_t cand_region, cand_total;
  // score filter (one query token, wave path, no dense scores asked for): the dense pass writes
  // per-(token, row) codes, the bounds pass keeps upper-bound digits and a lower-bound histogram per
  // list, the exact pass recomputes only the tokens that can reach the k'-th score (cand_wgs
  // workgroups as in candidate mode, regions of f_region pairs)
  int filter, f_chunk;
  int64_t code_tiles, u_stride, f_region;
  size_t off_acc, off_ml, off_lse2, off_scores, off_sel, off_codes, off_udig, off_lhist, total;
  hs::SelectPlan sel;
};

int pow2_at_least(int x) { int p = 1; while (p < x) p <<= 1; return p; }

hs_status plan_full(const hs_kv_cache* kv, const hs_attn_params* p, hs_dtype q_dtype, const CacheInfo& ci,
                    FullPlan& pl) {
  const int H = p->num_q_heads;
  pl.G = H / ci.n_kv;
  pl.R = p->q_tokens * pl.G;
  pl.ct = (kv->dtype == HS_F32 || q_dtype == HS_F32) ? hs::CT_F32 : hs::CT_BF16;
  // The many-row score kernel sums a query token's heads inside one workgroup of 32 * 2^i rows, so
  // a token's G rows must not straddle two workgroups: G is a power of two.
  if (!(pl.G == 8 || pl.G == 16 || pl.G == 32 || pl.G == 64 || pl.G == 128 || pl.G == 256))
    return fail(HS_ERR_UNSUPPORTED, "heads per KV head G = %d: selection scores need G in {8, 16, 32, 64, "
                "128, 256}", pl.G);
  if (pl.ct == hs::CT_F32 && pl.G > 128)
    return fail(HS_ERR_UNSUPPORTED, "fp32 queries/caches support at most 128 heads per KV head");
  pl.nwr = pl.ct == hs::CT_F32 ? (pl.R <= 32 ? 1 : 4) : hs::rows_per_wave_group(pl.R);
  pl.n_lists = ci.B * ci.n_kv;
  pl.wave = pl.ct == hs::CT_BF16 && pl.R <= 32;
  pl.rows = pl.ct == hs::CT_BF16 && pl.R > 32;
  pl.nrg = pl.rows ? hs::rows_groups(pl.R) : 0;
  const int tt = pl.wave ? 256 : pl.rows ? hs::rows_tile_tokens(pl.nrg) : hs::partial_tile_tokens(pl.nwr);
  const int zb = pl.rows ? (pl.R + 32 * pl.nrg - 1) / (32 * pl.nrg) : (pl.R + 32 * pl.nwr - 1) / (32 * pl.nwr);
  int chunk = env_int("HS_SPLIT_TOKENS", 0);
  if (chunk <= 0) {
    if (pl.wave) {
      // Whole rounds of workgroups (one 8-wave workgroup per CU at a time): the smallest chunk,
      // a multiple of 256 tokens, whose workgroup count fills r rounds of 256 for the smallest r
      // that keeps chunks <= 32768 (>= 1024).  A last round of only a few workgroups leaves HBM
      // under-used; ragged lengths make equal-size chunks land there unless the count is planned.
      auto wg_count = [&](int64_t c) {
        int64_t n = 0;
        for (int b = 0; b < ci.B; ++b) n += (kv->h_seq_len[b] + c - 1) / c;
        return n;
      };
      const int64_t cmax = (int64_t)align_up((size_t)ci.maxL, 256);
      int64_t c = 32768;
      for (int64_t r = 1; r < 1 << 20; ++r) {
        if (wg_count(cmax) > 256 * r) continue;                   // more sequences than slots
        int64_t lo = 1, hi = cmax / 256;                          // in units of 256 tokens
        while (lo < hi) {
          const int64_t mid = (lo + hi) / 2;
          if (wg_count(mid * 256) <= 256 * r) hi = mid; else lo = mid + 1;
        }
        if (lo * 256 <= 32768) { c = lo * 256; break; }
      }
      chunk = (int)std::max<int64_t>(1024, c);
    } else if (pl.rows) {
      // about 256 workgroups (one per CU: compute-bound, and few partials to merge), >= one super-tile
      const int64_t per = (ci.total * zb + 255) / 256;
      chunk = (int)std::min<int64_t>(32768, std::max<int64_t>(tt, per));
    } else {
      // about 1024 work items over the whole batch, 512..16384 tokens each
      const int64_t per = (ci.total * zb + 1023) / 1024;
      chunk = (int)std::min<int64_t>(16384, std::max<int64_t>(512, per));
    }
  }
  pl.chunk = (int)align_up((size_t)chunk, (size_t)tt);
  pl.max_chunks = (ci.maxL + pl.chunk - 1) / pl.chunk;

  int nwr_s = pl.ct == hs::CT_F32 ? (pl.R <= 32 ? 1 : pl.R <= 64 ? 2 : 4) : hs::rows_per_wave_group(pl.R);
  nwr_s = std::max(nwr_s, pow2_at_least((pl.G + 31) / 32));
  pl.nwr_s = nwr_s;
  int maxc = 0;
  for (int b = 0; b < ci.B; ++b) maxc = std::max(maxc, kv->h_seq_len[b] - std::min(p->window, kv->h_seq_len[b]));
  pl.s_stride = maxc;
  // score pass chunk: the dense one, halved for the many-row kernel (its registers allow two
  // workgroups per CU, which hide more of the latency between its MFMA and exp phases)
  pl.chunk_s = env_int("HS_SCORE_CHUNK", 0) > 0 ? (int)align_up((size_t)env_int("HS_SCORE_CHUNK", 0), 256)
               : pl.rows ? std::max(tt, (int)align_up((size_t)(pl.chunk / 2), (size_t)tt)) : pl.chunk;
  pl.max_chunks_s = (maxc + pl.chunk_s - 1) / pl.chunk_s;

  size_t off = 0;
  pl.off_acc = off;
  off += align_up((size_t)pl.n_lists * pl.max_chunks * pl.R * 128 * 4, 256);
  pl.off_ml = off;
  off += align_up((size_t)pl.n_lists * pl.max_chunks * pl.R * 2 * 4, 256);
  pl.off_lse2 = off;
  off += align_up((size_t)ci.B * p->q_tokens * H * 4, 256);
  pl.off_scores = off;
  off += align_up((size_t)ci.B * p->q_tokens * ci.n_kv * pl.s_stride * 4, 256);
  bool equal_len = true;
  for (int b = 1; b < ci.B; ++b) equal_len = equal_len && kv->h_seq_len[b] == kv->h_seq_len[0];
  // At least 16 lists (HS_CAND_MIN_LISTS): with fewer, each list has more score workgroups, which
  // contend on its counter and histogram (ragged, 8 lists: 246 us against 241 with the dense
  // selection; 16 lists: 392 against 403; 32: 707 against 737).  Ragged lengths: at most 64 lists
  // (each score workgroup finds its list by a prefix over them).
  const int cand_min_lists = env_int("HS_CAND_MIN_LISTS", 16);
  pl.cand = pl.wave && p->q_tokens == 1 && p->select_block == 0 && pl.n_lists >= cand_min_lists &&
            (equal_len || pl.n_lists <= 64) && pl.s_stride <= hs::SELECT_CAND_MAX_N &&
            !env_int("HS_DENSE_SELECT", 0);
  pl.filter = pl.wave && p->q_tokens == 1 && p->select_block == 0 && pl.s_stride <= hs::SELECT_CAND_MAX_N &&
              !env_int("HS_DENSE_SELECT", 0) && env_int("HS_SCORE_FILTER", 1) != 0;
  pl.cand_wgs = 0;
  pl.cand_region = 0;
  pl.cand_uniform = equal_len;
  pl.cand_total = 0;
  pl.f_region = 0;
  int64_t cand_pairs = 0;
  if (pl.cand || pl.filter) {
    for (int l = 0; l < pl.n_lists; ++l) {
      const int64_t L = kv->h_seq_len[l / ci.n_kv];
      pl.cand_total += L - std::min<int64_t>(p->window, L);
    }
    int max_nper = 0;
    for (int l = 0; l < pl.n_lists; ++l) {
      const int64_t L = kv->h_seq_len[l / ci.n_kv], nc = L - std::min<int64_t>(p->window, L);
      const int np = hs::cand_nper(nc, pl.cand_total);
      pl.cand_wgs += np;
      max_nper = std::max(max_nper, np);
      if (pl.cand) pl.cand_region = std::max(pl.cand_region, hs::scores_cand_region(nc, np));
      if (pl.filter)   // the exact pass: a workgroup's token range, each token at most one pair
        pl.f_region = std::max<int64_t>(pl.f_region, align_up((size_t)((nc + np - 1) / np), hs::FILTER_SPAN_ALIGN));
    }
    cand_pairs = std::max(pl.cand_region, pl.f_region) * max_nper;
  }
  hs::select_plan(pl.s_stride, pl.sel, cand_pairs);
  pl.off_sel = off;
  off += align_up((size_t)ci.B * p->q_tokens * ci.n_kv * pl.sel.ws_stride * 4, 256);
  pl.code_tiles = (ci.maxL + 31) / 32;
  pl.u_stride = (int64_t)align_up((size_t)std::max<int64_t>(pl.s_stride, 1), 32);
  pl.f_chunk = (int)align_up((size_t)std::max<int64_t>(hs::FILTER_BOUNDS_CHUNK, (pl.cand_total + 511) / 512),
                             hs::FILTER_BOUNDS_CHUNK);
  pl.off_codes = pl.off_udig = pl.off_lhist = 0;
  if (pl.filter) {
    pl.off_codes = off;
    off += align_up((size_t)pl.n_lists * pl.code_tiles * hs::CODE_TILE_BYTES, 256);
    pl.off_udig = off;
    off += align_up((size_t)pl.n_lists * pl.u_stride * 2, 256);
    pl.off_lhist = off;
    off += align_up((size_t)pl.n_lists * 2048 * 4, 256);
  }
  pl.total = off;
  return HS_OK;
}

struct SparsePlan {
  int gather;  // 1: attn_gather (bf16 Q, bf16/FP8 cache); several chunks are combined by attn_merge
  int ct, nwr, G, n_lists, chunk, max_chunks, cap;
  size_t off_acc, off_ml, total;
};

void plan_sparse(const hs_kv_cache* kv, const hs_attn_params* p, hs_dtype q_dtype, const CacheInfo& ci,
                 SparsePlan& pl) {
  pl.G = p->num_q_heads / ci.n_kv;
  pl.ct = (kv->dtype == HS_F32 || q_dtype == HS_F32) ? hs::CT_F32 : hs::CT_BF16;
  pl.nwr = pl.ct == hs::CT_F32 ? (pl.G <= 32 ? 1 : 4) : hs::rows_per_wave_group(pl.G);
  pl.n_lists = ci.B * p->q_tokens * ci.n_kv;
  pl.cap = p->top_k + p->window;
  pl.gather = pl.ct == hs::CT_BF16;
  const int tt = pl.gather ? 32 : hs::partial_tile_tokens(pl.nwr);  // attn_gather: 32-row wave tiles
  const int tiles = (pl.cap + tt - 1) / tt;
  int per_list = std::max(1, std::min(tiles, (512 + pl.n_lists - 1) / pl.n_lists));
  // attn_gather: about one workgroup per CU (256), in chunks of at least 64 rows (a multiple of the
  // 32-row wave tile): the layer is latency-bound, so spreading a list over more CUs shortens it
  // until the merge's extra partials cost more than they save.  HS_SPARSE_CHUNK overrides (>= cap:
  // one workgroup per list, no merge).
  int chunk = env_int("HS_SPARSE_CHUNK", 0);
  if (chunk <= 0 && pl.gather) {
    const int units = pl.n_lists * ((pl.G + 31) / 32);
    const int per = std::max(1, 256 / units);
    chunk = std::max(64, (int)align_up((size_t)((pl.cap + per - 1) / per), 32));
  }
  if (chunk <= 0) chunk = ((tiles + per_list - 1) / per_list) * tt;
  pl.chunk = std::min((int)align_up((size_t)chunk, (size_t)tt), 1152);
  pl.max_chunks = (pl.cap + pl.chunk - 1) / pl.chunk;
  size_t off = 0;
  pl.off_acc = off;
  off += align_up((size_t)pl.n_lists * pl.max_chunks * pl.G * 128 * 4, 256);
  pl.off_ml = off;
  off += align_up((size_t)pl.n_lists * pl.max_chunks * pl.G * 2 * 4, 256);
  pl.total = off;
}

}  // namespace

namespace {

// Shared by hs_kv_bridge and hs_kv_append: validates the targets and fills the launch arguments.
// Rows are checked by the callers.
hs_status bridge_args(const void* hidden, int64_t n_tokens, int32_t d_model, int32_t n_targets,
                      const void* const* w_k, const void* const* w_v, const hs_kv_cache* const* targets,
                      hs::BridgeArgs& a) {
  if (!hidden || !w_k || !w_v || !targets) return fail(HS_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (n_tokens < 0) return fail(HS_ERR_INVALID_ARGUMENT, "n_tokens %lld", (long long)n_tokens);
  if (d_model < 64 || d_model % 64) return fail(HS_ERR_INVALID_ARGUMENT, "d_model %d must be a positive multiple of 64", d_model);
  if (n_targets < 1 || n_targets > 8) return fail(HS_ERR_UNSUPPORTED, "n_targets %d (1..8 supported)", n_targets);
  if (!aligned16(hidden)) return fail(HS_ERR_INVALID_ARGUMENT, "hidden not 16-byte aligned");
  int fp8 = -1;
  for (int l = 0; l < n_targets; ++l) {
    const hs_kv_cache* t = targets[l];
    if (!t || !w_k[l] || !w_v[l]) return fail(HS_ERR_INVALID_ARGUMENT, "target %d: NULL pointer", l);
    CacheInfo ci;
    hs_status st = check_cache(t, ci, false);
    if (st != HS_OK) return st;
    if (t->dtype != HS_BF16 && t->dtype != HS_FP8_E4M3)
      return fail(HS_ERR_INVALID_ARGUMENT, "target %d: bridge output must be BF16 or FP8_E4M3", l);
    if (t->num_kv_heads != 1) return fail(HS_ERR_UNSUPPORTED, "target %d: bridge targets have one KV head", l);
    const int f = t->dtype == HS_FP8_E4M3;
    if (fp8 >= 0 && f != fp8) return fail(HS_ERR_UNSUPPORTED, "all targets of one call must share a dtype");
    fp8 = f;
    if (!aligned16(w_k[l]) || !aligned16(w_v[l])) return fail(HS_ERR_INVALID_ARGUMENT, "target %d: weights not 16-byte aligned", l);
    a.w[2 * l] = (const uint16_t*)w_k[l];
    a.w[2 * l + 1] = (const uint16_t*)w_v[l];
    a.out[2 * l] = t->k;
    a.out[2 * l + 1] = t->v;
    a.scale[2 * l] = t->k_scale;
    a.scale[2 * l + 1] = t->v_scale;
  }
  a.x = (const uint16_t*)hidden; a.T = n_tokens; a.Dm = d_model; a.n_targets = n_targets; a.fp8 = fp8;
  return HS_OK;
}

// ---------------------------------------------------------------- static scratch of hs_sparse_attn_noalloc

// The sparse layer's chunk partials for callers that cannot allocate: one array per GPU, loaded with
// the library's code object and kept until the process ends.  Host code never uses the array's name
// as an address (on the host it is only a stand-in): the device address of each GPU's copy is looked
// up once, with that device current, and kept here.
__device__ __align__(256) static char scratch[HS_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

// Device address of the current device's scratch array; the stream (null: the current device's null
// stream) must belong to that device.
hs_status scratch_for_stream(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(HS_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, MAX_DEVICES);
  if (stream) {
    int sdev = -1;
    if ((e = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(HS_ERR_INVALID_ARGUMENT, "stream of device %d while device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess)
      return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(HS_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HS_OK;
}

// hs_sparse_attn with its scratch either from the caller's workspace or (noalloc) from the static array.
hs_status sparse_attn_impl(const hs_kv_cache* kv, const hs_attn_params* p, const void* q, hs_dtype q_dtype,
                           const int32_t* sel_idx, const int32_t* sel_count, float* out, void* workspace,
                           size_t workspace_bytes, bool noalloc, void* stream);

// hs_swa_attn's checks and launch arguments (nothing is launched here).
// od: the output dtype's value, read from the caller's enum as an int (a C caller may pass any value)
hs_status swa_prepare(const hs_kv_cache* kv, const hs_attn_params* p, const void* q, hs_dtype q_dtype, void* out,
                      int32_t od, hs::AttnArgs& a) {
  CacheInfo ci;
  hs_status st = check_cache(kv, ci, true);
  if (st != HS_OK) return st;
  if (!p) return fail(HS_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->num_q_heads < 1 || p->num_q_heads % ci.n_kv)
    return fail(HS_ERR_INVALID_ARGUMENT, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                p->num_q_heads, ci.n_kv);
  if (p->window < 1) return fail(HS_ERR_INVALID_ARGUMENT, "window %d must be >= 1", p->window);
  if (!(p->softmax_scale >= 0.f) || !isfinite(p->softmax_scale))
    return fail(HS_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (p->q_tokens < 1) return fail(HS_ERR_INVALID_ARGUMENT, "q_tokens %d", p->q_tokens);
  for (int b = 0; b < kv->batch; ++b)
    if (p->q_tokens > kv->h_seq_len[b])
      return fail(HS_ERR_INVALID_ARGUMENT, "q_tokens %d > seq_len[%d] = %d", p->q_tokens, b, kv->h_seq_len[b]);
  if (!q || !out) return fail(HS_ERR_INVALID_ARGUMENT, "q/out is NULL");
  if (q_dtype != HS_BF16) return fail(HS_ERR_UNSUPPORTED, "q dtype must be BF16");
  if (od != HS_F32 && od != HS_BF16) return fail(HS_ERR_INVALID_ARGUMENT, "output dtype %d (F32 or BF16)", (int)od);
  if (kv->dtype == HS_F32) return fail(HS_ERR_UNSUPPORTED, "F32 caches are not supported here");
  if (!aligned16(q) || !aligned16(out)) return fail(HS_ERR_INVALID_ARGUMENT, "q/out not 16-byte aligned");
  if ((int64_t)kv->batch * ci.n_kv > MAX_LISTS) return fail(HS_ERR_UNSUPPORTED, "batch * num_kv_heads > 65535");
  a = hs::AttnArgs{};
  a.k = kv->k; a.v = kv->v; a.k_scale = kv->k_scale; a.v_scale = kv->v_scale;
  a.row_start = kv->d_row_start; a.seq_len = kv->d_seq_len;
  a.q = q; a.q_f32 = 0;
  a.n_kv = ci.n_kv; a.H = p->num_q_heads; a.G = p->num_q_heads / ci.n_kv; a.n_q = p->q_tokens;
  a.R = a.G; a.n_lists = kv->batch * ci.n_kv;
  a.scale_log2 = scale_log2(p);
  a.out = (float*)out; a.out_bf16 = od == HS_BF16; a.window = p->window;
  // bf16 caches with windows the ring form holds: contiguous token ranges, a multiple of 8 tokens
  // each, sized so the workgroups fill one round of the 256 CUs.  HS_SWA_RING=0 selects the
  // per-group form, a value n >= 2 fixes n tokens (rounded up to a multiple of 8) per workgroup.
  a.chunk = 0;
  const int ring = env_int("HS_SWA_RING", 1);
  if (kv->dtype == HS_BF16 && hs::swa_ring_fits(p->window) && ring != 0) {
    const int64_t units = (int64_t)a.n_lists * ((a.G + 31) / 32);
    const int64_t per_unit = std::max<int64_t>(1, (256 + units - 1) / units);
    const int64_t tokens = ring >= 2 ? ring : (a.n_q + per_unit - 1) / per_unit;
    a.chunk = (int)align_up((size_t)std::min<int64_t>(tokens, a.n_q), 8);
  }
  return HS_OK;
}

// hs_kv_bridge's checks and launch arguments (nothing is launched here).
hs_status bridge_prepare(const void* hidden, int64_t n_tokens, int32_t d_model, int32_t n_targets,
                         const void* const* w_k, const void* const* w_v, const hs_kv_cache* const* targets,
                         int64_t row_offset, hs::BridgeArgs& a) {
  a = hs::BridgeArgs{};
  hs_status st = bridge_args(hidden, n_tokens, d_model, n_targets, w_k, w_v, targets, a);
  if (st != HS_OK) return st;
  if (row_offset < 0) return fail(HS_ERR_INVALID_ARGUMENT, "row_offset %lld", (long long)row_offset);
  for (int l = 0; l < n_targets; ++l)
    if (row_offset + n_tokens > targets[l]->capacity_rows)
      return fail(HS_ERR_INVALID_ARGUMENT, "target %d: rows [%lld, %lld) exceed capacity %lld", l,
                  (long long)row_offset, (long long)(row_offset + n_tokens), (long long)targets[l]->capacity_rows);
  a.row_offset = row_offset;
  return HS_OK;
}

}  // namespace

extern "C" {

int hs_abi_version(void) { return HS_ABI_VERSION; }

const char* hs_status_string(hs_status s) {
  switch (s) {
    case HS_OK: return "HS_OK";
    case HS_ERR_INVALID_ARGUMENT: return "HS_ERR_INVALID_ARGUMENT";
    case HS_ERR_UNSUPPORTED: return "HS_ERR_UNSUPPORTED";
    case HS_ERR_WORKSPACE_TOO_SMALL: return "HS_ERR_WORKSPACE_TOO_SMALL";
    case HS_ERR_HIP: return "HS_ERR_HIP";
  }
  return "unknown hs_status";
}

const char* hs_last_error(void) { return g_last_error.c_str(); }

void hs_timing_enable(int enable) { g_timing = enable != 0; }

int hs_timing_collect(hs_kernel_time* out, int max) {
  int n = 0;
  bool ok = true;
  for (const TimeRec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) ok = false;
    if (out && n < max) out[n++] = hs_kernel_time{r.name, ms};
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return ok ? n : -1;
}

hs_status hs_read_probe(const void* buf, size_t bytes, int non_temporal, int32_t grid, void* sink, void* stream) {
  g_last_error.clear();
  if (!buf || !sink) return fail(HS_ERR_INVALID_ARGUMENT, "buf/sink is NULL");
  if (!aligned16(buf) || !aligned16(sink) || bytes % 16)
    return fail(HS_ERR_INVALID_ARGUMENT, "buf/sink not 16-byte aligned or bytes %zu not a multiple of 16", bytes);
  if (grid < 1 || grid > 65535) return fail(HS_ERR_INVALID_ARGUMENT, "grid %d", grid);
  hipError_t e = timed("read_probe", (hipStream_t)stream,
                       [&] { return hs::launch_read_probe(buf, bytes, non_temporal, grid, sink, (hipStream_t)stream); });
  if (e != hipSuccess) return hip_fail(e, "read probe");
  return HS_OK;
}

hs_status hs_e4m3_check(unsigned long long* counts, void* stream) {
  g_last_error.clear();
  if (!counts) return fail(HS_ERR_INVALID_ARGUMENT, "counts is NULL");
  if ((uintptr_t)counts % 8) return fail(HS_ERR_INVALID_ARGUMENT, "counts not 8-byte aligned");
  hipError_t e = timed("e4m3_check", (hipStream_t)stream, [&] { return hs::launch_e4m3_check(counts, (hipStream_t)stream); });
  if (e != hipSuccess) return hip_fail(e, "e4m3 check");
  return HS_OK;
}

size_t hs_full_attn_select_workspace_size(const hs_kv_cache* kv, const hs_attn_params* p) {
  // a size query leaves the caller's last error as it was
  const std::string saved = g_last_error;
  size_t need = 0;
  CacheInfo ci;
  if (check_cache(kv, ci, true) == HS_OK && check_params(p, ci.n_kv) == HS_OK) {
    // The plan depends on the query type only through the compute type: each plan is sized on its
    // own (fp32 plans reject more than 128 heads per KV head, bf16 plans allow 256), and the
    // largest plan that exists is the answer.
    for (hs_dtype qt : {HS_F32, HS_BF16}) {
      FullPlan pl;
      if (plan_full(kv, p, qt, ci, pl) == HS_OK) need = std::max(need, pl.total);
    }
  }
  g_last_error = saved;
  return need;
}

size_t hs_sparse_attn_workspace_size(const hs_kv_cache* kv, const hs_attn_params* p) {
  const std::string saved = g_last_error;
  size_t need = 0;
  CacheInfo ci;
  if (check_cache(kv, ci, true) == HS_OK && check_params(p, ci.n_kv) == HS_OK) {
    SparsePlan a, b;
    plan_sparse(kv, p, HS_F32, ci, a);
    plan_sparse(kv, p, HS_BF16, ci, b);
    need = std::max(a.total, b.total);
  }
  g_last_error = saved;
  return need;
}

size_t hs_select_workspace_size(int32_t batch, int32_t q_tokens, int32_t n_kv, int32_t max_len, int32_t top_k,
                                int32_t window) {
  if (batch < 1 || q_tokens < 1 || n_kv < 1 || max_len < 1 || top_k < 0 || window < 0) return 0;
  hs::SelectPlan sp;
  hs::select_plan(max_len - std::min(window, max_len), sp);
  return align_up((size_t)batch * q_tokens * n_kv * sp.ws_stride * 4, 256);
}

hs_status hs_full_attn_select(const hs_kv_cache* kv, const hs_attn_params* p, const void* q, hs_dtype q_dtype,
                              float* out, float* lse, int32_t* sel_idx, int32_t* sel_count, float* scores_out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  CacheInfo ci;
  hs_status st = check_cache(kv, ci, true);
  if (st != HS_OK) return st;
  if ((st = check_params(p, ci.n_kv)) != HS_OK) return st;
  if (!q || !out || !sel_idx || !sel_count) return fail(HS_ERR_INVALID_ARGUMENT, "q/out/sel_idx/sel_count is NULL");
  if (q_dtype != HS_F32 && q_dtype != HS_BF16) return fail(HS_ERR_INVALID_ARGUMENT, "q dtype must be F32 or BF16");
  if (!aligned16(q)) return fail(HS_ERR_INVALID_ARGUMENT, "q not 16-byte aligned");
  if (!aligned16(out)) return fail(HS_ERR_INVALID_ARGUMENT, "out not 16-byte aligned");
  if (!aligned4(lse) || !aligned4(sel_idx) || !aligned4(sel_count) || !aligned4(scores_out))
    return fail(HS_ERR_INVALID_ARGUMENT, "lse/sel_idx/sel_count/scores_out not 4-byte aligned");
  if ((int64_t)ci.B * p->q_tokens * ci.n_kv > MAX_LISTS)
    return fail(HS_ERR_UNSUPPORTED, "batch * q_tokens * num_kv_heads = %lld selection lists (at most %lld)",
                (long long)ci.B * p->q_tokens * ci.n_kv, (long long)MAX_LISTS);
  FullPlan pl;
  if ((st = plan_full(kv, p, q_dtype, ci, pl)) != HS_OK) return st;
  if ((st = check_block_select(p->select_block, pl.s_stride)) != HS_OK) return st;
  if (!workspace && pl.total) return fail(HS_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (workspace_bytes < pl.total)
    return fail(HS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, pl.total);
  if (!aligned16(workspace)) return fail(HS_ERR_INVALID_ARGUMENT, "workspace not 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int kvt = kv_type(kv->dtype);
  const float sl2 = scale_log2(p);
  float* lse2 = (float*)(ws + pl.off_lse2);
  float* scores = scores_out ? scores_out : (float*)(ws + pl.off_scores);

  hs::AttnArgs a{};
  a.k = kv->k; a.v = kv->v; a.k_scale = kv->k_scale; a.v_scale = kv->v_scale;
  a.row_start = kv->d_row_start; a.seq_len = kv->d_seq_len;
  a.q = q; a.q_f32 = q_dtype == HS_F32;
  a.n_kv = ci.n_kv; a.H = p->num_q_heads; a.G = pl.G; a.n_q = p->q_tokens;
  a.R = pl.R; a.n_lists = pl.n_lists; a.chunk = pl.chunk; a.max_chunks = pl.max_chunks;
  a.scale_log2 = sl2;
  a.part_acc = (float*)(ws + pl.off_acc); a.part_ml = (float*)(ws + pl.off_ml);
  a.direct = pl.wave && pl.max_chunks == 1; a.out = out; a.lse = lse; a.lse2 = lse2;
  const int n_sel_lists = ci.B * p->q_tokens * ci.n_kv;
  // the many-row score kernel builds the selection's first-digit histogram when a workgroup spans
  // at most 4 query tokens
  const bool rows_scores = pl.rows && pl.G >= 16;
  const bool rows_hist = rows_scores && (pl.G >= 32 * pl.nrg ? 1 : 32 * pl.nrg / pl.G) <= 4;
  const bool fused_prefix = pl.wave || rows_hist;
  if (fused_prefix) {
    a.zero_ptr = (uint32_t*)(ws + pl.off_sel);                 // the selection's histograms, cleared here
    a.zero_stride = pl.sel.ws_stride;
    a.zero_words = hs::SELECT_ZERO_WORDS;
    a.zero_lists = n_sel_lists;
  }
  // score filter when no dense scores are asked for: the dense pass leaves its codes and clears the
  // lower-bound histograms
  const bool use_filter = pl.filter && !scores_out;
  if (use_filter) {
    a.codes = (uint8_t*)(ws + pl.off_codes);
    a.code_tiles = pl.code_tiles;
    a.zero2_ptr = (uint32_t*)(ws + pl.off_lhist);
    a.zero2_words = (int64_t)pl.n_lists * 2048;
  }
  // items of the one-dimensional grids: chunks with work per list (lists in order)
  // (and the per-list count when it is the same for every list, which spares the kernel the search)
  auto count_items = [&](int chunk, int sub, int min_items, int& uniform) {
    int64_t n = 0;
    uniform = -1;
    for (int b = 0; b < ci.B; ++b) {
      const int L = kv->h_seq_len[b];
      const int c = std::max(min_items, (L - std::min(sub, L) + chunk - 1) / chunk);
      uniform = uniform == -1 || uniform == c ? c : 0;
      n += (int64_t)ci.n_kv * c;
    }
    if (uniform < 0 || env_int("HS_GRID_SEARCH", 0)) uniform = 0;
    return (int)n;
  };
  a.n_items = count_items(pl.chunk, 0, 1, a.uniform_items);
  hipError_t e;
  if (pl.wave)
    e = timed("attn_wave_dense", s, [&] { return hs::launch_attn_wave(a, kvt, s); });
  else if (pl.rows) {
    // opt-in: Q K^T of the many-row pass on FP8 MFMA for E4M3 caches (Q quantised per row)
    a.qk_fp8 = kvt == hs::KV_FP8 && env_int("HS_MANY_ROW_FP8_QK", 0) != 0;
    e = timed("attn_rows_dense", s, [&] { return hs::launch_attn_rows(a, kvt, pl.nrg, s); });
  }
  else
    e = timed("attn_partial_dense", s, [&] { return hs::launch_attn_partial(a, kvt, pl.ct, pl.nwr, false, s); });
  if (e != hipSuccess) return hip_fail(e, "full attention pass 1");

  hs::MergeArgs m{};
  m.part_acc = a.part_acc; m.part_ml = a.part_ml; m.seq_len = kv->d_seq_len; m.sel_count = nullptr;
  m.gather = 0; m.n_kv = ci.n_kv; m.H = a.H; m.G = pl.G; m.n_q = a.n_q; m.R = pl.R; m.n_lists = pl.n_lists;
  m.chunk = pl.chunk; m.max_chunks = pl.max_chunks; m.out = out; m.lse = lse; m.lse2 = lse2;
  const bool fold_merge = pl.wave && !a.direct && pl.max_chunks <= 64;   // scores_wave merges O, writes LSE
  // candidate mode: the score pass appends the pairs that can still reach the k'-th key and the
  // selection runs on them in one workgroup per list; dense scores only on request
  const bool cand_mode = pl.cand;
  if (!a.direct && !fold_merge)                                   // several chunks: merge them
    if ((e = timed("attn_merge_dense", s, [&] { return hs::launch_attn_merge(m, s); })) != hipSuccess)
      return hip_fail(e, "full attention merge");

  if (use_filter) {
    hs::FilterArgs fa{};
    fa.k = kv->k; fa.k_scale = kv->k_scale; fa.row_start = kv->d_row_start; fa.seq_len = kv->d_seq_len;
    fa.q = q; fa.q_f32 = a.q_f32; fa.n_kv = ci.n_kv; fa.H = a.H; fa.G = pl.G; fa.R = pl.R; fa.n_lists = pl.n_lists;
    fa.window = p->window; fa.top_k = p->top_k; fa.scale_log2 = sl2;
    fa.codes = a.codes; fa.code_tiles = pl.code_tiles;
    fa.udig = (uint16_t*)(ws + pl.off_udig); fa.u_stride = pl.u_stride;
    fa.lhist = (uint32_t*)(ws + pl.off_lhist); fa.lse2 = lse2;
    fa.chunk = pl.f_chunk;
    fa.n_items = count_items(pl.f_chunk, p->window, 1, fa.uniform_items);
    if (fold_merge) {
      fa.part_acc = a.part_acc; fa.part_ml = a.part_ml; fa.dchunk = pl.chunk; fa.dmax_chunks = pl.max_chunks;
      fa.out = out; fa.lse = lse;
    }
    fa.sel_ws = (uint32_t*)(ws + pl.off_sel); fa.sel_stride = pl.sel.ws_stride; fa.cand_off = pl.sel.cand_off;
    fa.cand_region = pl.f_region; fa.cand_total = pl.cand_total; fa.cand_uniform = pl.cand_uniform;
    fa.n_wg2 = pl.cand_wgs;
    if ((e = timed("filter_bounds", s, [&] { return hs::launch_filter_bounds(fa, s); })) != hipSuccess)
      return hip_fail(e, "score filter bounds");
    if ((e = timed("filter_exact", s, [&] { return hs::launch_filter_exact(fa, kvt, s); })) != hipSuccess)
      return hip_fail(e, "score filter exact scores");
  } else if (pl.max_chunks_s > 0 || fold_merge) {
    hs::ScoreArgs sa{};
    sa.k = kv->k; sa.k_scale = kv->k_scale; sa.row_start = kv->d_row_start; sa.seq_len = kv->d_seq_len;
    sa.q = q; sa.q_f32 = a.q_f32; sa.n_kv = ci.n_kv; sa.H = a.H; sa.G = pl.G; sa.n_q = a.n_q; sa.R = pl.R;
    sa.n_lists = pl.n_lists; sa.window = p->window; sa.chunk = pl.chunk_s; sa.max_chunks = pl.max_chunks_s;
    sa.scale_log2 = sl2; sa.lse2 = lse2; sa.scores = scores; sa.s_stride = pl.s_stride;
    if (rows_scores) {
      if (rows_hist) {
        sa.hist = (uint32_t*)(ws + pl.off_sel);
        sa.hist_stride = pl.sel.ws_stride;
      }
      if ((e = timed("attn_rows_scores", s, [&] { return hs::launch_attn_rows_scores(sa, kvt, pl.nrg, s); })) !=
          hipSuccess)
        return hip_fail(e, "selection scores");
    } else if (pl.wave) {
      sa.hist = (uint32_t*)(ws + pl.off_sel);
      sa.hist_stride = pl.sel.ws_stride;
      if (fold_merge) {
        sa.part_acc = a.part_acc; sa.part_ml = a.part_ml; sa.dchunk = pl.chunk; sa.dmax_chunks = pl.max_chunks;
        sa.out = out; sa.lse = lse;
      }
      sa.n_items = count_items(pl.chunk_s, p->window, fold_merge ? 1 : 0, sa.uniform_items);
      if (cand_mode) {                                            // about one workgroup per CU, each on one list
        sa.scores = scores_out;                                   // nullable: the test hook only
        sa.cand_off = pl.sel.cand_off;
        sa.cand_region = pl.cand_region;
        sa.cand_uniform = pl.cand_uniform;
        sa.cand_total = pl.cand_total;
        sa.top_k = p->top_k;
        sa.chunk = hs::scores_cand_chunk();
        sa.n_items = pl.cand_wgs;
      }
      if (sa.n_items > 0 &&
          (e = timed("scores_wave", s, [&] { return hs::launch_scores_wave(sa, kvt, s); })) != hipSuccess)
        return hip_fail(e, "selection scores");
    } else if ((e = timed("attn_scores", s, [&] { return hs::launch_attn_scores(sa, kvt, pl.ct, pl.nwr_s, s); })) !=
               hipSuccess) {
      return hip_fail(e, "selection scores");
    }
  }

  hs::SelectArgs se{};
  se.scores = scores; se.s_stride = pl.s_stride; se.seq_len = kv->d_seq_len; se.n_q = p->q_tokens;
  se.n_kv = ci.n_kv; se.top_k = p->top_k; se.window = p->window; se.cap = p->top_k + p->window;
  se.sel_idx = sel_idx; se.sel_count = sel_count;
  se.ws = (uint32_t*)(ws + pl.off_sel); se.ws_stride = pl.sel.ws_stride; se.cand_off = pl.sel.cand_off;
  se.chunk = pl.sel.chunk; se.max_chunks = pl.sel.max_chunks;
  se.cand_region = use_filter ? pl.f_region : pl.cand_region;   // region count per list: from the score pass
  if (p->select_block == 64)
    e = timed("select_blocks", s, [&] { return hs::launch_select_blocks(se, n_sel_lists, pl.s_stride, s); });
  else if (cand_mode || use_filter)
    e = timed("select_cand", s, [&] { return hs::launch_select_cand(se, n_sel_lists, s); });
  else
    e = timed("select_topk", s, [&] { return hs::launch_select(se, n_sel_lists, fused_prefix, s); });
  if (e != hipSuccess) return hip_fail(e, "selection");
  return HS_OK;
}

hs_status hs_sparse_attn(const hs_kv_cache* kv, const hs_attn_params* p, const void* q, hs_dtype q_dtype,
                         const int32_t* sel_idx, const int32_t* sel_count, float* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return sparse_attn_impl(kv, p, q, q_dtype, sel_idx, sel_count, out, workspace, workspace_bytes, false, stream);
}

hs_status hs_sparse_attn_noalloc(const hs_kv_cache* kv, const hs_attn_params* p, const void* q, hs_dtype q_dtype,
                                 const int32_t* sel_idx, const int32_t* sel_count, float* out, void* stream) {
  g_last_error.clear();
  return sparse_attn_impl(kv, p, q, q_dtype, sel_idx, sel_count, out, nullptr, 0, true, stream);
}

hs_status hs_swa_attn(const hs_kv_cache* kv, const hs_attn_params* p, const void* q, hs_dtype q_dtype,
                      float* out, void* stream) {
  return hs_swa_attn_out(kv, p, q, q_dtype, out, HS_F32, stream);
}

hs_status hs_swa_attn_out(const hs_kv_cache* kv, const hs_attn_params* p, const void* q, hs_dtype q_dtype,
                          void* out, hs_dtype out_dtype, void* stream) {
  g_last_error.clear();
  int32_t od;
  memcpy(&od, &out_dtype, sizeof od);
  hs::AttnArgs a{};
  hs_status st = swa_prepare(kv, p, q, q_dtype, out, od, a);
  if (st != HS_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed("swa_attn", s, [&] { return hs::launch_swa_attn(a, kv_type(kv->dtype), s); });
  if (e != hipSuccess) return hip_fail(e, "sliding-window attention");
  return HS_OK;
}

hs_status hs_select_from_scores(const float* scores, const int32_t* d_seq_len, const int32_t* h_seq_len,
                                int32_t batch, int32_t q_tokens, int32_t n_kv, int32_t max_len, int32_t top_k,
                                int32_t window, int32_t select_block, int32_t* sel_idx, int32_t* sel_count,
                                void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!scores || !d_seq_len || !h_seq_len || !sel_idx || !sel_count)
    return fail(HS_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (batch < 1 || q_tokens < 1 || n_kv < 1 || max_len < 1)
    return fail(HS_ERR_INVALID_ARGUMENT, "batch/q_tokens/n_kv/max_len must be >= 1");
  if (top_k < 0 || window < 0 || (int64_t)top_k + window < 1)
    return fail(HS_ERR_INVALID_ARGUMENT, "top_k %d / window %d", top_k, window);
  for (int b = 0; b < batch; ++b)
    if (h_seq_len[b] < 1 || h_seq_len[b] > max_len)
      return fail(HS_ERR_INVALID_ARGUMENT, "seq_len[%d] = %d outside [1, max_len]", b, h_seq_len[b]);
  if (select_block != 0 && select_block != 1 && select_block != 64)
    return fail(HS_ERR_UNSUPPORTED, "select_block %d (0, 1 or 64)", select_block);
  if (!aligned4(scores) || !aligned4(sel_idx) || !aligned4(sel_count))
    return fail(HS_ERR_INVALID_ARGUMENT, "scores/sel_idx/sel_count not 4-byte aligned");
  if ((int64_t)batch * q_tokens * n_kv > MAX_LISTS)
    return fail(HS_ERR_UNSUPPORTED, "batch * q_tokens * n_kv = %lld selection lists (at most %lld)",
                (long long)batch * q_tokens * n_kv, (long long)MAX_LISTS);
  hs_status bst = check_block_select(select_block, max_len - std::min(window, max_len));
  if (bst != HS_OK) return bst;
  const size_t need = hs_select_workspace_size(batch, q_tokens, n_kv, max_len, top_k, window);
  if (!workspace) return fail(HS_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(HS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(HS_ERR_INVALID_ARGUMENT, "workspace not 16-byte aligned");
  hs::SelectArgs se{};
  se.scores = scores; se.s_stride = max_len - std::min(window, max_len); se.seq_len = d_seq_len;
  se.n_q = q_tokens; se.n_kv = n_kv; se.top_k = top_k; se.window = window; se.cap = top_k + window;
  se.sel_idx = sel_idx; se.sel_count = sel_count;
  hs::SelectPlan sp;
  hs::select_plan(se.s_stride, sp);
  se.ws = (uint32_t*)workspace; se.ws_stride = sp.ws_stride; se.cand_off = sp.cand_off;
  se.chunk = sp.chunk; se.max_chunks = sp.max_chunks;
  const int n_lists = batch * q_tokens * n_kv;
  hipError_t e = select_block == 64
                     ? timed("select_blocks", (hipStream_t)stream,
                             [&] { return hs::launch_select_blocks(se, n_lists, se.s_stride, (hipStream_t)stream); })
                     : timed("select_topk", (hipStream_t)stream,
                             [&] { return hs::launch_select(se, n_lists, false, (hipStream_t)stream); });
  if (e != hipSuccess) return hip_fail(e, "selection");
  return HS_OK;
}

hs_status hs_kv_bridge(const void* hidden, int64_t n_tokens, int32_t d_model, int32_t n_targets,
                       const void* const* w_k, const void* const* w_v, const hs_kv_cache* const* targets,
                       int64_t row_offset, void* stream) {
  g_last_error.clear();
  hs::BridgeArgs a;
  hs_status st = bridge_prepare(hidden, n_tokens, d_model, n_targets, w_k, w_v, targets, row_offset, a);
  if (st != HS_OK) return st;
  if (n_tokens == 0) return HS_OK;
  hipError_t e = timed("kv_bridge", (hipStream_t)stream, [&] { return hs::launch_bridge(a, (hipStream_t)stream); });
  if (e != hipSuccess) return hip_fail(e, "kv bridge");
  return HS_OK;
}

hs_status hs_prefill_chunk(const hs_kv_cache* self_kv, const hs_attn_params* swa_p, const void* q, hs_dtype q_dtype,
                           void* swa_out, hs_dtype swa_out_dtype, const void* hidden, int64_t n_tokens,
                           int32_t d_model, int32_t n_targets, const void* const* w_k, const void* const* w_v,
                           const hs_kv_cache* const* targets, int64_t row_offset, void* stream) {
  g_last_error.clear();
  int32_t od;
  memcpy(&od, &swa_out_dtype, sizeof od);
  hs::AttnArgs sa;
  hs_status st = swa_prepare(self_kv, swa_p, q, q_dtype, swa_out, od, sa);
  if (st != HS_OK) return st;
  if (self_kv->batch != 1) return fail(HS_ERR_INVALID_ARGUMENT, "the chunk belongs to one prompt: batch %d", self_kv->batch);
  if (swa_p->q_tokens != n_tokens)
    return fail(HS_ERR_INVALID_ARGUMENT, "q_tokens %d != n_tokens %lld: the chunk's queries and hidden states",
                swa_p->q_tokens, (long long)n_tokens);
  hs::BridgeArgs ba;
  if ((st = bridge_prepare(hidden, n_tokens, d_model, n_targets, w_k, w_v, targets, row_offset, ba)) != HS_OK)
    return st;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = timed("swa_attn", s, [&] { return hs::launch_swa_attn(sa, kv_type(self_kv->dtype), s); });
  if (e != hipSuccess) return hip_fail(e, "sliding-window attention");
  if ((e = timed("kv_bridge", s, [&] { return hs::launch_bridge(ba, s); })) != hipSuccess) return hip_fail(e, "kv bridge");
  return HS_OK;
}

size_t hs_kv_append_workspace_size(int64_t n_tokens, int32_t d_model, int32_t n_targets) {
  if (n_tokens < 1 || n_tokens > hs::APPEND_MAX_TOKENS || d_model < 64 || d_model % 64 || n_targets < 1 ||
      n_targets > 8)
    return 0;
  hs::AppendArgs ap{};
  hs::append_plan(n_tokens, d_model, n_targets, ap);
  return hs::append_workspace_bytes(ap);
}

hs_status hs_kv_append(const void* hidden, int64_t n_tokens, int32_t d_model, int32_t n_targets,
                       const void* const* w_k, const void* const* w_v, const hs_kv_cache* const* targets,
                       const int64_t* d_rows, const int64_t* h_rows, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_last_error.clear();
  hs::BridgeArgs a{};
  hs_status st = bridge_args(hidden, n_tokens, d_model, n_targets, w_k, w_v, targets, a);
  if (st != HS_OK) return st;
  if (n_tokens > 0 && (!d_rows || !h_rows)) return fail(HS_ERR_INVALID_ARGUMENT, "d_rows / h_rows is NULL");
  int64_t cap = INT64_MAX;
  for (int l = 0; l < n_targets; ++l) cap = std::min<int64_t>(cap, targets[l]->capacity_rows);
  std::vector<int64_t> sorted(h_rows, h_rows + n_tokens);
  std::sort(sorted.begin(), sorted.end());
  for (int64_t i = 0; i < n_tokens; ++i) {
    if (sorted[i] < 0 || sorted[i] >= cap)
      return fail(HS_ERR_INVALID_ARGUMENT, "row %lld outside [0, %lld)", (long long)sorted[i], (long long)cap);
    if (i && sorted[i] == sorted[i - 1])
      return fail(HS_ERR_INVALID_ARGUMENT, "row %lld named twice", (long long)sorted[i]);
  }
  if (n_tokens == 0) return HS_OK;
  hipError_t e;
  if (n_tokens <= hs::APPEND_MAX_TOKENS) {
    hs::AppendArgs ap{};
    hs::append_plan(n_tokens, d_model, n_targets, ap);
    const size_t need = hs::append_workspace_bytes(ap);
    if (!workspace) return fail(HS_ERR_INVALID_ARGUMENT, "workspace is NULL");
    if (workspace_bytes < need)
      return fail(HS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    if (!aligned16(workspace)) return fail(HS_ERR_INVALID_ARGUMENT, "workspace not 16-byte aligned");
    ap.x = a.x; ap.T = n_tokens; ap.Dm = d_model; ap.fp8 = a.fp8; ap.rows = d_rows; ap.part = (float*)workspace;
    for (int i = 0; i < 2 * n_targets; ++i) { ap.w[i] = a.w[i]; ap.out[i] = a.out[i]; ap.scale[i] = a.scale[i]; }
    e = timed("kv_append", (hipStream_t)stream, [&] { return hs::launch_append(ap, (hipStream_t)stream); });
  } else {
    a.rows = d_rows;
    e = timed("kv_append", (hipStream_t)stream, [&] { return hs::launch_bridge(a, (hipStream_t)stream); });
  }
  if (e != hipSuccess) return hip_fail(e, "kv append");
  return HS_OK;
}

}  // extern "C"

namespace {

hs_status sparse_attn_impl(const hs_kv_cache* kv, const hs_attn_params* p, const void* q, hs_dtype q_dtype,
                           const int32_t* sel_idx, const int32_t* sel_count, float* out, void* workspace,
                           size_t workspace_bytes, bool noalloc, void* stream) {
  CacheInfo ci;
  hs_status st = check_cache(kv, ci, true);
  if (st != HS_OK) return st;
  if ((st = check_params(p, ci.n_kv)) != HS_OK) return st;
  if (!q || !out || !sel_idx || !sel_count) return fail(HS_ERR_INVALID_ARGUMENT, "q/out/sel_idx/sel_count is NULL");
  if (q_dtype != HS_F32 && q_dtype != HS_BF16) return fail(HS_ERR_INVALID_ARGUMENT, "q dtype must be F32 or BF16");
  if (!aligned16(q)) return fail(HS_ERR_INVALID_ARGUMENT, "q not 16-byte aligned");
  if (!aligned16(out)) return fail(HS_ERR_INVALID_ARGUMENT, "out not 16-byte aligned");
  if (!aligned4(sel_idx) || !aligned4(sel_count))
    return fail(HS_ERR_INVALID_ARGUMENT, "sel_idx/sel_count not 4-byte aligned");
  if ((int64_t)ci.B * p->q_tokens * ci.n_kv > MAX_LISTS)
    return fail(HS_ERR_UNSUPPORTED, "batch * q_tokens * num_kv_heads = %lld selection lists (at most %lld)",
                (long long)ci.B * p->q_tokens * ci.n_kv, (long long)MAX_LISTS);
  if ((int64_t)p->top_k + p->window > 1152 * 64)
    return fail(HS_ERR_UNSUPPORTED, "selection capacity %d too large", p->top_k + p->window);
  SparsePlan pl;
  plan_sparse(kv, p, q_dtype, ci, pl);
  if (noalloc) {
    // the partials go to the static array; one workgroup per list (attn_gather's direct form) needs none
    const size_t need = (pl.gather && pl.max_chunks == 1) ? 0 : pl.total;
    if (need > HS_NOALLOC_SCRATCH_BYTES)
      return fail(HS_ERR_UNSUPPORTED, "these shapes need %zu bytes of scratch, more than the %zu-byte static "
                  "array of hs_sparse_attn_noalloc (use hs_sparse_attn with a workspace)", need,
                  (size_t)HS_NOALLOC_SCRATCH_BYTES);
    hs_status sst = scratch_for_stream((hipStream_t)stream, &workspace);
    if (sst != HS_OK) return sst;
    workspace_bytes = HS_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace && pl.total) return fail(HS_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (workspace_bytes < pl.total && !noalloc)
    return fail(HS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, pl.total);
  if (!aligned16(workspace)) return fail(HS_ERR_INVALID_ARGUMENT, "workspace not 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  hs::AttnArgs a{};
  a.k = kv->k; a.v = kv->v; a.k_scale = kv->k_scale; a.v_scale = kv->v_scale;
  a.row_start = kv->d_row_start; a.seq_len = kv->d_seq_len;
  a.q = q; a.q_f32 = q_dtype == HS_F32;
  a.n_kv = ci.n_kv; a.H = p->num_q_heads; a.G = pl.G; a.n_q = p->q_tokens;
  a.R = pl.G; a.n_lists = pl.n_lists; a.chunk = pl.chunk; a.max_chunks = pl.max_chunks;
  a.scale_log2 = scale_log2(p);
  a.sel_idx = sel_idx; a.sel_count = sel_count; a.sel_cap = pl.cap;
  a.part_acc = (float*)(ws + pl.off_acc); a.part_ml = (float*)(ws + pl.off_ml);
  if (pl.gather) {
    a.direct = pl.max_chunks == 1; a.out = out; a.lse = nullptr; a.lse2 = nullptr;
    hipError_t e = timed("attn_gather", s, [&] { return hs::launch_attn_gather(a, kv_type(kv->dtype), s); });
    if (e != hipSuccess) return hip_fail(e, "sparse attention");
    if (a.direct) return HS_OK;
  }
  hipError_t e = hipSuccess;
  if (!pl.gather) {
    e = timed("attn_partial_gather", s, [&] { return hs::launch_attn_partial(a, kv_type(kv->dtype), pl.ct, pl.nwr, true, s); });
    if (e != hipSuccess) return hip_fail(e, "sparse attention");
  }
  hs::MergeArgs m{};
  m.part_acc = a.part_acc; m.part_ml = a.part_ml; m.seq_len = kv->d_seq_len; m.sel_count = sel_count;
  m.sel_cap = pl.cap;
  m.gather = 1; m.n_kv = ci.n_kv; m.H = a.H; m.G = pl.G; m.n_q = a.n_q; m.R = pl.G; m.n_lists = pl.n_lists;
  m.chunk = pl.chunk; m.max_chunks = pl.max_chunks; m.out = out; m.lse = nullptr; m.lse2 = nullptr;
  if ((e = timed("attn_merge_gather", s, [&] { return hs::launch_attn_merge(m, s); })) != hipSuccess)
    return hip_fail(e, "sparse attention merge");
  return HS_OK;
}

}  // namespace
