// Token-level selection: top-k global tokens + forced recent window (gfx950).
//
// ithome page "小米公开 MiMo-V3 核心架构 HySparse2", recent-window paragraph after
// section "KV Reuse": the most recent 128 tokens are always selected and 1,024
// global tokens are taken from outside that window (same split on the cnyes
// page, section "檢索精確到token").  The order among candidates is the float
// order of the scores with ties going to the lower index; the emitted list is
// the global set in ascending index order, then the window rows, then -1.
//
// Multi-workgroup radix select on the order-preserving uint32 key of each
// score, so that every list is spread over many CUs:
//   sel_zero      clears the per-list histograms and counters (workspace)
//   sel_hist1     per chunk: LDS histogram of the top 11 key bits -> global
//   sel_cand      per chunk: finds the boundary bin b1 of the k'-th key, counts
//                 keys above it per chunk, appends the keys inside it to a
//                 candidate buffer and histograms their next 11 bits
//   sel_finalize  per list: resolves the remaining 21 bits on the candidates ->
//                 exact k'-th key T and the number `need` of keys == T taken
//                 (lowest indices first); per-chunk output offsets; window part
//   sel_write     per chunk: index-ordered compaction with block scans, so the
//                 list comes out ascending with no sort
// Counts are integers, so the result does not depend on atomic ordering.

#include <algorithm>

#include "hs_common.hpp"
#include "hs_internal.hpp"

namespace hs {

namespace {

constexpr int CH_NT = 256;                 // threads of the per-chunk kernels
constexpr int FIN_NT = 1024;               // threads of the per-list kernel

struct ListInfo {
  int n;       // candidates L - W'
  int kk;      // global budget k'
  int w;       // window rows W'
};

__device__ __forceinline__ ListInfo list_info(const SelectArgs& a, int list) {
  const int b = list / (a.n_q * a.n_kv);
  const int Lb = a.seq_len[b];
  ListInfo li;
  li.w = min(a.window, Lb);
  li.n = Lb - li.w;
  li.kk = max(0, min(a.top_k, Lb - a.window));
  return li;
}

// per-list workspace words: two 2048-bin histograms, candidate count, T, need,
// then 4 arrays of max_chunks words (keys above the boundary bin, output offset,
// ties before, selected count), then the (key, index) candidate pairs
__device__ __forceinline__ uint32_t* ws_list(const SelectArgs& a, int list) { return a.ws + (size_t)list * a.ws_stride; }
constexpr int W_HIST1 = 0, W_HIST2 = 2048, W_CCOUNT = 4096, W_T = 4097, W_NEED = 4098, W_ZERO = 4100, W_CHUNKS = 4100;

template <int NT>
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* sh, uint32_t& total, bool reverse) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = reverse ? __shfl_down(incl, o) : __shfl_up(incl, o);
    if (reverse ? (lane + o < 64) : (lane >= o)) incl += y;
  }
  if (lane == (reverse ? 0 : 63)) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const uint32_t x = lane < NW ? sh[lane] : 0u;
    uint32_t xi = x;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const uint32_t y = reverse ? __shfl_down(xi, o) : __shfl_up(xi, o);
      if (reverse ? (lane + o < NW) : (lane >= o)) xi += y;
    }
    if (lane < NW) sh[NW + lane] = xi - x;
    if (lane == (reverse ? 0 : NW - 1)) sh[2 * NW] = xi;
  }
  __syncthreads();
  const uint32_t r = sh[NW + wave] + incl - v;
  total = sh[2 * NW];
  __syncthreads();
  return r;
}

// Digit d of a NB-bin histogram with (#keys in bins above d) < rem <= (# in bins >= d);
// rem_out = rem minus the keys above d.  Every thread of the block gets the result.
template <int NT, int NB>
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t rem, uint32_t* sh, uint32_t& digit,
                                           uint32_t& rem_out) {
  constexpr int PER = NB >= NT ? NB / NT : 1;                   // fewer bins than threads: one each
  const int t = threadIdx.x;
  uint32_t h[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    h[i] = t * PER + i < NB ? hist[t * PER + i] : 0u;
    sum += h[i];
  }
  uint32_t tot;
  uint32_t above = block_scan_excl<NT>(sum, sh, tot, true);      // keys in bins of higher threads
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    if (above < rem && rem <= above + h[i]) {
      sh[3 * (NT / 64) + 1] = (uint32_t)(t * PER + i);
      sh[3 * (NT / 64) + 2] = rem - above;
    }
    above += h[i];
  }
  __syncthreads();
  digit = sh[3 * (NT / 64) + 1];
  rem_out = sh[3 * (NT / 64) + 2];
  __syncthreads();
}

}  // namespace

__global__ __launch_bounds__(CH_NT) void sel_zero_kernel(SelectArgs a) {
  uint32_t* w = ws_list(a, blockIdx.x);
  for (int i = threadIdx.x; i < W_ZERO; i += CH_NT) w[i] = 0u;
}

__global__ __launch_bounds__(CH_NT) void sel_hist1_kernel(SelectArgs a) {
  const int list = blockIdx.y;
  const ListInfo li = list_info(a, list);
  if (li.kk == 0 || li.kk >= li.n) return;
  const int c0 = blockIdx.x * a.chunk;
  if (c0 >= li.n) return;
  const int c1 = min(li.n, c0 + a.chunk);
  __shared__ uint32_t hist[2048];
  for (int i = threadIdx.x; i < 2048; i += CH_NT) hist[i] = 0u;
  __syncthreads();
  const float* s = a.scores + (size_t)list * a.s_stride;
  for (int j = c0 + threadIdx.x; j < c1; j += CH_NT) atomicAdd(&hist[f32_key(s[j]) >> 21], 1u);
  __syncthreads();
  uint32_t* g = ws_list(a, list) + W_HIST1;
  for (int i = threadIdx.x; i < 2048; i += CH_NT)
    if (hist[i]) atomicAdd(&g[i], hist[i]);
}

__global__ __launch_bounds__(CH_NT) void sel_cand_kernel(SelectArgs a) {
  constexpr int PER = 16;                                        // scores per thread per batch
  const int list = blockIdx.y;
  const ListInfo li = list_info(a, list);
  if (li.kk == 0 || li.kk >= li.n) return;
  const int c0 = blockIdx.x * a.chunk;
  if (c0 >= li.n) return;
  const int c1 = min(li.n, c0 + a.chunk);
  __shared__ uint32_t sh[3 * (CH_NT / 64) + 3];
  __shared__ uint32_t hist2[2048];
  __shared__ uint32_t s_base;
  const int tid = threadIdx.x;
  const float* s = a.scores + (size_t)list * a.s_stride;
  float v[PER];
  auto load = [&](int j0) {                                      // clamped: in bounds, no branch
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = s[min(j0 + e * CH_NT + tid, c1 - 1)];
  };
  load(c0);                                                      // in flight during find_digit
  uint32_t* w = ws_list(a, list);
  uint32_t b1, rem1;
  find_digit<CH_NT, 2048>(w + W_HIST1, (uint32_t)li.kk, sh, b1, rem1);
  for (int i = tid; i < 2048; i += CH_NT) hist2[i] = 0u;
  __syncthreads();
  uint2* cand = (uint2*)(w + a.cand_off);
  uint32_t gt = 0;
  for (int j0 = c0; j0 < c1; j0 += PER * CH_NT) {
    if (j0 != c0) load(j0);
    uint32_t key[PER], in = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      key[e] = f32_key(v[e]);
      const bool ok = j0 + e * CH_NT + tid < c1;
      const uint32_t d1 = key[e] >> 21;
      gt += (ok && d1 > b1) ? 1u : 0u;
      in |= (ok && d1 == b1 ? 1u : 0u) << e;
    }
    // one reservation in the list's candidate buffer per workgroup and batch
    uint32_t tot;
    uint32_t slot = block_scan_excl<CH_NT>((uint32_t)__builtin_popcount(in), sh, tot, false);
    if (tot == 0u) continue;                                     // uniform over the block
    if (tid == 0) s_base = atomicAdd(&w[W_CCOUNT], tot);
    __syncthreads();
    slot += s_base;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if ((in >> e) & 1u) {
        cand[slot++] = make_uint2(key[e], (uint32_t)(j0 + e * CH_NT + tid));
        atomicAdd(&hist2[(key[e] >> 10) & 0x7FFu], 1u);
      }
  }
  uint32_t tot;
  block_scan_excl<CH_NT>(gt, sh, tot, false);
  if (tid == 0) w[W_CHUNKS + blockIdx.x] = tot;                  // keys above the boundary bin
  __syncthreads();
  for (int i = tid; i < 2048; i += CH_NT)
    if (hist2[i]) atomicAdd(&w[W_HIST2 + i], hist2[i]);
}

__global__ __launch_bounds__(FIN_NT) void sel_finalize_kernel(SelectArgs a) {
  const int list = blockIdx.x;
  const ListInfo li = list_info(a, list);
  int32_t* out = a.sel_idx + (size_t)list * a.cap;
  const int tid = threadIdx.x;
  for (int i = tid; i < li.w; i += FIN_NT) out[li.kk + i] = li.n + i;   // window rows L-W' .. L-1
  for (int i = li.kk + li.w + tid; i < a.cap; i += FIN_NT) out[i] = -1;
  if (tid == 0) a.sel_count[list] = li.kk + li.w;
  if (li.kk == 0 || li.kk >= li.n) return;

  __shared__ uint32_t sh[3 * (FIN_NT / 64) + 3];
  __shared__ uint32_t hist3[1024];
  __shared__ uint32_t gtx[1024], eqc[1024];
  uint32_t* w = ws_list(a, list);
  const uint32_t nc = w[W_CCOUNT];
  const uint2* cand = (const uint2*)(w + a.cand_off);
  constexpr int CPT = 4;                                          // candidates per thread per batch
  uint2 cr[CPT];
  auto cload = [&](uint32_t i0) {                                 // clamped: in bounds, no branch
#pragma unroll
    for (int u = 0; u < CPT; ++u) cr[u] = cand[min(i0 + u * FIN_NT + tid, max(nc, 1u) - 1u)];
  };
  cload(0);                                                       // in flight during the first two digits
  uint32_t b1, rem1, b2, rem2, b3, rem3;
  find_digit<FIN_NT, 2048>(w + W_HIST1, (uint32_t)li.kk, sh, b1, rem1);
  find_digit<FIN_NT, 2048>(w + W_HIST2, rem1, sh, b2, rem2);
  hist3[tid] = 0u;
  gtx[tid] = 0u;
  eqc[tid] = 0u;
  __syncthreads();
  for (uint32_t i0 = 0; i0 < nc; i0 += CPT * FIN_NT) {
    if (i0) cload(i0);
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      if (i0 + u * FIN_NT + tid < nc && ((cr[u].x >> 10) & 0x7FFu) == b2) atomicAdd(&hist3[cr[u].x & 0x3FFu], 1u);
  }
  __syncthreads();
  find_digit<FIN_NT, 1024>(hist3, rem2, sh, b3, rem3);
  const uint32_t T = (b1 << 21) | (b2 << 10) | b3;
  const uint32_t need = rem3;                                     // keys == T taken, lowest index first
  for (uint32_t i0 = 0; i0 < nc; i0 += CPT * FIN_NT) {
    if (nc > CPT * FIN_NT) cload(i0);                             // else the registers hold them all
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      if (i0 + u * FIN_NT + tid >= nc) continue;
      const int ch = (int)(cr[u].y / (uint32_t)a.chunk);
      if (cr[u].x > T) atomicAdd(&gtx[ch], 1u);
      else if (cr[u].x == T) atomicAdd(&eqc[ch], 1u);
    }
  }
  __syncthreads();
  // per-chunk prefix: ties before the chunk, then the output offset of the chunk
  const int nch = (li.n + a.chunk - 1) / a.chunk;
  const uint32_t my_eq = tid < nch ? eqc[tid] : 0u;
  uint32_t tot;
  const uint32_t tb = block_scan_excl<FIN_NT>(my_eq, sh, tot, false);
  const uint32_t take = tb >= need ? 0u : min(need - tb, my_eq);
  const uint32_t my_sel = tid < nch ? w[W_CHUNKS + tid] + gtx[tid] + take : 0u;
  const uint32_t off = block_scan_excl<FIN_NT>(my_sel, sh, tot, false);
  if (tid < nch) {
    w[W_CHUNKS + a.max_chunks + tid] = off;                       // output offset of the chunk
    w[W_CHUNKS + 2 * a.max_chunks + tid] = tb;                    // ties in earlier chunks
    w[W_CHUNKS + 3 * a.max_chunks + tid] = my_sel;                // selected in the chunk
  }
  if (tid == 0) {
    w[W_T] = T;
    w[W_NEED] = need;
  }
}

__global__ __launch_bounds__(CH_NT) void sel_write_kernel(SelectArgs a) {
  constexpr int E = 16;                                          // consecutive elements per thread
  const int list = blockIdx.y;
  const ListInfo li = list_info(a, list);
  const int c0 = blockIdx.x * a.chunk;
  if (li.kk == 0 || c0 >= li.n) return;
  const int c1 = min(li.n, c0 + a.chunk);
  int32_t* out = a.sel_idx + (size_t)list * a.cap;
  if (li.kk >= li.n) {                                           // every candidate selected
    for (int j = c0 + threadIdx.x; j < c1; j += CH_NT) out[j] = j;
    return;
  }
  const float* s = a.scores + (size_t)list * a.s_stride;
  float v[E];
  auto load = [&](int p0) {                                      // coalesced, clamped, all in flight
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = s[min(p0 + e * CH_NT + (int)threadIdx.x, c1 - 1)];
  };
  load(c0);                                                      // before the workspace reads
  const uint32_t* w = ws_list(a, list);
  const int ch = blockIdx.x;
  const uint32_t nsel = w[W_CHUNKS + 3 * a.max_chunks + ch];
  if (nsel == 0u) return;
  const uint32_t T = w[W_T], need = w[W_NEED];
  uint32_t pos_base = w[W_CHUNKS + a.max_chunks + ch];
  uint32_t ties = w[W_CHUNKS + 2 * a.max_chunks + ch];
  __shared__ float stage[E * CH_NT];
  __shared__ uint32_t sh[3 * (CH_NT / 64) + 3];
  for (int p0 = c0; p0 < c1; p0 += E * CH_NT) {
    const int pn = min(E * CH_NT, c1 - p0);
    if (p0 != c0) {
      __syncthreads();                                           // previous batch read from stage
      load(p0);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) stage[e * CH_NT + threadIdx.x] = v[e];
    __syncthreads();
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = threadIdx.x * E + e;
      if (i < pn) {
        const uint32_t key = f32_key(stage[i]);
        gt |= (key > T ? 1u : 0u) << e;
        eq |= (key == T ? 1u : 0u) << e;
      }
    }
    uint32_t tot_eq, tot_sel;
    uint32_t r = ties + block_scan_excl<CH_NT>(__builtin_popcount(eq), sh, tot_eq, false);
    uint32_t sel = gt;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((eq >> e) & 1u) {
        if (r < need) sel |= 1u << e;
        ++r;
      }
    uint32_t pos = pos_base + block_scan_excl<CH_NT>(__builtin_popcount(sel), sh, tot_sel, false);
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((sel >> e) & 1u) {
        if (pos < (uint32_t)li.kk) out[pos] = p0 + threadIdx.x * E + e;
        ++pos;
      }
    pos_base += tot_sel;
    ties += tot_eq;
  }
}

// ---------------------------------------------------------------- candidate mode
//
// The score pass appended, per list, the (key, index) pairs of every score whose first digit could
// still reach the k'-th key (all pairs of the boundary digit and above, in no particular order; each
// score workgroup fills its own region of the list's buffer and records its count) and built the
// full first-digit histogram.  Its scores are >= +0, so every key has bit 31 set and the
// digits are bits 30..20, 19..9 and 8..0.  One workgroup per list:
//   * first digit from the histogram; the second and third digits from the candidates in the
//     boundary bin -> the exact k'-th key T and the number `need` of keys equal to T taken;
//   * the selected positions are set in an LDS bitmap over the list's candidates (ties to T: a
//     first bitmap of the tied positions gives the position of the need-th one, so the lowest
//     indices win);
//   * the bitmap read in order yields the ascending index list without a sort.
constexpr int CAND_MAX_WORDS = SELECT_CAND_MAX_N / 32;    // bitmap words in LDS (128 KB)

__global__ __launch_bounds__(FIN_NT) void sel_cand_select_kernel(SelectArgs a) {
  const int list = blockIdx.x;
  const ListInfo li = list_info(a, list);
  int32_t* out = a.sel_idx + (size_t)list * a.cap;
  const int tid = threadIdx.x;
  for (int i = tid; i < li.w; i += FIN_NT) out[li.kk + i] = li.n + i;   // window rows L-W' .. L-1
  for (int i = li.kk + li.w + tid; i < a.cap; i += FIN_NT) out[i] = -1;
  if (tid == 0) a.sel_count[list] = li.kk + li.w;
  if (li.kk == 0) return;
  if (li.kk >= li.n) {                                            // every candidate selected
    for (int j = tid; j < li.n; j += FIN_NT) out[j] = j;
    return;
  }
  __shared__ uint32_t sh[3 * (FIN_NT / 64) + 3];
  __shared__ uint32_t hist2[2048];
  __shared__ uint32_t bits[CAND_MAX_WORDS];
  __shared__ uint32_t s_cut;
  __shared__ uint32_t rcnt[256];                                  // pairs in each region
  __shared__ uint32_t s_maxc;
  const uint32_t* w = ws_list(a, list);
  const uint2* cand = (const uint2*)(w + a.cand_off);
  const int nreg = (int)min(max(w[SELECT_NREG_WORD], 1u), 256u);  // the list's regions, from the score pass
  // the first-digit histogram is loaded first (it does not depend on the region counts) and searched
  // in LDS, so neither the counts nor the search wait for it
  uint32_t h1[2048 / FIN_NT];
#pragma unroll
  for (int i = 0; i < 2048 / FIN_NT; ++i) h1[i] = w[W_HIST1 + i * FIN_NT + tid];
  if (tid == 0) s_maxc = 1u;
  __syncthreads();
  if (tid < nreg) {
    const uint32_t c = w[SELECT_RCOUNT_WORD + tid];
    rcnt[tid] = c;
    atomicMax(&s_maxc, c);
  }
  __syncthreads();
  // positions p in [0, nreg * maxc): region p / maxc, slot p % maxc, a pair when the slot is below
  // the region's count; addresses need no search, so the loads of a batch go out together
  const uint32_t maxc = s_maxc, npos = (uint32_t)nreg * maxc;
  const float rmaxc = 1.0f / (float)maxc;
  // Positions in batches of CPT per thread.  Batches 0 and 1 are loaded once and stay in registers
  // for every pass (lists of up to 2 * BATCH positions never reload); longer lists reload their
  // later batches in every pass, issuing them before the pass works through batch 0.
  constexpr int CPT = 16;                                         // positions per thread per batch
  constexpr uint32_t BATCH = CPT * FIN_NT;
  auto cload = [&](uint2 (&cr)[CPT], uint32_t& cv, uint32_t i0) {  // clamped: in bounds, no branch
    cv = 0u;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const uint32_t p = i0 + u * FIN_NT + tid, pc = min(p, npos - 1u);
      uint32_t r = (uint32_t)((float)pc * rmaxc);                // pc < 2^24: off by at most one
      r -= r * maxc > pc ? 1u : 0u;
      r += (r + 1u) * maxc <= pc ? 1u : 0u;
      const uint32_t j = pc - r * maxc;
      cr[u] = cand[(size_t)r * a.cand_region + j];
      cv |= (p < npos && j < rcnt[r] ? 1u : 0u) << u;
    }
  };
  uint2 c0[CPT], c1[CPT];
  uint32_t v0 = 0u, v1 = 0u;
  const bool resident = npos <= 2 * BATCH;
  auto for_cand = [&](auto&& f) {                                 // f(key, index) over all candidates
    if (!resident) cload(c1, v1, BATCH);
#pragma unroll
    for (int u = 0; u < CPT; ++u)
      if ((v0 >> u) & 1u) f(c0[u].x, c0[u].y);
    for (uint32_t i0 = BATCH; i0 < npos; i0 += BATCH) {
      if (i0 > BATCH) cload(c1, v1, i0);
#pragma unroll
      for (int u = 0; u < CPT; ++u)
        if ((v1 >> u) & 1u) f(c1[u].x, c1[u].y);
    }
  };
  cload(c0, v0, 0);                                               // in flight during the first digit
  if (resident && npos > BATCH) cload(c1, v1, BATCH);
#pragma unroll
  for (int i = 0; i < 2048 / FIN_NT; ++i) hist2[i * FIN_NT + tid] = h1[i];
  __syncthreads();
  uint32_t b1, rem1, b2, rem2, b3, rem3;
  find_digit<FIN_NT, 2048>(hist2, (uint32_t)li.kk, sh, b1, rem1);   // (ends with a barrier)
  for (int i = tid; i < 2048; i += FIN_NT) hist2[i] = 0u;
  __syncthreads();
  for_cand([&](uint32_t key, uint32_t) {
    if (((key >> 20) & 0x7FFu) == b1) atomicAdd(&hist2[(key >> 9) & 0x7FFu], 1u);
  });
  __syncthreads();
  find_digit<FIN_NT, 2048>(hist2, rem1, sh, b2, rem2);
  for (int i = tid; i < 512; i += FIN_NT) hist2[i] = 0u;          // third digit: 9 bits
  __syncthreads();
  const uint32_t hi = 0x400000u | (b1 << 11) | b2;                // key bits 31..9
  for_cand([&](uint32_t key, uint32_t) {
    if ((key >> 9) == hi) atomicAdd(&hist2[key & 0x1FFu], 1u);
  });
  __syncthreads();
  find_digit<FIN_NT, 512>(hist2, rem2, sh, b3, rem3);
  const uint32_t T = (hi << 9) | b3;
  const uint32_t need = rem3;                                     // keys == T taken, lowest index first
  const uint32_t ties = hist2[b3];
  const int nw = (li.n + 31) / 32;
  const int wpt = (nw + FIN_NT - 1) / FIN_NT;                     // bitmap words per thread (contiguous)
  uint32_t cut = 0xFFFFFFFFu;                                     // ties with index <= cut are taken
  if (need < ties) {
    for (int i = tid; i < nw; i += FIN_NT) bits[i] = 0u;
    __syncthreads();
    for_cand([&](uint32_t key, uint32_t j) {
      if (key == T) atomicOr(&bits[j >> 5], 1u << (j & 31));
    });
    __syncthreads();
    uint32_t cnt = 0;
    for (int i = 0; i < wpt; ++i) {
      const int wi = tid * wpt + i;
      if (wi < nw) cnt += __builtin_popcount(bits[wi]);
    }
    uint32_t tot;
    uint32_t before = block_scan_excl<FIN_NT>(cnt, sh, tot, false);
    if (before < need && need <= before + cnt) {                  // this thread holds the need-th tie
      for (int i = 0; i < wpt; ++i) {
        const int wi = tid * wpt + i;
        uint32_t x = wi < nw ? bits[wi] : 0u;
        const uint32_t c = __builtin_popcount(x);
        if (before + c >= need) {
          for (uint32_t r = need - before; r > 1; --r) x &= x - 1u;   // drop the lower set bits
          s_cut = (uint32_t)wi * 32u + (uint32_t)__builtin_ctz(x);
          break;
        }
        before += c;
      }
    }
    __syncthreads();
    cut = s_cut;
  }
  for (int i = tid; i < nw; i += FIN_NT) bits[i] = 0u;
  __syncthreads();
  for_cand([&](uint32_t key, uint32_t j) {
    if (key > T || (key == T && j <= cut)) atomicOr(&bits[j >> 5], 1u << (j & 31));
  });
  __syncthreads();
  uint32_t cnt = 0;
  for (int i = 0; i < wpt; ++i) {
    const int wi = tid * wpt + i;
    if (wi < nw) cnt += __builtin_popcount(bits[wi]);
  }
  uint32_t tot;
  uint32_t pos = block_scan_excl<FIN_NT>(cnt, sh, tot, false);
  for (int i = 0; i < wpt; ++i) {
    const int wi = tid * wpt + i;
    uint32_t x = wi < nw ? bits[wi] : 0u;
    while (x) {
      const int bit = __builtin_ctz(x);
      if (pos < (uint32_t)li.kk) out[pos] = wi * 32 + bit;
      ++pos;
      x &= x - 1u;
    }
  }
}

// ---------------------------------------------------------------- block-level variant (HySparse v1)
//
// dpshk page, section 03: the previous generation chose history in 64-token blocks.  Block b
// covers candidates [64 b, min(64 b + 64, n)); its score is the sum of its tokens' scores, added
// as a balanced pairwise tree in index order in float32 (a wave butterfly); the budget k' buys
// floor(k' / 64) whole blocks (score descending, ties to the lower block) unless k' >= n, when
// every candidate is taken.  Block scores live in the candidate area of the list's workspace.

constexpr int BLK = 64;
constexpr int MAX_BLOCKS = 32768;              // block keys of one list held in LDS

__global__ __launch_bounds__(256) void sel_block_pool_kernel(SelectArgs a) {
  const int list = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int blk = blockIdx.x * 4 + (threadIdx.x >> 6);
  const ListInfo li = list_info(a, list);
  if (li.kk == 0 || li.kk >= li.n) return;                       // nothing to rank
  if (blk >= (li.n + BLK - 1) / BLK) return;
  const int j = blk * BLK + lane;
  float v = j < li.n ? a.scores[(size_t)list * a.s_stride + j] : 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);       // same tree on every lane
  if (lane == 0) ws_list(a, list)[a.cand_off + blk] = f32_key(v);
}

__global__ __launch_bounds__(FIN_NT) void sel_block_select_kernel(SelectArgs a) {
  __shared__ uint32_t key[MAX_BLOCKS];
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t sh[3 * (FIN_NT / 64) + 3];
  __shared__ int s_last_taken;
  const int list = blockIdx.x;
  const ListInfo li = list_info(a, list);
  int32_t* out = a.sel_idx + (size_t)list * a.cap;
  const int tid = threadIdx.x;
  if (tid == 0) s_last_taken = 0;
  int g = 0;                                                      // global tokens emitted
  if (li.kk >= li.n) {
    for (int i = tid; i < li.n; i += FIN_NT) out[i] = i;
    g = li.n;
  } else if (li.kk / BLK > 0) {
    const int nb = (li.n + BLK - 1) / BLK, kb = li.kk / BLK;
    const uint32_t* wk = ws_list(a, list) + a.cand_off;
    for (int b = tid; b < nb; b += FIN_NT) key[b] = wk[b];
    // exact kb-th largest key T over three digits (11, 11, 10 bits), and `need` keys == T taken
    uint32_t prefix = 0, rem = (uint32_t)kb;
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
      const uint32_t bins = pass == 2 ? 1024u : 2048u;
      const uint32_t hmask = pass == 0 ? 0u : pass == 1 ? 0xFFE00000u : 0xFFFFFC00u;
      for (int i = tid; i < 2048; i += FIN_NT) hist[i] = 0u;
      __syncthreads();
      for (int b = tid; b < nb; b += FIN_NT)
        if ((key[b] & hmask) == prefix) atomicAdd(&hist[(key[b] >> shift) & (bins - 1)], 1u);
      __syncthreads();
      uint32_t d;
      if (pass == 2) find_digit<FIN_NT, 1024>(hist, rem, sh, d, rem);
      else find_digit<FIN_NT, 2048>(hist, rem, sh, d, rem);
      prefix |= d << shift;
    }
    const uint32_t T = prefix, need = rem;
    // contiguous blocks per thread, so scans follow block order
    const int per = (nb + FIN_NT - 1) / FIN_NT;
    const int b0 = min(nb, tid * per), b1 = min(nb, b0 + per);
    uint32_t ties = 0;
    for (int b = b0; b < b1; ++b) ties += key[b] == T;
    uint32_t tot;
    uint32_t tie_rank = block_scan_excl<FIN_NT>(ties, sh, tot, false);
    uint32_t mine = 0;
    for (int b = b0; b < b1; ++b) {
      const uint32_t k = key[b];
      if (k > T) ++mine;
      else if (k == T) mine += tie_rank++ < need;
    }
    uint32_t nsel;
    uint32_t slot = block_scan_excl<FIN_NT>(mine, sh, nsel, false);
    tie_rank -= ties;                                             // back to this thread's first tie
    for (int b = b0; b < b1; ++b) {
      const uint32_t k = key[b];
      bool take = k > T;
      if (k == T) take = tie_rank++ < need;
      if (!take) continue;
      const int j1 = min(b * BLK + BLK, li.n);
      for (int j = b * BLK; j < j1; ++j) out[slot * BLK + (j - b * BLK)] = j;
      ++slot;
      if (b == nb - 1) s_last_taken = 1;
    }
    __syncthreads();
    // only the last block can be partial, and it is the last one emitted when chosen
    g = (int)nsel * BLK - (s_last_taken ? nb * BLK - li.n : 0);
  }
  __syncthreads();
  for (int i = tid; i < li.w; i += FIN_NT) out[g + i] = li.n + i;   // window rows L-W' .. L-1
  for (int i = g + li.w + tid; i < a.cap; i += FIN_NT) out[i] = -1;
  if (tid == 0) a.sel_count[list] = g + li.w;
}

hipError_t launch_select_blocks(const SelectArgs& a, int n_lists, int64_t max_cand, hipStream_t st) {
  const int nb_max = (int)((max_cand + BLK - 1) / BLK);
  if (nb_max > 0) hipLaunchKernelGGL(sel_block_pool_kernel, dim3((nb_max + 3) / 4, n_lists), dim3(256), 0, st, a);
  hipLaunchKernelGGL(sel_block_select_kernel, dim3(n_lists), dim3(FIN_NT), 0, st, a);
  return hipGetLastError();
}

int64_t select_blocks_max_candidates() { return (int64_t)MAX_BLOCKS * BLK; }

hipError_t launch_select_cand(const SelectArgs& a, int n_lists, hipStream_t st) {
  hipLaunchKernelGGL(sel_cand_select_kernel, dim3(n_lists), dim3(FIN_NT), 0, st, a);
  return hipGetLastError();
}

static_assert(W_ZERO == SELECT_ZERO_WORDS, "cleared words of the selection workspace");
static_assert(W_CCOUNT == SELECT_CCOUNT_WORD, "candidate count word of the selection workspace");

hipError_t launch_select(const SelectArgs& a, int n_lists, bool fused_prefix, hipStream_t st) {
  const dim3 g(a.max_chunks, n_lists);
  if (!fused_prefix) {
    hipLaunchKernelGGL(sel_zero_kernel, dim3(n_lists), dim3(CH_NT), 0, st, a);
    hipLaunchKernelGGL(sel_hist1_kernel, g, dim3(CH_NT), 0, st, a);
  }
  hipLaunchKernelGGL(sel_cand_kernel, g, dim3(CH_NT), 0, st, a);
  hipLaunchKernelGGL(sel_finalize_kernel, dim3(n_lists), dim3(FIN_NT), 0, st, a);
  hipLaunchKernelGGL(sel_write_kernel, g, dim3(CH_NT), 0, st, a);
  return hipGetLastError();
}

// Chunking and workspace layout of the selection, shared with the host planner.
void select_plan(int64_t s_stride, SelectPlan& p, int64_t cand_pairs) {
  p.chunk = 4096;
  while ((s_stride + p.chunk - 1) / p.chunk > 1024) p.chunk *= 2;  // finalize handles <= 1024 chunks
  p.max_chunks = (int)std::max<int64_t>(1, (s_stride + p.chunk - 1) / p.chunk);
  p.cand_off = (W_CHUNKS + 4 * (int64_t)p.max_chunks + 1) & ~(int64_t)1;   // 8-byte aligned pairs
  p.ws_stride = p.cand_off + 2 * std::max<int64_t>(std::max<int64_t>(s_stride, cand_pairs), 1);
}

}  // namespace hs
