// Token-level selection: top-k global tokens + forced recent window (gfx950).
//
// ithome page "小米公开 MiMo-V3 核心架构 HySparse2", recent-window paragraph after
// section "KV Reuse": the most recent 128 tokens are always selected and 1,024
// global tokens are taken from outside that window (same split on the cnyes
// page, section "檢索精確到token").  The order among candidates is the float
// order of the scores with ties going to the lower index; the emitted list is
// the global set in ascending index order, then the window rows, then -1.
//
// One 1024-thread workgroup per list (b, t, g):
//   1. radix select on the order-preserving uint32 key of each float score,
//      three LDS histogram passes (11 + 11 + 10 bits), each restricted to the
//      key prefix fixed so far -> T = exact k'-th largest key and `need` =
//      how many keys equal to T belong to the set;
//   2. compaction in index order: every element with key > T, plus the first
//      `need` elements with key == T; block-wide exclusive scans give each
//      thread its output offset, so the list comes out ascending with no sort.

#include "hs_common.hpp"
#include "hs_internal.hpp"

namespace hs {

constexpr int SEL_NT = 1024;
constexpr int SEL_NW = SEL_NT / 64;

// Block-wide exclusive scan of one uint per thread; also returns the total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < SEL_NW ? wsum[lane] : 0u;
    uint32_t xi = x;
#pragma unroll
    for (int o = 1; o < SEL_NW; o <<= 1) {
      uint32_t y = __shfl_up(xi, o);
      if (lane >= o) xi += y;
    }
    if (lane < SEL_NW) wsum[SEL_NW + lane] = xi - x;       // exclusive prefix of wave totals
    if (lane == SEL_NW - 1) wsum[2 * SEL_NW] = xi;
  }
  __syncthreads();
  const uint32_t r = wsum[SEL_NW + wave] + incl - v;
  total = wsum[2 * SEL_NW];
  __syncthreads();
  return r;
}

// Same, in reverse thread order: returns the sum over threads with a larger index.
__device__ __forceinline__ uint32_t block_excl_scan_rev(uint32_t v, uint32_t* wsum, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;                                           // sum over lanes >= lane
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_down(incl, o);
    if (lane + o < 64) incl += y;
  }
  if (lane == 0) wsum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < SEL_NW ? wsum[lane] : 0u;
    uint32_t xi = x;
#pragma unroll
    for (int o = 1; o < SEL_NW; o <<= 1) {
      uint32_t y = __shfl_down(xi, o);
      if (lane + o < SEL_NW) xi += y;
    }
    if (lane < SEL_NW) wsum[SEL_NW + lane] = xi - x;           // sum over waves above
    if (lane == 0) wsum[2 * SEL_NW] = xi;
  }
  __syncthreads();
  const uint32_t r = wsum[SEL_NW + wave] + incl - v;
  total = wsum[2 * SEL_NW];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(SEL_NT) void select_kernel(SelectArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[2 * SEL_NW + 1];
  __shared__ uint32_t found[2];
  const int tid = threadIdx.x;
  const int list = blockIdx.x;
  const int b = list / (a.n_q * a.n_kv);
  const int Lb = a.seq_len[b];
  const int w = min(a.window, Lb);
  const int n = Lb - w;
  const int kk = max(0, min(a.top_k, Lb - a.window));
  const float* s = a.scores + (size_t)list * a.s_stride;
  int32_t* out = a.sel_idx + (size_t)list * a.cap;

  if (kk >= n) {
    for (int i = tid; i < n; i += SEL_NT) out[i] = i;         // every candidate selected
  } else if (kk > 0) {
    uint32_t prefix = 0u, pmask = 0u, rem = (uint32_t)kk;
    const int shifts[3] = {21, 10, 0};
    const uint32_t dmasks[3] = {0x7FFu, 0x7FFu, 0x3FFu};
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = shifts[pass];
      const uint32_t dm = dmasks[pass];
      hist[2 * tid] = 0u;
      hist[2 * tid + 1] = 0u;
      __syncthreads();
      for (int j = tid; j < n; j += SEL_NT) {
        const uint32_t key = f32_key(s[j]);
        if ((key & pmask) == prefix) atomicAdd(&hist[(key >> sh) & dm], 1u);
      }
      __syncthreads();
      // thread t owns bins 2t, 2t+1; count of keys in bins above them = reverse exclusive scan
      const uint32_t h1 = hist[2 * tid + 1], h0 = hist[2 * tid];
      uint32_t tot;
      const uint32_t above = block_excl_scan_rev(h0 + h1, wsum, tot);
      if (above < rem && rem <= above + h1) {
        found[0] = 2u * tid + 1u;
        found[1] = rem - above;
      } else if (above + h1 < rem && rem <= above + h1 + h0) {
        found[0] = 2u * tid;
        found[1] = rem - above - h1;
      }
      __syncthreads();
      prefix |= found[0] << sh;
      pmask |= dm << sh;
      rem = found[1];
      __syncthreads();
    }
    const uint32_t T = prefix;
    const uint32_t need = rem;                                 // keys == T to take, lowest index first
    uint32_t written = 0u, ties_before = 0u;
    constexpr int E = 4;
    for (int start = 0; start < n && written < (uint32_t)kk; start += SEL_NT * E) {
      const int j0 = start + tid * E;
      uint32_t gt = 0u, eq = 0u;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if (j0 + e < n) {
          const uint32_t key = f32_key(s[j0 + e]);
          gt |= (key > T ? 1u : 0u) << e;
          eq |= (key == T ? 1u : 0u) << e;
        }
      }
      uint32_t tot_eq, tot_sel;
      const uint32_t eq_rank = ties_before + block_excl_scan(__builtin_popcount(eq), wsum, tot_eq);
      uint32_t sel = gt, r = eq_rank;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((eq >> e) & 1u) { if (r < need) sel |= 1u << e; ++r; }
      uint32_t pos = written + block_excl_scan(__builtin_popcount(sel), wsum, tot_sel);
#pragma unroll
      for (int e = 0; e < E; ++e)
        if ((sel >> e) & 1u) { if (pos < (uint32_t)kk) out[pos] = j0 + e; ++pos; }
      written += tot_sel;
      ties_before += tot_eq;
    }
  }
  for (int i = tid; i < w; i += SEL_NT) out[kk + i] = n + i;  // recent window rows L-W' .. L-1
  for (int i = kk + w + tid; i < a.cap; i += SEL_NT) out[i] = -1;
  if (tid == 0) a.sel_count[list] = kk + w;
}

hipError_t launch_select(const SelectArgs& a, int n_lists, hipStream_t st) {
  hipLaunchKernelGGL(select_kernel, dim3(n_lists), dim3(SEL_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs
