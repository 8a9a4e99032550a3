// Score filter of the full layer's selection: exact selection scores for only the tokens that can
// still reach the top k' (ithome page "小米公开 MiMo-V3 核心架构 HySparse2", section "KV Reuse": the
// full layer picks positions from its own attention scores; recent-window paragraphs: k' global
// tokens from outside the recent window).
//
// The score of candidate j is s_j = sum over the rows h of 2^(l_hj - lse2_h) (log2 units).  The
// dense pass (attn_wave) leaves, for every (token, row), a byte c = floor(8 (l_hj - m_h) + 191)
// clamped to [0, 255], with m_h the row's reference in that tile (stored beside the codes).  So
// l_hj - lse2_h lies in [(c - 191) / 8, (c - 190) / 8) + (m_h - lse2_h) for c >= 1 and below
// -190 / 8 + (m_h - lse2_h) for c = 0: each code brackets its term within a factor 2^(1/8).
//
//   filter_bounds  per token: U = an upper bound of the exact score, L = a lower bound; the first
//                  digit of U is kept (2 bytes per token) and L is histogrammed per list.  The
//                  terms are summed as floats built from their bits: the exponent field of 2^e is
//                  (e + 127) 2^23, and (c << 20) adds c / 8 to it, so one integer add per term gives
//                  a float that is at least 2^e (the float between two powers of two is the chord of
//                  2^x, which lies above the curve by at most a factor 1.0615).
//   filter_exact   per list: d = the highest first digit whose lower-bound bins hold k' tokens, so
//                  the k'-th largest score is at least the smallest float of digit d; every token
//                  whose upper bound reaches it is recomputed exactly (its K row gathered, the score
//                  pass's MFMA and tile_scores), and its (key, index) pair goes to the selection.
//
// Every score at or above the k'-th largest is recomputed, so the selection on the pairs equals
// the selection on all scores bit for bit.  Margins: the bounds widen each term by DELTA (log2
// units), far more than the difference between the two passes' float32 logits, the rounding of the
// reference difference and of the code arithmetic; the float sums are widened by 2^-16 relative
// and tiny absolute terms cover results below the normal range.

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

namespace {

constexpr float DELTA = 1.0f / 64.0f;
// lower bound of a code >= 1 relative to its upper-bound float:
// 2^(-1/8 - 2 DELTA - 2^-16) / 1.0615 * (1 - 2^-21) * (1 - 2^-18), rounded down
constexpr float KAPPA = 0.845351994f;

// Highest first digit d (float bits >> 20) whose bins >= d hold kk counts of a 2048-bin histogram
// in global memory; 0 when fewer than kk are counted.  Whole wave.
__device__ int kth_digit(const uint32_t* hist, uint32_t kk, int lane) {
  uint32_t h[32], tot = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    h[i] = hist[32 * lane + i];
    tot += h[i];
  }
  uint32_t suf = tot;                                             // counts in this lane's bins and above
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(suf, o);
    if (lane + o < 64) suf += y;
  }
  const unsigned long long reach = __ballot(suf >= kk);
  if (!reach) return 0;
  const int top = 63 - __clzll((long long)reach);
  uint32_t above = __shfl(suf - tot, top);
  int found = 0;
#pragma unroll
  for (int i = 31; i >= 0; --i) {
    above += h[i];
    found += above < kk ? 1 : 0;
  }
  return 32 * top + 31 - __shfl(found, top);
}

}  // namespace

// ---------------------------------------------------------------- bounds

template <int NW>
__global__ __launch_bounds__(64 * NW) void filter_bounds_kernel(FilterArgs a) {
  __shared__ uint32_t hist[2048];
  __shared__ __align__(16) int sB[NW][8][32];                     // per wave: per tile of its unit, per row
  __shared__ float s_lse2[32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int list, cidx;
  grid_item(a.seq_len, a.n_kv, a.n_lists, a.chunk, a.window, 1, a.uniform_items, blockIdx.x, list, cidx);
  if (list < 0) return;
  const int g = list % a.n_kv, b = list / a.n_kv;
  const int Lb = a.seq_len[b];
  const int ncand = Lb - min(a.window, Lb);
  const int c0 = cidx * a.chunk, c1 = min(ncand, c0 + a.chunk);
  if (a.part_ml) {
    const int nwg = max(1, (ncand + a.chunk - 1) / a.chunk);
    fold_merge<NW>(a.part_acc, a.part_ml, a.dchunk, a.dmax_chunks, a.R, a.G, a.H, 1, b, g, list, Lb, cidx, nwg,
                   s_lse2, a.out, a.lse, a.lse2, wave, lane);
  } else if (tid < 32) {
    s_lse2[tid] = a.lse2[(size_t)b * a.H + (size_t)g * a.G + min(tid, a.R - 1)];
  }
  for (int i = tid; i < 2048; i += 64 * NW) hist[i] = 0u;
  __syncthreads();
  if (c0 < c1) {
    const int t_lo = c0 >> 5, t_hi = (c1 + 31) >> 5;              // c0: a multiple of the chunk granule
    const int tt = lane >> 3, qd = lane & 7;                      // tile of the unit, token quad
    const uint8_t* lrec = a.codes + (size_t)list * a.code_tiles * CODE_TILE_BYTES;
    uint16_t* ud = a.udig + (size_t)list * a.u_stride;
    // code-0 float bits of rows 4 qd .. 4 qd + 3 from their references: ceil((m - lse2 + 127 + DELTA)
    // 2^23) - 190 2^20, at least 0 (rows past R contribute only that junk, which the margins absorb)
    float cb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int h = 4 * qd + e;
      cb[e] = h < a.R ? (127.0f + DELTA) - s_lse2[h] : -INFINITY;
    }
    for (int u = t_lo + 8 * wave; u < t_hi; u += 8 * NW) {
      const bool tile_ok = u + tt < t_hi;
      const int tile = min(u + tt, t_hi - 1);                       // clamped: every load in bounds
      const char* rec = (const char*)lrec + (size_t)tile * CODE_TILE_BYTES;
      u32x4 cw[8];                                                  // word 4 i + e: row 4 i + e, tokens 4 qd ..
#pragma unroll
      for (int i = 0; i < 8; ++i) cw[i] = *(const u32x4*)(rec + qd * 128 + 16 * i);
      const f32x4 rf = *(const f32x4*)(rec + 1024 + 16 * qd);
      int4 bq;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y = fmaf(rf[e] + cb[e], 8388608.0f, -199229440.0f);   // (m - lse2 + 127 + DELTA) 2^23 - 190 2^20
        (&bq.x)[e] = (int)__builtin_ceilf(fmaxf(y, 0.0f));
      }
      wave_sync();                                                  // the previous unit's reads are done
      *(int4*)&sB[wave][tt][4 * qd] = bq;
      wave_sync();
      int B[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int4 v = *(const int4*)&sB[wave][tt][4 * i];
        B[4 * i] = v.x; B[4 * i + 1] = v.y; B[4 * i + 2] = v.z; B[4 * i + 3] = v.w;
      }
      float U[4] = {0.f, 0.f, 0.f, 0.f}, Z = 0.f;
#pragma unroll
      for (int h = 0; h < 32; ++h) {
        const uint32_t w = cw[h >> 2][h & 3];
        Z += __int_as_float(B[h]);
#pragma unroll
        for (int i = 0; i < 4; ++i) U[i] += __int_as_float((int)(((w >> (8 * i)) & 0xFFu) << 20) + B[h]);
      }
      const int pos0 = (u + tt) * 32 + 4 * qd;
      uint32_t dg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float Uu = fmaf(U[i], 1.0f + 0x1p-16f, 0x1p-100f);
        const float Ll = fmaf(KAPPA * (1.0f - 0x1p-18f), U[i] - Z, -(KAPPA * 0x1p-18f * (U[i] + Z) + 0x1p-80f));
        dg[i] = __float_as_uint(Uu) >> 20;
        if (tile_ok && pos0 + i < c1 && Ll > 0.f) atomicAdd(&hist[__float_as_uint(Ll) >> 20], 1u);
      }
      if (tile_ok) *(uint2*)(ud + pos0) = make_uint2(dg[0] | (dg[1] << 16), dg[2] | (dg[3] << 16));
    }
  }
  __syncthreads();
  uint32_t* gh = a.lhist + (size_t)list * 2048;
  for (int i = tid; i < 2048; i += 64 * NW) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(gh + i, v);
  }
}

// ---------------------------------------------------------------- exact scores of the candidates

template <int KVT, int NW>
__global__ __launch_bounds__(64 * NW) void filter_exact_kernel(FilterArgs a) {
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr int ROWB = 272;                                       // as the score pass's K tile
  constexpr int QCAP = 32 + 512;                                  // queue: < 32 left over + one 512-token piece
  __shared__ uint32_t hist[2048];
  __shared__ __align__(16) char qs[32 * ROWB];
  __shared__ __align__(16) char ktile[NW][32 * ROWB];
  __shared__ int queue[NW][QCAP];
  __shared__ float ksc[FP8 ? NW : 1][32];
  __shared__ int s_d;
  __shared__ uint32_t s_cc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int list, slot, nper;
  if (a.cand_uniform) {
    nper = (int)gridDim.x / a.n_lists;
    list = (int)blockIdx.x / nper;
    slot = (int)blockIdx.x % nper;
  } else {                                                        // prefix over the lists
    int acc = 0;
    list = a.n_lists - 1;
    nper = 1;
    for (int l = 0; l < a.n_lists; ++l) {
      const int L = a.seq_len[l / a.n_kv];
      const int np = cand_nper(L - min(a.window, L), a.cand_total);
      if ((int)blockIdx.x < acc + np) { list = l; nper = np; break; }
      acc += np;
    }
    slot = (int)blockIdx.x - acc;
  }
  const int g = list % a.n_kv, b = list / a.n_kv;
  const int Lb = a.seq_len[b];
  const int ncand = Lb - min(a.window, Lb);
  const int kk = max(0, min(a.top_k, Lb - a.window));
  uint32_t* ws = a.sel_ws + (size_t)list * a.sel_stride;
  if (kk == 0 || kk >= ncand) return;                             // the selection needs no pairs
  const int span = (ncand + nper - 1) / nper;
  const int spanr = (span + FILTER_SPAN_ALIGN - 1) / FILTER_SPAN_ALIGN * FILTER_SPAN_ALIGN;
  const int r0 = slot * spanr, r1 = min(ncand, r0 + spanr);
  for (int i = tid; i < 2048; i += 64 * NW) hist[i] = 0u;
  if (wave == 0) {
    const int d = kth_digit(a.lhist + (size_t)list * 2048, (uint32_t)kk, lane);
    if (lane == 0) { s_d = d; s_cc = 0u; }
  }
  for (int p = tid; p < 32 * 16; p += 64 * NW) {                  // Q rows -> LDS (rows >= R: zero)
    const int r = p >> 4, c = p & 15;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < a.R) {
      const size_t qoff = ((size_t)b * a.H + (size_t)g * a.G + r) * D + c * 8;
      if (a.q_f32) {
        const float* qf = (const float*)a.q + qoff;
        for (int j = 0; j < 4; ++j) x[j] = f32_to_bf16_rne(qf[2 * j]) | (f32_to_bf16_rne(qf[2 * j + 1]) << 16);
      } else {
        x = *(const u32x4*)((const uint16_t*)a.q + qoff);
      }
    }
    *(u32x4*)(qs + r * ROWB + c * 16) = x;
  }
  __syncthreads();
  s16x8 qop[8];
#pragma unroll
  for (int st = 0; st < 8; ++st) qop[st] = *(const s16x8*)(qs + (lane & 31) * ROWB + (16 * st + 8 * (lane >> 5)) * 2);
  float lse2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rw = crow(lane, r);
    lse2[r] = rw < a.R ? a.lse2[(size_t)b * a.H + (size_t)g * a.G + rw] : INFINITY;
  }
  const int tpw = a.G >= 32 ? 1 : 32 / a.G;
  const uint32_t d = (uint32_t)s_d;
  const int64_t rs = a.row_start[b];
  constexpr int SB = FP8 ? D : 2 * D;
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SB;
  const size_t rstride = (size_t)a.n_kv * SB;
  uint2* const region = (uint2*)(ws + a.cand_off) + (size_t)slot * a.cand_region;
  const uint16_t* ud = a.udig + (size_t)list * a.u_stride;
  char* const kt = ktile[wave];
  int* const qu = queue[wave];

  // exact scores of the n <= 32 candidates at qu[o ..]: their K rows -> the wave's tile -> S = Q K^T
  auto process = [&](int o, int n) {
    if constexpr (FP8) {                                          // 128-byte rows: 8 pieces of 16 codes
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = (lane >> 3) + 8 * i, c = lane & 7;
        const int j = qu[o + min(tk, n - 1)];
        const u32x4 x = *(const u32x4*)(kbase + (size_t)j * rstride + 16 * c);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4 ov;
#pragma unroll
          for (int ww = 0; ww < 4; ++ww) {
            const uint32_t word = x[2 * h + (ww >> 1)];
            const uint32_t c0b = (word >> (16 * (ww & 1))) & 0xFFu, c1b = (word >> (16 * (ww & 1) + 8)) & 0xFFu;
            ov[ww] = (__float_as_uint(e4m3_to_f32(c0b)) >> 16) | (__float_as_uint(e4m3_to_f32(c1b)) & 0xFFFF0000u);
          }
          *(u32x4*)(kt + tk * ROWB + c * 32 + 16 * h) = ov;
        }
      }
      if (lane < 32) ksc[wave][lane] = a.k_scale[((size_t)rs + qu[o + min(lane, n - 1)]) * a.n_kv + g];
    } else {                                                      // 256-byte rows: 16 pieces
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tk = (lane >> 4) + 4 * i, c = lane & 15;
        const int j = qu[o + min(tk, n - 1)];
        *(u32x4*)(kt + tk * ROWB + c * 16) = *(const u32x4*)(kbase + (size_t)j * rstride + 16 * c);
      }
    }
    wave_sync();
    f32x16 s = {};
    const char* kb = kt + (lane & 31) * ROWB + (lane >> 5) * 16;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const s16x8 kv = *(const s16x8*)(kb + 32 * st);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qop[st]), __builtin_bit_cast(bf16x8, kv), s,
                                                  0, 0, 0);
    }
    const float f = a.scale_log2 * (FP8 ? ksc[wave][lane & 31] : 1.f);
    float tv[1];
    tile_scores<1>(s, f, lse2, tpw, tv);
    const bool keep = lane < n;                                   // lanes 32.. hold the same tokens
    const int j = qu[o + min(lane & 31, n - 1)];
    const uint32_t key = f32_key(tv[0]);
    const unsigned long long mk = __ballot(keep);
    uint32_t base = 0u;
    if (lane == 0) base = atomicAdd(&s_cc, (uint32_t)__popcll(mk));
    base = __shfl(base, 0);
    if (keep) {
      region[base + __popcll(mk & ((1ull << lane) - 1ull))] = make_uint2(key, (uint32_t)j);
      atomicAdd(&hist[(key >> 20) & 0x7FFu], 1u);
    }
    wave_sync();                                                  // tile reads done before its next writes
  };

  int qn = 0;                                                     // candidates waiting in the queue
  for (int p0 = r0 + 512 * wave; p0 < r1; p0 += 512 * NW) {
    // 8 digits per lane: tokens p0 + 8 lane .. + 7 (positions past r1 read the list's own row, ignored)
    const int pl = p0 + 8 * lane;
    const u32x4 dv = *(const u32x4*)(ud + min(pl, (r1 - 1) & ~7));
    uint32_t m8 = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t dg = (dv[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      m8 |= (pl + i < r1 && dg >= d ? 1u : 0u) << i;
    }
    // compaction in token order: exclusive prefix of the per-lane counts
    const uint32_t cnt = __builtin_popcount(m8);
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const int tot = __shfl(incl, 63);
    int w = qn + (int)(incl - cnt);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((m8 >> i) & 1u) qu[w++] = pl + i;
    qn += tot;
    wave_sync();
    int o = 0;
    for (; qn - o >= 32; o += 32) process(o, 32);
    if (o > 0) {                                                  // move the rest (< 32) to the front
      const int rest = qn - o;
      const int v = lane < rest ? qu[o + lane] : 0;
      wave_sync();
      if (lane < rest) qu[lane] = v;
      wave_sync();
      qn = rest;
    }
  }
  if (qn > 0) process(0, qn);
  __syncthreads();
  if (tid == 0) ws[SELECT_RCOUNT_WORD + slot] = s_cc;
  if (tid == 0 && slot == 0) ws[SELECT_NREG_WORD] = (uint32_t)nper;
  for (int i = tid; i < 2048; i += 64 * NW) {
    const uint32_t v = hist[i];
    if (v) atomicAdd(ws + i, v);                                  // the first-digit histogram (cleared before)
  }
}

hipError_t launch_filter_bounds(const FilterArgs& a, hipStream_t st) {
  if (a.R > 32 || a.chunk % FILTER_BOUNDS_CHUNK || a.u_stride % 32) return hipErrorInvalidValue;
  hipLaunchKernelGGL((filter_bounds_kernel<8>), dim3(a.n_items), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_filter_exact(const FilterArgs& a, int kvt, hipStream_t st) {
  if (a.R > 32 || a.n_wg2 < a.n_lists || (a.cand_uniform && a.n_wg2 % a.n_lists) ||
      (!a.cand_uniform && a.cand_total < 0))
    return hipErrorInvalidValue;
  if (kvt == KV_BF16)
    hipLaunchKernelGGL((filter_exact_kernel<KV_BF16, 8>), dim3(a.n_wg2), dim3(512), 0, st, a);
  else if (kvt == KV_FP8)
    hipLaunchKernelGGL((filter_exact_kernel<KV_FP8, 8>), dim3(a.n_wg2), dim3(512), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace hs
