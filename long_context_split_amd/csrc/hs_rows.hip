// Full-attention pass 1 for many query rows per KV head (gfx950, bf16 MFMA; for E4M3 caches an
// opt-in form takes Q K^T on FP8 MFMA, see QK8 below).
//
// ithome page "小米公开 MiMo-V3 核心架构 HySparse2", section "KV Reuse": the full
// layer attends over every cached row of the sequence; with several query
// tokens per step and many heads per KV head (R = n_q * G up to 256 rows), one
// K/V row feeds all R rows, so the work per byte is high and the kernel is
// bound by MFMA and exp throughput, not by HBM.
//
// One workgroup = NRG waves; wave w owns query rows 32w .. 32w + 31 (of its z
// block).  The workgroup streams super-tiles of TT tokens: the next super-tile
// is prefetched into registers (clamped addresses, no branch around a load)
// while the current one is computed from LDS, where K is stored [token][d]
// and V transposed, [d][token], both bf16 (E4M3 codes convert exactly).  The
// transposed V makes every MFMA operand a 16-byte LDS read:
//   S^T[32 tok x 32 rows] = K Q^T           (A = K rows, B = Q rows)
//   online softmax per row in log2 units
//   O^T[128 d x 32 rows] += V^T P^T         (A = V^T rows, B = P; bf16 caches
//                                            split P into bf16 hi + lo)
// Within each 16-token group the V^T columns are stored in the order the P
// operand holds its tokens (bits 2 and 3 of the token index swapped), so a
// lane's 8 k-values are contiguous.  Each thread loads the same 16-byte piece of
// two adjacent tokens, so V^T is written as 32-bit words (one per row: both
// tokens' values); the 16-byte columns of every 16-row block of V^T are XOR-
// swizzled by the block index, which keeps both the transposing writes and the
// operand reads free of LDS bank conflicts (row pitch 272 bytes).
//
// Output: one (m, l, acc) partial per (list, chunk, row), combined by
// attn_merge (or by the score kernel), exactly as the other pass-1 kernels.

#include <type_traits>

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

namespace {

typedef int v8i32 __attribute__((ext_vector_type(8)));

// position of token o (0..15) inside its 16-token group of the V^T tile
__device__ __forceinline__ int vt_col(int tok) {
  const int o = tok & 15;
  return (tok & ~15) | (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1);
}

// byte offset of the 16-byte column quad q of V^T row d: XOR swizzle per 16-row block, kept inside
// the row's NQ quads (NQ a power of two)
template <int NQ>
__device__ __forceinline__ int vt_quad(int d, int q) { return (q ^ ((2 * (d >> 4)) & (NQ - 1))) * 16; }

}  // namespace

// QK8 (E4M3 caches only): S^T = K Q^T on FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, unit block
// scales): K stays as its E4M3 codes in LDS, Q is quantised to E4M3 per query row (scale = the row's
// amax / 448, round to nearest even) and both scales multiply the raw products inside exp2's fma.
// The V side, the softmax and the outputs are as in the bf16 form.
template <int KVT, int NRG, bool QK8>
__global__ __launch_bounds__(64 * NRG) void attn_rows_kernel(AttnArgs a) {
  static_assert(!QK8 || KVT == KV_FP8, "FP8 products need an E4M3 cache");
  constexpr int NT = 64 * NRG;
  constexpr int TT = NRG >= 4 ? 128 : 64;                        // tokens per super-tile
  constexpr int NSUB = TT / 32;
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr bool SPLIT = !FP8;                                   // bf16 cache: P as bf16 hi + lo
  constexpr int SB = (FP8 ? 1 : 2) * D;                          // storage bytes per row
  constexpr int PPR = SB / 16;                                   // 16-byte pieces per row
  constexpr int EPP = FP8 ? 16 : 8;                              // elements per piece
  constexpr int PPT = TT * PPR / NT;                             // pieces per thread per tensor
  static_assert(TT * PPR % NT == 0, "super-tile pieces split evenly over the threads");
  constexpr int KROW = QK8 ? 144 : 272;                         // K tile: 128 codes or 256 B of bf16, + 16 pad
  constexpr int VROW = TT * 2 + 16;                              // V^T tile row: TT tokens + 16 pad
  __shared__ __align__(16) char kt[TT * KROW];
  __shared__ __align__(16) char vt[D * VROW];
  __shared__ float ksc[FP8 ? TT : 1], vsc[FP8 ? TT : 1];
  __shared__ float fmm[FP8 ? TT / 64 : 1][2];                    // per wave of the store: max, min logit factor

  zero_words_grid(a.zero_ptr, a.zero_stride, a.zero_words, a.zero_lists);   // the selection's histograms
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int list = blockIdx.y, chunk = blockIdx.x;
  const int g = list % a.n_kv, b = list / a.n_kv;
  const int Lb = a.seq_len[b];
  const int c0 = chunk * a.chunk;
  if (c0 >= Lb) return;                                           // no work: the merge skips it
  const int c1 = min(Lb, c0 + a.chunk);
  const int64_t rs = a.row_start[b];
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SB;
  const char* vbase = (const char*)a.v + ((size_t)rs * a.n_kv + g) * SB;
  const size_t rstride = (size_t)a.n_kv * SB;
  const int last = c0 + ((c1 - 1 - c0) / TT) * TT;               // first token of the last super-tile

  // ---- prefetch (registers): clamped rows, so every load is in bounds and unconditional
  u32x4 rk[PPT], rv[PPT];
  float sk = 0.f, sv = 0.f;
  // pair j of this thread: tokens 2m, 2m + 1 (m = q / PPR), piece c = q % PPR, q = tid + j * NT
  auto prefetch = [&](int base) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int q = tid + (i >> 1) * NT;
      const int tok = 2 * (q / PPR) + (i & 1);
      const size_t off = (size_t)min(base + tok, c1 - 1) * rstride + (q % PPR) * 16;
      rk[i] = load_stream(kbase + off);
      rv[i] = load_stream(vbase + off);
    }
    if (FP8 && tid < TT) {
      const size_t r = ((size_t)rs + min(base + tid, c1 - 1)) * a.n_kv + g;
      sk = a.k_scale[r];
      sv = a.v_scale[r];
    }
  };
  prefetch(c0);

  // ---- this wave's 32 query rows (row r = t * G + hh), bf16 B operand
  const int row = blockIdx.z * 32 * NRG + 32 * wave + (lane & 31);
  const bool row_ok = row < a.R;
  Mma<CT_BF16>::QOp q;
  v8i32 q8[2];                                                    // QK8: E4M3 Q operand, k-step kk holds
  float qs = 1.f;                                                 // d = 64 kk + 32 (lane >> 5) + byte
  {
    const int t = row_ok ? row / a.G : 0, hh = row_ok ? row % a.G : 0;
    const size_t qoff = (((size_t)b * a.n_q + t) * a.H + (size_t)g * a.G + hh) * D;
    const void* qrow = a.q_f32 ? (const void*)((const float*)a.q + qoff) : (const void*)((const uint16_t*)a.q + qoff);
    if constexpr (QK8) {
      float x[64];                                                // x[32 kk + j]: d = 64 kk + 32 (lane >> 5) + j
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int d0 = 64 * kk + 32 * (lane >> 5);
        if (a.q_f32) {
#pragma unroll
          for (int j = 0; j < 32; ++j) x[32 * kk + j] = row_ok ? ((const float*)qrow)[d0 + j] : 0.f;
        } else {
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const u32x4 w = row_ok ? *(const u32x4*)((const uint16_t*)qrow + d0 + 8 * h) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[32 * kk + 8 * h + 2 * e] = __uint_as_float(w[e] << 16);
              x[32 * kk + 8 * h + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
          }
        }
      }
      float am = 0.f;
#pragma unroll
      for (int j = 0; j < 64; ++j) am = fmaxf(am, fabsf(x[j]));
      am = fmaxf(am, __shfl_xor(am, 32));                         // the row's other 64 d
      qs = am / 448.0f;
      if (qs == 0.f) qs = 1.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const float* y = x + 32 * kk + 4 * w;
          q8[kk][w] = (int)e4m3x4_hw(y[0] / qs, y[1] / qs, y[2] / qs, y[3] / qs);
        }
    } else {
      Mma<CT_BF16>::load_q(q, qrow, a.q_f32, row_ok, lane);
    }
  }

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[4] = {};
  const float sl2 = a.scale_log2;
  // V^T operand of (row block mt4, k-step u, sub-tile st) for this lane: row d = 32 mt4 + (l & 31),
  // column quad q = 4 st + 2 u + (l >> 5), swizzled as vt_quad does; with b = bit 4 of the lane,
  // q ^ (2 (d >> 4)) = 4 (st ^ (mt4 mod NSUB)) + 2 (u ^ b) + (l >> 5), so the address is one of two
  // per-lane bases plus a constant
  const int vlb = (lane >> 4) & 1;
  const char* const vb0 = vt + (lane & 31) * VROW + 16 * ((lane >> 5) + 2 * vlb);
  const char* const vb1 = vt + (lane & 31) * VROW + 16 * ((lane >> 5) + 2 * (1 - vlb));

  for (int base = c0; base < c1; base += TT) {
    // ---- registers -> LDS: K as [token][d], V transposed as [d][token'] (bf16)
#pragma unroll
    for (int jp = 0; jp < PPT / 2; ++jp) {
      const int q = tid + jp * NT, m2 = 2 * (q / PPR), c = q % PPR;
      uint32_t kw[2][EPP / 2], vw[2][EPP / 2];                    // bf16 pairs (d, d + 1) of each token
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const u32x4 xk = rk[2 * jp + t2], xv = rv[2 * jp + t2];
        if constexpr (FP8) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if (!QK8) e4m3x4_to_bf16x4(xk[w], kw[t2][2 * w], kw[t2][2 * w + 1]);
            e4m3x4_to_bf16x4(xv[w], vw[t2][2 * w], vw[t2][2 * w + 1]);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 4; ++w) { kw[t2][w] = xk[w]; vw[t2][w] = xv[w]; }
        }
        if constexpr (QK8) {
          *(u32x4*)(kt + (m2 + t2) * KROW + c * 16) = xk;           // the row's codes, d order
        } else {
          char* kd = kt + (m2 + t2) * KROW + c * (2 * EPP);
#pragma unroll
          for (int h = 0; h < EPP / 8; ++h)
            *(u32x4*)(kd + 16 * h) = u32x4{kw[t2][4 * h], kw[t2][4 * h + 1], kw[t2][4 * h + 2], kw[t2][4 * h + 3]};
        }
      }
      const int col = vt_col(m2);                                 // even; token m2 + 1 is at col + 1
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const int d = c * EPP + e;
        const uint32_t a0 = vw[0][e >> 1], a1 = vw[1][e >> 1];
        const uint32_t word = (e & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
        *(uint32_t*)(vt + d * VROW + vt_quad<TT / 8>(d, col >> 3) + (col & 7) * 2) = word;
      }
    }
    if (FP8 && tid < TT) {                                        // logit factor: K scale x softmax scale
      const float f = sk * sl2;
      ksc[tid] = f;
      vsc[tid] = sv;
      const float fx = wave_max_dpp(f), fn = -wave_max_dpp(-f);   // the super-tile's extreme factors
      if (lane == 0) { fmm[wave][0] = fx; fmm[wave][1] = fn; }
    }
    __syncthreads();
    prefetch(base < last ? base + TT : c1);                       // past the end: every row clamps to the last one
    float fmax_t = sl2, fmin_t = sl2;
    if (FP8) {
#pragma unroll
      for (int w = 0; w < TT / 64; ++w) { fmax_t = w ? fmaxf(fmax_t, fmm[w][0]) : fmm[w][0]; fmin_t = w ? fminf(fmin_t, fmm[w][1]) : fmm[w][1]; }
    }

    // ---- each wave: its 32 rows against the NSUB 32-token sub-tiles.  Lazy rescaling: a row's
    // running max m moves only when a tile's max exceeds it by more than TAU (log2 units), so most
    // tiles skip rescaling acc; p = 2^(x - m) <= 2^TAU stays well inside fp32 and bf16 range.  The
    // tile max is taken on the raw products s and scaled by the super-tile's largest (smallest, for
    // a negative max) logit factor: an upper bound of the true max, which is all the rescaling needs
    // (m only has to stay at or above the logits, minus TAU; LSE = m + log2(l) is exact for any m),
    // and the logits themselves are formed inside exp2's argument as fma(s, f, -m).
    constexpr float TAU = 8.f;
    auto tile = [&](int st, bool MASK) {
      s16x8 va[4][2];                                               // V^T operands, read ahead of the softmax
#pragma unroll
      for (int mt4 = 0; mt4 < 4; ++mt4)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          va[mt4][u] = *(const s16x8*)((u ? vb1 : vb0) + mt4 * 32 * VROW + 64 * (st ^ (mt4 & (NSUB - 1))));
      f32x16 s = {};
      if constexpr (QK8) {                                          // A: the token's codes d = 64 kk + 32 (lane >> 5) + 0..31
        const char* kb = kt + (32 * st + (lane & 31)) * KROW + (lane >> 5) * 32;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const u32x4 lo = *(const u32x4*)(kb + 64 * kk), hi = *(const u32x4*)(kb + 64 * kk + 16);
          const v8i32 ka = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
          s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, q8[kk], s, 0, 0, 0, 0, 0, 0);
        }
      } else {
        const char* kb = kt + (32 * st + (lane & 31)) * KROW + (lane >> 5) * 16;
#pragma unroll
        for (int k8 = 0; k8 < 8; ++k8) {
          const s16x8 ka = *(const s16x8*)(kb + 32 * k8);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, q.v[k8]),
                                                      s, 0, 0, 0);
        }
      }
      // this lane's tokens crow(lane, 4k4 + i) = 32 st + 8 k4 + 4 (lane >> 5) + i: four runs of 4
      if (MASK) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (base + 32 * st + crow(lane, r) >= c1) s[r] = -INFINITY;
      }
      float smax = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) smax = fmaxf(smax, s[r]);
      smax = xor32_max(smax);
      const float mt = smax * (smax >= 0.f ? fmax_t : fmin_t) * qs; // >= the tile's max logit (log2 units)
      const bool need = mt > m + TAU;                               // same for both lanes of a row
      if (__ballot(need)) {
        const float mn = need ? mt : m;
        const float alpha = exp2f(m - mn);                          // m = -inf (first tile): 0
        lsum *= alpha;
#pragma unroll
        for (int mt4 = 0; mt4 < 4; ++mt4) acc[mt4] *= alpha;
        m = mn;
      }
      float p[16];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int t0 = 32 * st + 8 * k4 + 4 * (lane >> 5);
        f32x4 f = {sl2, sl2, sl2, sl2}, v4 = {1.f, 1.f, 1.f, 1.f};
        if (FP8) {
          f = *(const f32x4*)(ksc + t0);
          v4 = *(const f32x4*)(vsc + t0);
          if (QK8) f *= qs;                                         // the row's Q scale
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * k4 + i;
          p[r] = exp2_fast(fmaf(s[r], f[i], -m));
          lsum += p[r];
          if (FP8) p[r] *= v4[i];                                   // V scale folded into P
        }
      }
      // P operand: k-step u, element j <-> p[8u + j] (token crow(lane, 8u + j))
      u32x4 ph[2], pl[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float a0 = p[8 * u + 2 * w], a1 = p[8 * u + 2 * w + 1];
          const uint32_t hw = pack_bf16x2(a0, a1);
          ph[u][w] = hw;
          if (SPLIT) pl[u][w] = pack_bf16x2(a0 - __uint_as_float(hw << 16), a1 - __uint_as_float(hw & 0xFFFF0000u));
        }
#pragma unroll
      for (int mt4 = 0; mt4 < 4; ++mt4) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          acc[mt4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[mt4][u]),
                                                             __builtin_bit_cast(bf16x8, ph[u]), acc[mt4], 0, 0, 0);
          if (SPLIT)
            acc[mt4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va[mt4][u]),
                                                               __builtin_bit_cast(bf16x8, pl[u]), acc[mt4], 0, 0, 0);
        }
      }
    };
    // one loop (a separate loop for the masked last super-tile kept a second copy of acc); only a
    // sub-tile that reaches past c1 masks
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
      if (base + 32 * st >= c1) break;
      tile(st, base + 32 * st + 32 > c1);
    }
    __syncthreads();
  }

  // ---- one partial per row: acc (unnormalised, d-major in the C layout) and (m, l)
  lsum = xor32_add(lsum);
  if (row_ok) {
    const size_t item = (size_t)list * a.max_chunks + chunk;
    float* pa = a.part_acc + (item * a.R + row) * D;
#pragma unroll
    for (int mt4 = 0; mt4 < 4; ++mt4)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 o = {acc[mt4][4 * r4], acc[mt4][4 * r4 + 1], acc[mt4][4 * r4 + 2], acc[mt4][4 * r4 + 3]};
        *(f32x4*)(pa + 32 * mt4 + crow(lane, 4 * r4)) = o;
      }
    if (lane < 32) *(float2*)(a.part_ml + (item * a.R + row) * 2) = make_float2(m, lsum);
  }
}

// Selection scores for many query rows per KV head (G >= 16): s[t][j] = sum over the G heads of query
// token t of 2^(l2 - LSE2), for the candidates j < L_b - W' (ithome page, section "KV Reuse",
// and the recent-window paragraph after it).  Same super-tile streaming as attn_rows (K only);
// S = Q K^T per wave (lane = token, 16 of the wave's rows per lane); the per-token sums of the
// waves are combined through LDS in a fixed order.  Optionally also builds the first-digit
// (11-bit) histogram of each list's score keys for the selection (NQT query tokens per workgroup
// at most; the host passes no histogram otherwise).
template <int KVT, int NRG, int NQT>
__global__ __launch_bounds__(64 * NRG) void attn_rows_scores_kernel(ScoreArgs a) {
  constexpr int NT = 64 * NRG;
  constexpr int TT = NRG >= 4 ? 128 : 64;
  constexpr int NSUB = TT / 32;
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr int SB = (FP8 ? 1 : 2) * D;
  constexpr int PPR = SB / 16;
  constexpr int EPP = FP8 ? 16 : 8;
  constexpr int PPT = TT * PPR / NT;
  static_assert(TT * PPR % NT == 0, "super-tile pieces split evenly over the threads");
  constexpr int KROW = 272;
  __shared__ __align__(16) char kt[TT * KROW];
  __shared__ float ksc[TT];
  __shared__ float part[NRG][2][TT];                              // per wave: up to 2 query tokens (G >= 16)
  __shared__ uint32_t hist[NQT][2048];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int list = blockIdx.y;
  const int g = list % a.n_kv, b = list / a.n_kv;
  const int Lb = a.seq_len[b];
  const int ncand = Lb - min(a.window, Lb);
  const int c0 = blockIdx.x * a.chunk;
  if (c0 >= ncand) return;
  const int c1 = min(ncand, c0 + a.chunk);
  const int64_t rs = a.row_start[b];
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SB;
  const size_t rstride = (size_t)a.n_kv * SB;
  const int last = c0 + ((c1 - 1 - c0) / TT) * TT;
  const float sl2 = a.scale_log2;

  u32x4 rk[PPT];
  float sk = 0.f;
  auto prefetch = [&](int base) {                                 // clamped rows: no branch, in bounds
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      rk[i] = load_stream(kbase + (size_t)min(base + p / PPR, c1 - 1) * rstride + (p % PPR) * 16);
    }
    if (FP8 && tid < TT) sk = a.k_scale[((size_t)rs + min(base + tid, c1 - 1)) * a.n_kv + g];
  };
  prefetch(c0);

  const bool do_hist = a.hist != nullptr;
  if (do_hist)
    for (int i = tid; i < NQT * 2048; i += NT) hist[i >> 11][i & 2047] = 0u;

  // this wave's 32 rows (A operand) and their LSE (log2); padding rows: +inf -> p = 0
  const int rb = blockIdx.z * 32 * NRG;
  const int row = rb + 32 * wave + (lane & 31);
  Mma<CT_BF16>::QOp q;
  {
    const bool ok = row < a.R;
    const int t = ok ? row / a.G : 0, hh = ok ? row % a.G : 0;
    const size_t qoff = (((size_t)b * a.n_q + t) * a.H + (size_t)g * a.G + hh) * D;
    const void* qrow = a.q_f32 ? (const void*)((const float*)a.q + qoff) : (const void*)((const uint16_t*)a.q + qoff);
    Mma<CT_BF16>::load_q(q, qrow, a.q_f32, ok, lane);
  }
  float lse2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rw = rb + 32 * wave + crow(lane, r), rc = min(rw, a.R - 1);
    const float v = a.lse2[((size_t)b * a.n_q + rc / a.G) * a.H + (size_t)g * a.G + rc % a.G];
    lse2[r] = rw < a.R ? v : INFINITY;
  }
  const int tpw = a.G >= 32 ? 1 : 32 / a.G;                       // query tokens per wave
  const int wpt = a.G >= 32 ? a.G / 32 : 1;                       // waves per query token
  const int t_first = rb / a.G;
  const int nt_wg = (min(a.R, rb + 32 * NRG) - rb + a.G - 1) / a.G;   // query tokens of this workgroup
  float* sout = a.scores + (size_t)b * a.n_q * a.n_kv * a.s_stride;

  for (int base = c0; base < c1; base += TT) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {                               // registers -> LDS, [token][d] bf16
      const int p = tid + i * NT, tok = p / PPR, c = p % PPR;
      char* kd = kt + tok * KROW + c * (2 * EPP);
      if constexpr (FP8) {
        uint32_t w8[8];
#pragma unroll
        for (int w = 0; w < 4; ++w) e4m3x4_to_bf16x4(rk[i][w], w8[2 * w], w8[2 * w + 1]);
        *(u32x4*)kd = u32x4{w8[0], w8[1], w8[2], w8[3]};
        *(u32x4*)(kd + 16) = u32x4{w8[4], w8[5], w8[6], w8[7]};
      } else {
        *(u32x4*)kd = rk[i];
      }
    }
    if (tid < TT) ksc[tid] = FP8 ? sk * sl2 : sl2;                // logit factor of the token
    __syncthreads();
    prefetch(base < last ? base + TT : c1);

#pragma unroll 1
    for (int st = 0; st < NSUB; ++st) {
      f32x16 s = {};                                              // S = Q K^T: lane = token (l & 31)
      const char* kb = kt + (32 * st + (lane & 31)) * KROW + (lane >> 5) * 16;
#pragma unroll
      for (int k8 = 0; k8 < 8; ++k8) {
        const s16x8 kb8 = *(const s16x8*)(kb + 32 * k8);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q.v[k8]), __builtin_bit_cast(bf16x8, kb8),
                                                    s, 0, 0, 0);
      }
      const int tk = 32 * st + (lane & 31);
      const float f = ksc[tk];
      float blk[4];                                               // rows 8 q4 + 4 (l >> 5) + 0..3
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) v += exp2_fast(s[4 * q4 + i] * f - lse2[4 * q4 + i]);
        blk[q4] = xor32_add(v);
      }
      if (lane < 32) {
        if (tpw == 1) part[wave][0][tk] = (blk[0] + blk[1]) + (blk[2] + blk[3]);
        else { part[wave][0][tk] = blk[0] + blk[1]; part[wave][1][tk] = blk[2] + blk[3]; }
      }
    }
    __syncthreads();
    // combine the waves of each query token (fixed order), store, histogram
    for (int i = tid; i < nt_wg * TT; i += NT) {
      const int lt = i / TT, tk = i % TT;
      const int pos = base + tk;
      if (pos >= c1) continue;
      float v = 0.f;
      if (tpw == 1) {
        for (int j = 0; j < wpt; ++j) v += part[lt * wpt + j][0][tk];
      } else {
        v = part[lt / tpw][lt % tpw][tk];
      }
      sout[((size_t)(t_first + lt) * a.n_kv + g) * a.s_stride + pos] = v;
      if (do_hist) atomicAdd(&hist[lt][f32_key(v) >> 21], 1u);
    }
    // the next iteration's LDS writes come after its first barrier; part[] is rewritten only after it
  }
  if (!do_hist) return;
  __syncthreads();
  for (int i = tid; i < nt_wg * 2048; i += NT) {
    const uint32_t v = hist[i >> 11][i & 2047];
    if (v) atomicAdd(a.hist + (((size_t)b * a.n_q + t_first + (i >> 11)) * a.n_kv + g) * a.hist_stride + (i & 2047), v);
  }
}

template <int KVT, int NRG>
static hipError_t launch_rows_scores_t(const ScoreArgs& a, hipStream_t st) {
  const int z = (a.R + 32 * NRG - 1) / (32 * NRG);
  dim3 grid(a.max_chunks, a.n_lists, z);
  hipLaunchKernelGGL((attn_rows_scores_kernel<KVT, NRG, 4>), grid, dim3(64 * NRG), 0, st, a);
  return hipGetLastError();
}

template <int KVT, int NRG, bool QK8>
static hipError_t launch_rows_t(const AttnArgs& a, hipStream_t st) {
  const int z = (a.R + 32 * NRG - 1) / (32 * NRG);
  dim3 grid(a.max_chunks, a.n_lists, z);
  hipLaunchKernelGGL((attn_rows_kernel<KVT, NRG, QK8>), grid, dim3(64 * NRG), 0, st, a);
  return hipGetLastError();
}

template <int KVT, bool QK8>
static hipError_t launch_rows_k(const AttnArgs& a, int nrg, hipStream_t st) {
  switch (nrg) {
    case 2: return launch_rows_t<KVT, 2, QK8>(a, st);
    case 4: return launch_rows_t<KVT, 4, QK8>(a, st);
    default: return launch_rows_t<KVT, 8, QK8>(a, st);
  }
}

int rows_groups(int R) { return R <= 64 ? 2 : R <= 128 ? 4 : 8; }

int rows_tile_tokens(int nrg) { return nrg >= 4 ? 128 : 64; }

hipError_t launch_attn_rows_scores(const ScoreArgs& a, int kvt, int nrg, hipStream_t st) {
  if (kvt == KV_BF16) {
    if (nrg == 2) return launch_rows_scores_t<KV_BF16, 2>(a, st);
    if (nrg == 4) return launch_rows_scores_t<KV_BF16, 4>(a, st);
    return launch_rows_scores_t<KV_BF16, 8>(a, st);
  }
  if (kvt == KV_FP8) {
    if (nrg == 2) return launch_rows_scores_t<KV_FP8, 2>(a, st);
    if (nrg == 4) return launch_rows_scores_t<KV_FP8, 4>(a, st);
    return launch_rows_scores_t<KV_FP8, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn_rows(const AttnArgs& a, int kvt, int nrg, hipStream_t st) {
  if (kvt == KV_BF16) return launch_rows_k<KV_BF16, false>(a, nrg, st);
  if (kvt == KV_FP8) return a.qk_fp8 ? launch_rows_k<KV_FP8, true>(a, nrg, st) : launch_rows_k<KV_FP8, false>(a, nrg, st);
  return hipErrorInvalidValue;
}

}  // namespace hs
