// Attention kernels of the hybrid block (gfx950, wave64, MFMA).
//
//  attn_partial  split-K flash-decoding pass.  Dense mode: the full-attention
//                layer over all L_b cache rows of a sequence.  Gather mode: a
//                sparse layer over the rows its selection list names (ithome
//                page "小米公开 MiMo-V3 核心架构 HySparse2", section "KV Reuse":
//                the sparse layers reuse the full layer's cache and indices).
//  attn_merge    fixed-order merge of the split partials -> O, LSE.
//  attn_scores   second pass of the full layer: per-head softmax probabilities
//                exp(l - LSE) summed over the heads sharing a KV head, for the
//                candidates outside the recent window (ithome page, section
//                "KV Reuse": the full layer selects positions from its attention
//                scores; recent-window paragraph: global tokens come from
//                outside the window).
//
// Data flow of one work item (sequence b, KV head g, chunk of tokens): the
// workgroup streams K/V super-tiles of 32*NWT tokens from HBM with coalesced
// 16-byte loads (prefetched into registers one super-tile ahead), converts them
// to the MFMA input type in LDS, and each wave multiplies its 32 query rows
// against its 32-token sub-tile:
//   S^T[32 tok x 32 rows] = K Q^T     (v_mfma_f32_32x32x16_bf16, or 32x32x2_f32)
//   online softmax per row (log2 domain)
//   O^T[128 d x 32 rows] += V^T P^T   (P split into bf16 hi + lo for bf16 caches)
// Query rows of a KV head are (token t, head) pairs: row r = t*G + hh for the
// G = H/n_kv heads of the group, so one K/V row is shared by all n_q*G rows.

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

// ---------------------------------------------------------------- K/V super-tile loader

// Moves one super-tile (TT token rows of one tensor) HBM -> registers -> LDS,
// converting storage type KVT to compute type CT.  Piece = 16 storage bytes.
template <int KVT, int CT, int TT, int NT>
struct TileLoader {
  static constexpr int SB = (KVT == KV_F32 ? 4 : KVT == KV_BF16 ? 2 : 1) * D;  // storage bytes / row
  static constexpr int PPR = SB / 16;
  static constexpr int NP = TT * PPR;
  static constexpr int PPT = (NP + NT - 1) / NT;
  static constexpr int EPP = 16 / (KVT == KV_F32 ? 4 : KVT == KV_BF16 ? 2 : 1);   // elements / piece
  static constexpr int ROWB = Mma<CT>::ROWB;
  u32x4 reg[PPT];

  // rowaddr(tok) -> byte pointer of that token's row; always a valid row (absent tokens are
  // clamped onto a present one and masked later), so the loads need no branch.
  template <class RowFn>
  __device__ void load(RowFn rowaddr, int tid) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = (NP % NT == 0) ? tid + i * NT : min(tid + i * NT, NP - 1);
      reg[i] = *(const u32x4*)(rowaddr(p / PPR) + (p % PPR) * 16);
    }
  }

  __device__ void store(char* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int p = tid + i * NT;
      if (!(NP % NT == 0 || p < NP)) continue;
      const int tok = p / PPR, e0 = (p % PPR) * EPP;     // first element of the piece
      char* dst = tile + tok * ROWB + e0 * Mma<CT>::ESZ;
      const u32x4 x = reg[i];
      if constexpr (CT == CT_BF16) {
        if constexpr (KVT == KV_BF16) {
          *(u32x4*)dst = x;
        } else {  // FP8 -> bf16 (exact): 16 codes -> 32 bytes
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 o;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t word = x[2 * h + (w >> 1)];
              const uint32_t c0 = (word >> (16 * (w & 1))) & 0xFFu, c1 = (word >> (16 * (w & 1) + 8)) & 0xFFu;
              o[w] = (__float_as_uint(e4m3_to_f32(c0)) >> 16) | (__float_as_uint(e4m3_to_f32(c1)) & 0xFFFF0000u);
            }
            *(u32x4*)(dst + 16 * h) = o;
          }
        }
      } else {  // fp32 compute: rows are 516 bytes apart (4-byte aligned stores)
        float* f = (float*)dst;
        if constexpr (KVT == KV_F32) {
#pragma unroll
          for (int w = 0; w < 4; ++w) f[w] = __uint_as_float(x[w]);
        } else if constexpr (KVT == KV_BF16) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            f[2 * w] = bf16_to_f32(x[w] & 0xFFFFu);
            f[2 * w + 1] = bf16_to_f32(x[w] >> 16);
          }
        } else {
#pragma unroll
          for (int w = 0; w < 16; ++w) f[w] = e4m3_to_f32((x[w >> 2] >> (8 * (w & 3))) & 0xFFu);
        }
      }
    }
  }
};

// ---------------------------------------------------------------- pass 1: split-K partials

template <int KVT, int CT, int NWR, int NWT, bool GATHER>
__global__ __launch_bounds__(64 * NWR * NWT) void attn_partial_kernel(AttnArgs a) {
  constexpr int NT = 64 * NWR * NWT;
  constexpr int TT = 32 * NWT;
  using M = Mma<CT>;
  constexpr int ROWB = M::ROWB;
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr bool SPLIT = (CT == CT_BF16) && (KVT != KV_FP8);
  constexpr int MAXG = 1152;                                      // gather chunk limit
  constexpr int TILES = 2 * TT * ROWB;
  constexpr int DP = D + 4;                                      // merge row pitch: 32 rows on distinct banks
  constexpr int MERGE = NWT > 1 ? NWR * NWT * 32 * (DP * 4 + 8) : 0;
  __shared__ __align__(16) char smem[TILES > MERGE ? TILES : MERGE];
  char* const kt = smem;
  char* const vt = smem + TT * ROWB;
  __shared__ float ksc[FP8 ? TT : 1], vsc[FP8 ? TT : 1];
  __shared__ int gidx[GATHER ? MAXG + TT : 1];                  // + TT: tail reads past the chunk stay inside

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gr = wave / NWT, tl = wave % NWT;
  const int list = blockIdx.y, chunk = blockIdx.x;

  int b, t0, g;
  if (GATHER) { g = list % a.n_kv; const int bt = list / a.n_kv; b = bt / a.n_q; t0 = bt % a.n_q; }
  else { g = list % a.n_kv; b = list / a.n_kv; t0 = 0; }
  const int Lb = a.seq_len[b];
  const int ntok = GATHER ? min(max(a.sel_count[(size_t)list], 0), a.sel_cap) : Lb;   // clamp caller data
  const int c0 = chunk * a.chunk;
  if (c0 >= ntok) return;                                         // no work: merge skips it
  const int c1 = min(ntok, c0 + a.chunk);
  const int64_t rs = a.row_start[b];
  const int SBy = TileLoader<KVT, CT, TT, NT>::SB;
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SBy;
  const char* vbase = (const char*)a.v + ((size_t)rs * a.n_kv + g) * SBy;
  const size_t rstride = (size_t)a.n_kv * SBy;

  if (GATHER) {
    const int32_t* il = a.sel_idx + (size_t)list * a.sel_cap;
    for (int i = tid; i < c1 - c0; i += NT) {
      int j = il[c0 + i];
      gidx[i] = (j >= 0 && j < Lb) ? j : -1;
    }
    __syncthreads();
  }

  // query rows of this wave
  const int row = blockIdx.z * 32 * NWR + 32 * gr + (lane & 31);
  const bool row_ok = row < a.R;
  typename M::QOp q;
  {
    const int t = t0 + (row_ok ? row / a.G : 0), hh = row_ok ? row % a.G : 0;
    const size_t qoff = (((size_t)b * a.n_q + t) * a.H + (size_t)g * a.G + hh) * D;
    const void* qrow = a.q_f32 ? (const void*)((const float*)a.q + qoff) : (const void*)((const uint16_t*)a.q + qoff);
    M::load_q(q, qrow, a.q_f32, row_ok, lane);
  }

  TileLoader<KVT, CT, TT, NT> kl, vl;
  // cache row of a tile token, clamped into the chunk (absent tokens are masked in the softmax)
  auto tok_row = [&](int base, int tok) -> int {
    const int pos = min(base + tok, c1 - 1);
    return GATHER ? max(gidx[pos - c0], 0) : pos;
  };
  auto issue = [&](int base) {
    kl.load([&](int tok) -> const char* { return kbase + (size_t)tok_row(base, tok) * rstride; }, tid);
    vl.load([&](int tok) -> const char* { return vbase + (size_t)tok_row(base, tok) * rstride; }, tid);
  };
  float sc_k = 0.f, sc_v = 0.f;
  auto issue_scales = [&](int base) {
    if (FP8) {
      const size_t r = (size_t)rs + tok_row(base, tid % TT);
      sc_k = a.k_scale[r * a.n_kv + g];
      sc_v = a.v_scale[r * a.n_kv + g];
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[4] = {};
  const float sl2 = a.scale_log2;

  issue(c0);
  issue_scales(c0);
  for (int base = c0; base < c1; base += TT) {
    kl.store(kt, tid);
    vl.store(vt, tid);
    if (FP8 && tid < TT) { ksc[tid] = sc_k; vsc[tid] = sc_v; }
    __syncthreads();
    if (base + TT < c1) { issue(base + TT); issue_scales(base + TT); }

    // ---- compute on this wave's 32-token sub-tile
    const int sub = base + tl * 32;                               // first list position of the sub-tile
    if (sub < c1) {
      const char* ks = kt + tl * 32 * ROWB;
      const char* vs = vt + tl * 32 * ROWB;
      f32x16 s = M::qk_t(ks, q, lane);
      float l2[16];
      float mt = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tk = tl * 32 + crow(lane, r);
        const int pos = base + tk;
        bool ok = pos < c1;
        if (GATHER) ok = ok && gidx[pos - c0] >= 0;
        float x = s[r] * sl2;
        if (FP8) x *= ksc[tk];
        l2[r] = ok ? x : -INFINITY;
        mt = fmaxf(mt, l2[r]);
      }
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      const float msub = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2f(m - msub);
      float p[16];
      lsum *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = exp2_fast(l2[r] - msub);
        lsum += p[r];
        if (FP8) p[r] *= vsc[tl * 32 + crow(lane, r)];            // v scale folded into P
      }
      m = mn;
#pragma unroll
      for (int mt4 = 0; mt4 < 4; ++mt4) acc[mt4] *= alpha;
      M::template pv<SPLIT>(acc, vs, p, lane);
    }
    __syncthreads();
  }

  lsum += __shfl_xor(lsum, 32);
  const size_t item = (size_t)list * a.max_chunks + chunk;
  const int rb = blockIdx.z * 32 * NWR;

  if constexpr (NWT == 1) {
    if (row_ok) {
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
  } else {
    // merge the NWT token lanes of each row group through LDS (tile buffers are free now)
    float* accb = (float*)smem;                                   // [gr][tl][32 rows][DP]
    float* mlb = accb + NWR * NWT * 32 * DP;                      // [gr][tl][32][2]
    {
      float* mine = accb + ((gr * NWT + tl) * 32 + (lane & 31)) * DP;
#pragma unroll
      for (int mt4 = 0; mt4 < 4; ++mt4)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 o = {acc[mt4][4 * r4], acc[mt4][4 * r4 + 1], acc[mt4][4 * r4 + 2], acc[mt4][4 * r4 + 3]};
          *(f32x4*)(mine + 32 * mt4 + crow(lane, 4 * r4)) = o;
        }
      if (lane < 32) {
        mlb[((gr * NWT + tl) * 32 + lane) * 2] = m;
        mlb[((gr * NWT + tl) * 32 + lane) * 2 + 1] = lsum;
      }
    }
    __syncthreads();
    // NT threads cover NWR*32 rows x 128 d; each does 16 consecutive d of one row
    constexpr int PER = NWR * 32 * D / NT;
    const int lin = tid * PER;
    const int rr = lin / D, d0 = lin % D;                         // rr = gr*32 + local row
    const int g2 = rr / 32, lr = rr % 32;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NWT; ++j) mx = fmaxf(mx, mlb[((g2 * NWT + j) * 32 + lr) * 2]);
    const float msub = mx == -INFINITY ? 0.f : mx;
    float w[NWT], ls = 0.f;
#pragma unroll
    for (int j = 0; j < NWT; ++j) {
      w[j] = exp2f(mlb[((g2 * NWT + j) * 32 + lr) * 2] - msub);
      ls += w[j] * mlb[((g2 * NWT + j) * 32 + lr) * 2 + 1];
    }
    const int grow = rb + rr;
    if (grow < a.R) {
      float* pa = a.part_acc + (item * a.R + grow) * D + d0;
#pragma unroll
      for (int e = 0; e < PER; e += 4) {
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NWT; ++j) o += w[j] * *(const f32x4*)(accb + ((g2 * NWT + j) * 32 + lr) * DP + d0 + e);
        *(f32x4*)(pa + e) = o;
      }
      if (d0 == 0) *(float2*)(a.part_ml + (item * a.R + grow) * 2) = make_float2(mx, ls);
    }
  }
}

// ---------------------------------------------------------------- merge

// Combines the chunks of a list for each row.  ROWW (few chunks, e.g. a sparse layer): one wave per
// (row, list), all chunks in one online pass; otherwise one workgroup per (row, list) whose wave w
// combines chunks w, w + 4, ..., then wave 0 combines the four parts in a fixed order.  The first
// partial loads do not wait for the list's count (merge_part_wave).
// ROWW: one wave per (row, list), four rows per workgroup (few chunks); otherwise one workgroup of
// NWM waves per (row, list), wave w taking chunks w, w + NWM, ... (8 loads in flight per wave), the
// waves' results combined through LDS in wave order.
template <bool ROWW, int NWM>
__global__ __launch_bounds__(64 * NWM) void attn_merge_kernel(MergeArgs a) {
  __shared__ float2 po[ROWW ? 1 : NWM][64];
  __shared__ float pm[NWM], pl[NWM];
  const int list = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = ROWW ? blockIdx.x * 4 + wave : blockIdx.x;
  if (ROWW && row >= a.R) return;
  int b, t, g;
  if (a.gather) { g = list % a.n_kv; const int bt = list / a.n_kv; b = bt / a.n_q; t = bt % a.n_q; }
  else { g = list % a.n_kv; b = list / a.n_kv; t = row / a.G; }
  const int hh = row % a.G;
  const int ntok = a.gather ? min(max(a.sel_count[list], 0), a.sel_cap) : a.seq_len[b];
  const int nch = min((ntok + a.chunk - 1) / a.chunk, a.max_chunks);
  const size_t first = (size_t)list * a.max_chunks * a.R + row;
  const MergePart r = merge_part_wave(a.part_ml + first * 2, (size_t)a.R * 2, a.part_acc + first * D, (size_t)a.R * D,
                                      ROWW ? 0 : wave, nch, a.max_chunks, ROWW ? 1 : NWM, lane);
  float mx, ls;
  float2 o;
  if constexpr (ROWW) {
    mx = r.m; ls = r.l; o = r.o;
  } else {
    po[wave][lane] = r.o;
    if (lane == 0) { pm[wave] = r.m; pl[wave] = r.l; }
    __syncthreads();
    if (wave) return;
    mx = pm[0];
#pragma unroll
    for (int w = 1; w < NWM; ++w) mx = fmaxf(mx, pm[w]);
    const float msub = mx == -INFINITY ? 0.f : mx;
    ls = 0.f;
    o = make_float2(0.f, 0.f);
#pragma unroll
    for (int w = 0; w < NWM; ++w) {
      const float wt = exp2f(pm[w] - msub);
      ls += wt * pl[w];
      o.x += wt * po[w][lane].x;
      o.y += wt * po[w][lane].y;
    }
  }
  const float inv = ls > 0.f ? 1.f / ls : 0.f;
  const size_t orow = ((size_t)b * a.n_q + t) * a.H + (size_t)g * a.G + hh;
  *(float2*)(a.out + orow * D + 2 * lane) = make_float2(o.x * inv, o.y * inv);
  if (lane == 0) {
    const float l2 = ls > 0.f ? mx + __log2f(ls) : -INFINITY;
    if (a.lse) a.lse[orow] = l2 * LN2;
    if (a.lse2) a.lse2[orow] = l2;
  }
}

// ---------------------------------------------------------------- pass 2: selection scores

// s[b, t, g, j] = sum_{hh < G} exp2(l2(t, hh, j) - lse2(t, hh)) for j < L_b - W'.
// S = Q K^T orientation: lane holds token (l & 31) and 16 rows, so the sum over
// a token-of-query's heads is mostly in-lane.  Requires G % 32 == 0 or G in {8, 16},
// and the rows of one query token inside one workgroup (checked by the host).
template <int KVT, int CT, int NWR, int NWT>
__global__ __launch_bounds__(64 * NWR * NWT) void attn_scores_kernel(ScoreArgs a) {
  constexpr int NT = 64 * NWR * NWT;
  constexpr int TT = 32 * NWT;
  using M = Mma<CT>;
  constexpr int ROWB = M::ROWB;
  constexpr bool FP8 = KVT == KV_FP8;
  __shared__ __align__(16) char kt[TT * ROWB];
  __shared__ float ksc[FP8 ? TT : 1];
  __shared__ float part[NWR][4][TT];                              // per-wave partial sums per local query token

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gr = wave / NWT, tl = wave % NWT;
  const int g = blockIdx.y % a.n_kv, b = blockIdx.y / a.n_kv;
  const int Lb = a.seq_len[b];
  const int w = min(a.window, Lb);
  const int ncand = Lb - w;
  const int c0 = blockIdx.x * a.chunk;
  if (c0 >= ncand) return;
  const int c1 = min(ncand, c0 + a.chunk);
  const int64_t rs = a.row_start[b];
  const int SBy = TileLoader<KVT, CT, TT, NT>::SB;
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SBy;
  const size_t rstride = (size_t)a.n_kv * SBy;

  const int rb = blockIdx.z * 32 * NWR;
  const int row = rb + 32 * gr + (lane & 31);
  typename M::QOp q;
  {
    const bool ok = row < a.R;
    const int t = ok ? row / a.G : 0, hh = ok ? row % a.G : 0;
    const size_t qoff = (((size_t)b * a.n_q + t) * a.H + (size_t)g * a.G + hh) * D;
    const void* qrow = a.q_f32 ? (const void*)((const float*)a.q + qoff) : (const void*)((const uint16_t*)a.q + qoff);
    M::load_q(q, qrow, a.q_f32, ok, lane);
  }
  // lse of this lane's 16 rows (rows 32 gr + crow(lane, r)); padding rows get +inf -> p = 0
  float lse2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {                                  // padding rows: +inf -> p = 0
    const int rw = rb + 32 * gr + crow(lane, r), rc = min(rw, a.R - 1);
    const float v = a.lse2[((size_t)b * a.n_q + rc / a.G) * a.H + (size_t)g * a.G + rc % a.G];
    lse2[r] = rw < a.R ? v : INFINITY;
  }
  // local query tokens of the workgroup: rows [rb, rb + 32*NWR) hold tokens rb/G ..
  const int tpw = a.G >= 32 ? 1 : 32 / a.G;                        // query tokens per wave
  const int wpt = a.G >= 32 ? a.G / 32 : 1;                        // waves per query token
  const int t_first = rb / a.G;
  const int nt_wg = (min(a.R, rb + 32 * NWR) - rb + a.G - 1) / a.G;

  TileLoader<KVT, CT, TT, NT> kl;
  auto issue = [&](int base) {                                    // clamped rows: no branch
    kl.load([&](int tok) -> const char* { return kbase + (size_t)min(base + tok, c1 - 1) * rstride; }, tid);
  };
  float sc_k = 0.f;
  auto issue_scales = [&](int base) {
    if (FP8) sc_k = a.k_scale[((size_t)rs + min(base + tid % TT, c1 - 1)) * a.n_kv + g];
  };
  issue(c0);
  issue_scales(c0);
  float* sout = a.scores + ((size_t)b * a.n_q * a.n_kv) * a.s_stride;
  for (int base = c0; base < c1; base += TT) {
    kl.store(kt, tid);
    if (FP8 && tid < TT) ksc[tid] = sc_k;
    __syncthreads();
    if (base + TT < c1) { issue(base + TT); issue_scales(base + TT); }
    const int sub = base + tl * 32;
    if (sub < c1) {
      f32x16 s = M::qk(kt + tl * 32 * ROWB, q, lane);
      const int tk = tl * 32 + (lane & 31);
      const float f = a.scale_log2 * (FP8 ? ksc[tk] : 1.f);
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = exp2_fast(s[r] * f - lse2[r]);
      if (tpw == 1) {
        float acc = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc += p[r];
        acc += __shfl_xor(acc, 32);
        if (lane < 32) part[gr][0][tk] = acc;
      } else {
        // rows 8*(r/4) + 4*(l>>5) + (r&3): each group of 4 r's is one 8-row block
        float blk[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          blk[q4] = p[4 * q4] + p[4 * q4 + 1] + p[4 * q4 + 2] + p[4 * q4 + 3];
          blk[q4] += __shfl_xor(blk[q4], 32);
        }
        if (lane < 32) {
          if (tpw == 4) {                                          // G = 8: one block per token
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) part[gr][q4][tk] = blk[q4];
          } else {                                                 // G = 16: two blocks per token
            part[gr][0][tk] = blk[0] + blk[1];
            part[gr][1][tk] = blk[2] + blk[3];
          }
        }
      }
    }
    __syncthreads();
    // combine waves of one query token (fixed order) and store
    for (int i = tid; i < nt_wg * TT; i += NT) {
      const int lt = i / TT, tk = i % TT;
      const int pos = base + tk;
      if (pos >= c1) continue;
      const int t = t_first + lt;
      float v = 0.f;
      if (tpw == 1) {
        for (int j = 0; j < wpt; ++j) v += part[lt * wpt + j][0][tk];   // waves of token lt, in order
      } else {
        v = part[lt / tpw][lt % tpw][tk];                              // wave lt/tpw holds tpw tokens
      }
      sout[((size_t)t * a.n_kv + g) * a.s_stride + pos] = v;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launchers

template <int KVT, int CT, int NWR, int NWT, bool GATHER>
static hipError_t launch_partial_t(const AttnArgs& a, int zblocks, hipStream_t st) {
  dim3 grid(a.max_chunks, a.n_lists, zblocks);
  hipLaunchKernelGGL((attn_partial_kernel<KVT, CT, NWR, NWT, GATHER>), grid, dim3(64 * NWR * NWT), 0, st, a);
  return hipGetLastError();
}

template <int KVT, int CT, bool GATHER>
static hipError_t launch_partial_shape(const AttnArgs& a, int nwr, hipStream_t st) {
  const int z = (a.R + 32 * nwr - 1) / (32 * nwr);
  if constexpr (CT == CT_F32) {                                  // fp32 path: at most 256 threads
    if (nwr == 1) return launch_partial_t<KVT, CT, 1, 4, GATHER>(a, z, st);
    return launch_partial_t<KVT, CT, 4, 1, GATHER>(a, z, st);
  } else {
    switch (nwr) {
      case 1: return launch_partial_t<KVT, CT, 1, 4, GATHER>(a, z, st);
      case 2: return launch_partial_t<KVT, CT, 2, 2, GATHER>(a, z, st);
      case 4: return launch_partial_t<KVT, CT, 4, 1, GATHER>(a, z, st);
      default: return launch_partial_t<KVT, CT, 8, 1, GATHER>(a, z, st);
    }
  }
}

int partial_tile_tokens(int nwr) { return nwr == 1 ? 128 : nwr == 2 ? 64 : 32; }

int rows_per_wave_group(int R) { return R <= 32 ? 1 : R <= 64 ? 2 : R <= 128 ? 4 : 8; }

template <bool GATHER>
static hipError_t launch_partial_g(const AttnArgs& a, int kvt, int ct, int nwr, hipStream_t st) {
  if (ct == CT_F32) {
    if (kvt == KV_F32) return launch_partial_shape<KV_F32, CT_F32, GATHER>(a, nwr, st);
    if (kvt == KV_BF16) return launch_partial_shape<KV_BF16, CT_F32, GATHER>(a, nwr, st);
    return launch_partial_shape<KV_FP8, CT_F32, GATHER>(a, nwr, st);
  }
  if (kvt == KV_BF16) return launch_partial_shape<KV_BF16, CT_BF16, GATHER>(a, nwr, st);
  if (kvt == KV_FP8) return launch_partial_shape<KV_FP8, CT_BF16, GATHER>(a, nwr, st);
  return hipErrorInvalidValue;
}

hipError_t launch_attn_partial(const AttnArgs& a, int kvt, int ct, int nwr, bool gather, hipStream_t st) {
  if (ct == CT_F32 && nwr != 1 && nwr != 4) return hipErrorInvalidValue;
  return gather ? launch_partial_g<true>(a, kvt, ct, nwr, st) : launch_partial_g<false>(a, kvt, ct, nwr, st);
}

hipError_t launch_attn_merge(const MergeArgs& m, hipStream_t st) {
  if (m.max_chunks <= 16) {
    dim3 grid((m.R + 3) / 4, m.n_lists);
    hipLaunchKernelGGL((attn_merge_kernel<true, 4>), grid, dim3(256), 0, st, m);
  } else if (m.max_chunks <= 64) {
    dim3 grid(m.R, m.n_lists);
    hipLaunchKernelGGL((attn_merge_kernel<false, 4>), grid, dim3(256), 0, st, m);
  } else {                                                        // 2 rounds of 8 loads per wave at 256 chunks
    dim3 grid(m.R, m.n_lists);
    hipLaunchKernelGGL((attn_merge_kernel<false, 16>), grid, dim3(1024), 0, st, m);
  }
  return hipGetLastError();
}

template <int KVT, int CT, int NWR, int NWT>
static hipError_t launch_scores_t(const ScoreArgs& a, hipStream_t st) {
  const int z = (a.R + 32 * NWR - 1) / (32 * NWR);
  dim3 grid(a.max_chunks, a.n_lists, z);
  hipLaunchKernelGGL((attn_scores_kernel<KVT, CT, NWR, NWT>), grid, dim3(64 * NWR * NWT), 0, st, a);
  return hipGetLastError();
}

template <int KVT, int CT>
static hipError_t launch_scores_shape(const ScoreArgs& a, int nwr, hipStream_t st) {
  switch (nwr) {
    case 1: return launch_scores_t<KVT, CT, 1, 4>(a, st);
    case 2: return launch_scores_t<KVT, CT, 2, 2>(a, st);
    case 4: return launch_scores_t<KVT, CT, 4, 1>(a, st);
    default:
      if constexpr (CT == CT_F32) return hipErrorInvalidValue;   // the host never asks for it
      else return launch_scores_t<KVT, CT, 8, 1>(a, st);
  }
}

hipError_t launch_attn_scores(const ScoreArgs& a, int kvt, int ct, int nwr, hipStream_t st) {
  if (ct == CT_F32) {
    if (kvt == KV_F32) return launch_scores_shape<KV_F32, CT_F32>(a, nwr, st);
    if (kvt == KV_BF16) return launch_scores_shape<KV_BF16, CT_F32>(a, nwr, st);
    return launch_scores_shape<KV_FP8, CT_F32>(a, nwr, st);
  }
  if (kvt == KV_BF16) return launch_scores_shape<KV_BF16, CT_BF16>(a, nwr, st);
  if (kvt == KV_FP8) return launch_scores_shape<KV_FP8, CT_BF16>(a, nwr, st);
  return hipErrorInvalidValue;
}

}  // namespace hs
