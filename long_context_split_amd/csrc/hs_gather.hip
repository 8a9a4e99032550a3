// Sparse-layer attention over a selection list (gfx950, bf16 MFMA), built for latency.
//
// ithome page "小米公开 MiMo-V3 核心架构 HySparse2", section "KV Reuse": a sparse
// layer attends, with its own queries, only to the cache rows that its hybrid
// block's full layer selected (the recent window plus the top-k positions), the
// softmax renormalised over that set.
//
// One list is about 1152 rows (590 KB of bf16 K and V), too little work to hide
// latency behind bandwidth, so the kernel keeps the dependent chain of a
// workgroup short.  Wave w takes the list positions c0 + 32 (w + NW i) .. + 31:
//   * lane l loads the row index of position l & 31; the rows follow at once
//     (indices passed between lanes), and every query head's Q row is held in
//     registers as the B operand of v_mfma_f32_32x32x16_bf16, so there is no
//     workgroup barrier before the final combine;
//   * K goes through a wave-private LDS tile ([token][d], coalesced row
//     loads) for bf16 caches; E4M3 rows (one 128-byte line) go straight into
//     registers in the A-operand layout (lane l: token l & 31, d in
//     64 (l >> 5) .. + 63, the same d order as Q's operand);
//   * V goes through a wave-private LDS tile, transposed ([d][token], written
//     as 32-bit token pairs), so the PV A operand is one 16-byte read;
//   * which positions are valid (inside the list's count, index in [0, L_b))
//     comes from a ballot over the wave's own index loads.
// The NW waves are combined through LDS at the end.  One workgroup per
// (chunk, list, block of 32 query heads) writes O when the chunk is the whole
// list, else one (m, l, acc) partial per head that attn_merge combines.

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

namespace {

constexpr int GVROW = 80;                          // V^T row: 32 tokens x 2 B + 16 B pad
constexpr int GVT = D * GVROW + (D / 16) * 64;     // one wave's V^T tile (+ 64 B per 16-row block)
constexpr int GKROW = 272;                         // K tile row: 256 B + 16 B pad (bank spread)

// Byte offset of row d of a V^T tile.  Each 16-row block is shifted by a further 64 bytes: the
// operand reads (16 lanes, 16 consecutive rows, one column quad) and the transposing writes
// (16 lanes, one row, 16 token pairs; the other lane groups 8, 16 or 32 rows away) then fall on
// distinct LDS banks.
__device__ __forceinline__ int gvt_row(int d) { return d * GVROW + (d >> 4) * 64; }

// Stored column of token t (0..31): within each 16-token group bits 2 and 3 are swapped, the order
// in which the P operand holds its tokens, so a lane's 8 k values are 8 adjacent columns.
__device__ __forceinline__ int gvt_col(int t) {
  const int o = t & 15;
  return (t & ~15) | (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1);
}

}  // namespace

template <int KVT, int NW>
__global__ __launch_bounds__(64 * NW) void attn_gather_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr bool SPLIT = !FP8;                      // bf16 cache: P as bf16 hi + lo
  constexpr int SB = (FP8 ? 1 : 2) * D;             // bytes per cache row
  constexpr int KPL = SB / 32;                      // 16-byte K pieces per lane per tile
  constexpr int PPR = SB / 16;                      // 16-byte pieces per row
  constexpr int NPP = PPR / 4;                      // V token-pair pieces per lane
  constexpr int EPP = FP8 ? 16 : 8;                 // elements per piece
  constexpr int DP = D + 4;                         // merge row pitch: 32 heads' rows on distinct banks
  constexpr int MERGE = NW * 32 * (DP + 2) * 4;
  constexpr int KT = FP8 ? 0 : 32 * GKROW;         // bf16: the wave's K tile
  constexpr int TILES = NW * (GVT + KT);
  __shared__ __align__(16) char smem[TILES > MERGE ? TILES : MERGE];
  __shared__ __align__(16) float scl[FP8 ? NW : 1][2][32];  // per wave: K scale x softmax scale, V scale

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, list = blockIdx.y, hb = blockIdx.z;
  const int g = list % a.n_kv, bt = list / a.n_kv, b = bt / a.n_q, t0 = bt % a.n_q;
  const int32_t* il = a.sel_idx + (size_t)list * a.sel_cap;
  const int c0 = chunk * a.chunk;                   // < sel_cap (grid)
  const int cend = min(c0 + a.chunk, a.sel_cap);
  const int tok = lane & 31, half = lane >> 5;
  // the first tile's row index goes out first: the K/V loads wait for this one load only
  int jn = il[min(c0 + 32 * wave + tok, cend - 1)];

  // Q operand: head hb*32 + tok; k-step st covers d = 16 st + 8 half .. + 7 (bf16, as the K tile is
  // read) or d = 64 half + 8 st .. + 7 (E4M3, as its K registers hold it).  Heads past G read head 0's
  // row (their columns of S are computed and never stored).
  const int head = hb * 32 + tok;
  s16x8 qv[8];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((size_t)b * a.n_q + t0) * a.H + (size_t)g * a.G + (head < a.G ? head : 0)) * D;
#pragma unroll
    for (int st = 0; st < 8; ++st) qv[st] = *(const s16x8*)(qrow + (FP8 ? 64 * half + 8 * st : 16 * st + 8 * half));
  }
  const int Lb = a.seq_len[b];
  const int ntok = min(max(a.sel_count[(size_t)list], 0), a.sel_cap);
  // whole workgroup: the merge skips this chunk; a direct workgroup (the whole list) goes on with no
  // tile, so an empty list gets zeros, as the merge writes for it
  if (c0 >= ntok && !a.direct) return;
  const int c1 = min(ntok, c0 + a.chunk);
  const int ntiles = (c1 - c0 + 31) / 32;
  const int64_t rs = a.row_start[b];
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SB;
  const char* vbase = (const char*)a.v + ((size_t)rs * a.n_kv + g) * SB;
  const size_t rstride = (size_t)a.n_kv * SB;
  char* const vt = smem + wave * (GVT + KT);
  char* const kt = vt + GVT;
  const float sl2 = a.scale_log2;

  // Rows of a tile from the raw index j of this lane's position: invalid positions (past the
  // list's count, negative or out-of-range indices) read row 0 and are masked in the softmax.
  u32x4 rk[KPL], rv[2 * NPP];
  float sk = 0.f, sv = 0.f;
  uint32_t vmask = 0u;
  auto load_rows = [&](int tile, int j) {
    const bool ok = c0 + 32 * tile + tok < c1 && j >= 0 && j < Lb;
    const int jr = ok ? j : 0;
    vmask = (uint32_t)__ballot(ok);                 // bit t: position t of the tile (lanes 32..63 repeat)
    if constexpr (FP8) {                            // half of this lane's row, in operand order
      const char* kr = kbase + (size_t)jr * rstride + (SB / 2) * half;
#pragma unroll
      for (int i = 0; i < KPL; ++i) rk[i] = *(const u32x4*)(kr + 16 * i);
    } else {                                        // token (lane >> 4) + 4 i, piece lane & 15
#pragma unroll
      for (int i = 0; i < KPL; ++i) {
        const int rr = __shfl(jr, (lane >> 4) + 4 * i);
        rk[i] = *(const u32x4*)(kbase + (size_t)rr * rstride + 16 * (lane & 15));
      }
    }
    const int r0 = __shfl(jr, 2 * (lane & 15)), r1 = __shfl(jr, 2 * (lane & 15) + 1);
#pragma unroll
    for (int i = 0; i < NPP; ++i) {                 // tokens 2m, 2m + 1 (m = lane & 15), piece c
      const int c = (lane >> 4) + 4 * i;
      rv[2 * i] = *(const u32x4*)(vbase + (size_t)r0 * rstride + 16 * c);
      rv[2 * i + 1] = *(const u32x4*)(vbase + (size_t)r1 * rstride + 16 * c);
    }
    if (FP8) {
      sk = a.k_scale[((size_t)rs + jr) * a.n_kv + g];
      sv = a.v_scale[((size_t)rs + jr) * a.n_kv + g];
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[4] = {};
  if (wave < ntiles) load_rows(wave, jn);
  for (int tile = wave; tile < ntiles; tile += NW) {
    const int nxt = tile + NW;
    if (nxt < ntiles) jn = il[min(c0 + 32 * nxt + tok, c1 - 1)];
    const uint32_t mask = vmask;
    // ---- V (registers) -> V^T tile, 32-bit words holding tokens (2m, 2m + 1) of one d
#pragma unroll
    for (int i = 0; i < NPP; ++i) {
      const int m2 = 2 * (lane & 15), c = (lane >> 4) + 4 * i;
      uint32_t w0[EPP / 2], w1[EPP / 2];            // bf16 pairs (d, d + 1) of tokens m2 and m2 + 1
      if constexpr (FP8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          e4m3x4_to_bf16x4(rv[2 * i][w], w0[2 * w], w0[2 * w + 1]);
          e4m3x4_to_bf16x4(rv[2 * i + 1][w], w1[2 * w], w1[2 * w + 1]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) { w0[w] = rv[2 * i][w]; w1[w] = rv[2 * i + 1][w]; }
      }
      const int cb = gvt_col(m2) * 2;               // token m2 + 1 is the next column
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const uint32_t a0 = w0[e >> 1], a1 = w1[e >> 1];
        const uint32_t word = (e & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
        *(uint32_t*)(vt + gvt_row(c * EPP + e) + cb) = word;
      }
    }
    if (FP8 && lane < 32) { scl[wave][0][lane] = sk * sl2; scl[wave][1][lane] = sv; }
    if constexpr (!FP8) {                           // K rows -> K tile [token][d]
#pragma unroll
      for (int i = 0; i < KPL; ++i) *(u32x4*)(kt + ((lane >> 4) + 4 * i) * GKROW + 16 * (lane & 15)) = rk[i];
      wave_sync();
    }

    // ---- S^T = K Q^T
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      u32x4 ka;
      if constexpr (FP8) {                          // 8 codes (d = 64 half + 8 st ..) -> 8 bf16, exact
        const u32x4 x = rk[st >> 1];
        uint32_t k0, k1, k2, k3;
        e4m3x4_to_bf16x4(x[2 * (st & 1)], k0, k1);
        e4m3x4_to_bf16x4(x[2 * (st & 1) + 1], k2, k3);
        ka = u32x4{k0, k1, k2, k3};
      } else {
        ka = *(const u32x4*)(kt + tok * GKROW + 32 * st + 16 * half);
      }
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qv[st]),
                                                  s, 0, 0, 0);
    }
    // the next tile's rows go out now: K and V registers are free once their MFMAs and LDS writes
    // have issued, and the loads overlap this tile's softmax and PV
    if (nxt < ntiles) load_rows(nxt, jn);
    wave_sync();                                    // V^T tile and scales visible to the wave

    // ---- online softmax (log2 units); lane: head tok, tokens crow(lane, r)
    float x[16], vs[16];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const int tb = 8 * k4 + 4 * half;             // crow(lane, 4 k4 + i) = tb + i
      f32x4 f = {sl2, sl2, sl2, sl2};
      if (FP8) {
        f = *(const f32x4*)&scl[wave][0][tb];
        const f32x4 v4 = *(const f32x4*)&scl[wave][1][tb];
#pragma unroll
        for (int i = 0; i < 4; ++i) vs[4 * k4 + i] = v4[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * k4 + i] = ((mask >> (tb + i)) & 1u) ? s[4 * k4 + i] * f[i] : -INFINITY;
    }
    float mt = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
    mt = xor32_max(mt);
    const float mn = fmaxf(m, mt);
    const float msub = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2f(m - msub);            // m = -inf: 0
    lsum *= alpha;
#pragma unroll
    for (int mt4 = 0; mt4 < 4; ++mt4) acc[mt4] *= alpha;
    m = mn;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = exp2_fast(x[r] - msub);
      lsum += p[r];
      if (FP8) p[r] *= vs[r];                       // V scale folded into P
    }
    // ---- O^T += V^T P^T: k-step u, element j <-> p[8u + j] <-> V^T columns 16u + 8 half + j
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
      const char* vr = vt + gvt_row(32 * mt4 + tok) + 16 * half;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const s16x8 va = *(const s16x8*)(vr + 32 * u);
        acc[mt4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                           __builtin_bit_cast(bf16x8, ph[u]), acc[mt4], 0, 0, 0);
        if (SPLIT)
          acc[mt4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                             __builtin_bit_cast(bf16x8, pl[u]), acc[mt4], 0, 0, 0);
      }
    }
    wave_sync();                                    // reads done before the next tile's writes
  }
  lsum = xor32_add(lsum);

  // ---- combine the NW waves (fixed order) through LDS
  __syncthreads();
  float* accb = (float*)smem;                       // [wave][32 heads][DP]
  float* mlb = accb + NW * 32 * DP;                 // [wave][32][2]
  {
    float* mine = accb + (wave * 32 + tok) * DP;
#pragma unroll
    for (int mt4 = 0; mt4 < 4; ++mt4)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 o = {acc[mt4][4 * r4], acc[mt4][4 * r4 + 1], acc[mt4][4 * r4 + 2], acc[mt4][4 * r4 + 3]};
        *(f32x4*)(mine + 32 * mt4 + crow(lane, 4 * r4)) = o;
      }
    if (lane < 32) {
      mlb[(wave * 32 + lane) * 2] = m;
      mlb[(wave * 32 + lane) * 2 + 1] = lsum;
    }
  }
  __syncthreads();
  constexpr int PER = 32 * D / NT;                  // d values per thread
  static_assert(PER % 4 == 0, "whole f32x4 per thread");
  const int lin = tid * PER, row = lin / D, d0 = lin % D;
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < NW; ++j) mx = fmaxf(mx, mlb[(j * 32 + row) * 2]);
  const float msub = mx == -INFINITY ? 0.f : mx;
  float ls = 0.f;
  f32x4 o[PER / 4];
#pragma unroll
  for (int e = 0; e < PER / 4; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    const float wj = exp2f(mlb[(j * 32 + row) * 2] - msub);
    ls += wj * mlb[(j * 32 + row) * 2 + 1];
#pragma unroll
    for (int e = 0; e < PER / 4; ++e) o[e] += wj * *(const f32x4*)(accb + (j * 32 + row) * DP + d0 + 4 * e);
  }
  const int gh = hb * 32 + row;                     // head within the KV group
  if (gh >= a.G) return;
  if (a.direct) {                                   // the chunk is the whole list: final output
    const size_t orow = ((size_t)b * a.n_q + t0) * a.H + (size_t)g * a.G + gh;
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
    for (int e = 0; e < PER / 4; ++e) *(f32x4*)(a.out + orow * D + d0 + 4 * e) = o[e] * inv;
    return;
  }
  const size_t item = (size_t)list * a.max_chunks + chunk;
  float* pa = a.part_acc + (item * a.R + gh) * D + d0;
#pragma unroll
  for (int e = 0; e < PER / 4; ++e) *(f32x4*)(pa + 4 * e) = o[e];
  if (d0 == 0) *(float2*)(a.part_ml + (item * a.R + gh) * 2) = make_float2(mx, ls);
}

template <int KVT>
static hipError_t launch_gather_t(const AttnArgs& a, hipStream_t st) {
  constexpr int NW = 8;
  dim3 grid(a.max_chunks, a.n_lists, (a.G + 31) / 32);
  hipLaunchKernelGGL((attn_gather_kernel<KVT, NW>), grid, dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_gather(const AttnArgs& a, int kvt, hipStream_t st) {
  if (a.q_f32 || a.chunk <= 0 || a.chunk % 32 || a.R != a.G) return hipErrorInvalidValue;
  if (kvt == KV_BF16) return launch_gather_t<KV_BF16>(a, st);
  if (kvt == KV_FP8) return launch_gather_t<KV_FP8>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace hs
