// Sliding-window attention over a cache chunk (gfx950, bf16 MFMA): the Self-Decoder side that feeds
// KV Bridging.
//
// ithome page "小米公开 MiMo-V3 核心架构 HySparse2", architecture overview: the Self-Decoder mixes
// full attention with sliding-window attention over the current input, and its full layers' hidden
// states feed the Cross-Decoder through KV Bridging.  The pages give no window size; it is a
// parameter here.  Query token i of sequence b (a chunk of n_q tokens ending at the last cache row)
// sits at position p = L_b - n_q + i and attends to rows max(0, p - w + 1) .. p of its own cache,
// the softmax taken over that band.
//
// One wave per query token and block of 32 query heads of one KV head, 8 waves (8 consecutive
// tokens) per workgroup; each wave walks its band in 32-row tiles with the sparse gather's tile code
// path (rows at computed positions instead of loaded indices):
//   * K through a wave-private LDS tile ([token][d]) for bf16 caches, E4M3 rows straight into
//     operand registers; V transposed into a wave-private LDS tile as 32-bit token pairs;
//   * S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16, online softmax in log2 units;
//   * the wave owns its token's whole band, so there is no partial and no merge: it normalises and
//     writes its 32 heads' rows through the same LDS area, 512 contiguous bytes per head row.
// Bands overlap between neighbouring tokens, so K/V rows come mostly from L2; the kernel's HBM
// traffic is Q in and O out.

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

namespace {

constexpr int SVROW = 80;                          // V^T row: 32 tokens x 2 B + 16 B pad
constexpr int SVT = D * SVROW + (D / 16) * 64;     // one wave's V^T tile (+ 64 B per 16-row block)
constexpr int SKROW = 272;                         // K tile row: 256 B + 16 B pad
constexpr int SOP = D + 4;                         // output staging row pitch (floats)

// row d of a V^T tile; each 16-row block shifted by a further 64 bytes (bank spread of the
// transposing writes and the operand reads)
__device__ __forceinline__ int svt_row(int d) { return d * SVROW + (d >> 4) * 64; }

// stored column of token t (0..31): bits 2 and 3 swapped within each 16-token group, the order in
// which the P operand holds its tokens
__device__ __forceinline__ int svt_col(int t) {
  const int o = t & 15;
  return (t & ~15) | (o & 3) | ((o & 4) << 1) | ((o & 8) >> 1);
}

}  // namespace

template <int KVT, int NW>
__global__ __launch_bounds__(64 * NW) void swa_attn_kernel(AttnArgs a) {
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr bool SPLIT = !FP8;                      // bf16 cache: P as bf16 hi + lo
  constexpr int SB = (FP8 ? 1 : 2) * D;             // bytes per cache row
  constexpr int KPL = SB / 32;                      // 16-byte K pieces per lane per tile
  constexpr int PPR = SB / 16;                      // 16-byte pieces per row
  constexpr int NPP = PPR / 4;                      // V token-pair pieces per lane
  constexpr int EPP = FP8 ? 16 : 8;                 // elements per piece
  constexpr int KT = FP8 ? 0 : 32 * SKROW;
  constexpr int TILE = SVT + KT;
  constexpr int STG = (32 * SOP + 32) * 4;          // output rows + per-head 1 / sum
  constexpr int PER_WAVE = TILE > STG ? TILE : STG;
  __shared__ __align__(16) char smem[NW * PER_WAVE];
  __shared__ __align__(16) float scl[FP8 ? NW : 1][2][32];  // per wave: K scale x softmax scale, V scale

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x * NW + wave;             // query token of this wave
  if (i >= a.n_q) return;                           // no workgroup barrier below: waves end on their own
  const int list = blockIdx.y, hb = blockIdx.z;
  const int g = list % a.n_kv, b = list / a.n_kv;
  const int tok = lane & 31, half = lane >> 5;
  const int Lb = a.seq_len[b];
  const int pos = Lb - a.n_q + i;                   // >= 0: n_q <= L_b is checked on the host
  const int jlo = max(0, pos - a.window + 1);
  const int ntiles = (pos - jlo + 32) / 32;         // >= 1

  const int head = hb * 32 + tok;                   // heads past G read head 0's row, never stored
  s16x8 qv[8];
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((size_t)b * a.n_q + i) * a.H + (size_t)g * a.G + (head < a.G ? head : 0)) * D;
#pragma unroll
    for (int st = 0; st < 8; ++st) qv[st] = *(const s16x8*)(qrow + (FP8 ? 64 * half + 8 * st : 16 * st + 8 * half));
  }
  const int64_t rs = a.row_start[b];
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SB;
  const char* vbase = (const char*)a.v + ((size_t)rs * a.n_kv + g) * SB;
  const size_t rstride = (size_t)a.n_kv * SB;
  char* const vt = smem + wave * PER_WAVE;
  char* const kt = vt + SVT;
  const float sl2 = a.scale_log2;

  // rows of a tile: position jlo + 32 tile + t, clamped to pos (the clamped ones are masked)
  u32x4 rk[KPL], rv[2 * NPP];
  float sk = 0.f, sv = 0.f;
  auto row_of = [&](int tile, int t) { return min(jlo + 32 * tile + t, pos); };
  auto load_rows = [&](int tile) {
    if constexpr (FP8) {                            // half of this lane's row, in operand order
      const char* kr = kbase + (size_t)row_of(tile, tok) * rstride + (SB / 2) * half;
#pragma unroll
      for (int k = 0; k < KPL; ++k) rk[k] = *(const u32x4*)(kr + 16 * k);
    } else {                                        // token (lane >> 4) + 4 k, piece lane & 15
#pragma unroll
      for (int k = 0; k < KPL; ++k)
        rk[k] = *(const u32x4*)(kbase + (size_t)row_of(tile, (lane >> 4) + 4 * k) * rstride + 16 * (lane & 15));
    }
    const size_t r0 = row_of(tile, 2 * (lane & 15)), r1 = row_of(tile, 2 * (lane & 15) + 1);
#pragma unroll
    for (int k = 0; k < NPP; ++k) {                 // tokens 2m, 2m + 1 (m = lane & 15), piece c
      const int c = (lane >> 4) + 4 * k;
      rv[2 * k] = *(const u32x4*)(vbase + r0 * rstride + 16 * c);
      rv[2 * k + 1] = *(const u32x4*)(vbase + r1 * rstride + 16 * c);
    }
    if (FP8) {
      const size_t r = ((size_t)rs + row_of(tile, tok)) * a.n_kv + g;
      sk = a.k_scale[r];
      sv = a.v_scale[r];
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[4] = {};
  load_rows(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    const int nvalid = min(32, pos - (jlo + 32 * tile) + 1);
    const uint32_t mask = nvalid >= 32 ? ~0u : (1u << nvalid) - 1u;   // bit t: position t of the tile
    // ---- V (registers) -> V^T tile, 32-bit words holding tokens (2m, 2m + 1) of one d
#pragma unroll
    for (int k = 0; k < NPP; ++k) {
      const int m2 = 2 * (lane & 15), c = (lane >> 4) + 4 * k;
      uint32_t w0[EPP / 2], w1[EPP / 2];
      if constexpr (FP8) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          e4m3x4_to_bf16x4(rv[2 * k][w], w0[2 * w], w0[2 * w + 1]);
          e4m3x4_to_bf16x4(rv[2 * k + 1][w], w1[2 * w], w1[2 * w + 1]);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) { w0[w] = rv[2 * k][w]; w1[w] = rv[2 * k + 1][w]; }
      }
      const int cb = svt_col(m2) * 2;
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        const uint32_t a0 = w0[e >> 1], a1 = w1[e >> 1];
        const uint32_t word = (e & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
        *(uint32_t*)(vt + svt_row(c * EPP + e) + cb) = word;
      }
    }
    if (FP8 && lane < 32) { scl[wave][0][lane] = sk * sl2; scl[wave][1][lane] = sv; }
    if constexpr (!FP8) {
#pragma unroll
      for (int k = 0; k < KPL; ++k) *(u32x4*)(kt + ((lane >> 4) + 4 * k) * SKROW + 16 * (lane & 15)) = rk[k];
      wave_sync();
    }

    // ---- S^T = K Q^T
    f32x16 s = {};
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      u32x4 ka;
      if constexpr (FP8) {
        const u32x4 x = rk[st >> 1];
        uint32_t k0, k1, k2, k3;
        e4m3x4_to_bf16x4(x[2 * (st & 1)], k0, k1);
        e4m3x4_to_bf16x4(x[2 * (st & 1) + 1], k2, k3);
        ka = u32x4{k0, k1, k2, k3};
      } else {
        ka = *(const u32x4*)(kt + tok * SKROW + 32 * st + 16 * half);
      }
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qv[st]),
                                                  s, 0, 0, 0);
    }
    if (tile + 1 < ntiles) load_rows(tile + 1);     // registers are free once the MFMAs and LDS writes issued
    wave_sync();

    // ---- online softmax (log2 units); lane: head tok, tokens crow(lane, r)
    float x[16], vs[16];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const int tb = 8 * k4 + 4 * half;
      f32x4 f = {sl2, sl2, sl2, sl2};
      if (FP8) {
        f = *(const f32x4*)&scl[wave][0][tb];
        const f32x4 v4 = *(const f32x4*)&scl[wave][1][tb];
#pragma unroll
        for (int r = 0; r < 4; ++r) vs[4 * k4 + r] = v4[r];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) x[4 * k4 + r] = ((mask >> (tb + r)) & 1u) ? s[4 * k4 + r] * f[r] : -INFINITY;
    }
    float mt = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mn = fmaxf(m, mt);
    const float msub = mn == -INFINITY ? 0.f : mn;
    const float alpha = exp2f(m - msub);
    lsum *= alpha;
#pragma unroll
    for (int mt4 = 0; mt4 < 4; ++mt4) acc[mt4] *= alpha;
    m = mn;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = exp2_fast(x[r] - msub);
      lsum += p[r];
      if (FP8) p[r] *= vs[r];
    }
    // ---- O^T += V^T P^T
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
      const char* vr = vt + svt_row(32 * mt4 + tok) + 16 * half;
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
  lsum += __shfl_xor(lsum, 32);

  // ---- normalise and write: O^T in acc (d = 32 mt4 + crow(lane, r), head tok) -> staging rows
  float* const orow_s = (float*)(smem + wave * PER_WAVE);
  float* const inv_s = orow_s + 32 * SOP;
#pragma unroll
  for (int mt4 = 0; mt4 < 4; ++mt4)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 o = {acc[mt4][4 * r4], acc[mt4][4 * r4 + 1], acc[mt4][4 * r4 + 2], acc[mt4][4 * r4 + 3]};
      *(f32x4*)(orow_s + tok * SOP + 32 * mt4 + crow(lane, 4 * r4)) = o;
    }
  if (lane < 32) inv_s[lane] = lsum > 0.f ? 1.f / lsum : 0.f;
  wave_sync();
  const size_t obase = ((size_t)b * a.n_q + i) * a.H + (size_t)g * a.G;
#pragma unroll
  for (int e = 0; e < 16; ++e) {                    // rows 2 e, 2 e + 1: 512 contiguous bytes each
    const int h = 2 * e + half, gh = hb * 32 + h;
    if (gh < a.G) {
      const f32x4 o = *(const f32x4*)(orow_s + h * SOP + 4 * tok) * inv_s[h];
      *(f32x4*)(a.out + (obase + gh) * D + 4 * tok) = o;
    }
  }
}

template <int KVT>
static hipError_t launch_swa_t(const AttnArgs& a, hipStream_t st) {
  constexpr int NW = 8;
  dim3 grid((a.n_q + NW - 1) / NW, a.n_lists, (a.G + 31) / 32);
  hipLaunchKernelGGL((swa_attn_kernel<KVT, NW>), grid, dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_swa_attn(const AttnArgs& a, int kvt, hipStream_t st) {
  if (a.q_f32 || a.window < 1 || a.n_q < 1) return hipErrorInvalidValue;
  if (kvt == KV_BF16) return launch_swa_t<KV_BF16>(a, st);
  if (kvt == KV_FP8) return launch_swa_t<KV_FP8>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace hs
