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
// tokens) per workgroup.  The 8 bands overlap almost entirely, so the workgroup walks their union
// in 32-row tiles: each tile is loaded once by all threads (next tile in registers while the
// current one is used), stored in LDS as bf16 [token][d] for K and V (E4M3 converted on the way),
// and every wave applies its own band as a mask.  S^T = K Q^T and O^T += V^T P^T run on bf16 MFMA
// with an online softmax in log2 units; the V^T operand comes from two LDS transpose reads (4 rows
// each, the token order of the P operand).  The output goes straight from the accumulators.
// Bands overlap between neighbouring workgroups too, so K/V rows come mostly from L2; the kernel's
// HBM traffic is Q in and O out.

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

namespace {

constexpr int SKROW = 272;                         // K tile row: 256 B + 16 B pad (16-byte operand reads)
constexpr int SVROW = 288;                         // V tile row: 256 B + 32 B pad (4-row transpose reads)
constexpr int SBUF = 32 * SKROW + 32 * SVROW;      // one tile: K then V (bf16)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
// LDS transpose read: lane L of each 16-lane group gets column L & 15 of the 4 x 16 block whose row
// (L & 15) >> 2, columns 4 (L & 3) .. + 3 it addresses
__device__ __forceinline__ u32x2 read_tr(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p)));
}

}  // namespace

template <int KVT, int NW>
__global__ __launch_bounds__(64 * NW) void swa_attn_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr bool SPLIT = !FP8;                      // bf16 cache: P as bf16 hi + lo
  constexpr int SB = (FP8 ? 1 : 2) * D;             // bytes per cache row
  constexpr int PPR = SB / 16;                      // 16-byte pieces per row
  constexpr int PPT = 2 * 32 * PPR / NT;            // 16-byte pieces per thread per tile (K and V)
  static_assert(PPT >= 1 && PPT * NT == 2 * 32 * PPR, "a tile's K and V pieces split evenly over the threads");
  __shared__ __align__(16) char smem[2 * SBUF];
  __shared__ float scl[2][2][32];                   // per buffer: K scale x softmax scale, V scale (E4M3)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int list = blockIdx.y, hb = blockIdx.z;
  const int g = list % a.n_kv, b = list / a.n_kv;
  const int tok = lane & 31, half = lane >> 5;
  const int Lb = a.seq_len[b];
  const int i0 = blockIdx.x * NW;                   // first query token of the workgroup (< n_q)
  const int i = i0 + wave;
  const bool active = i < a.n_q;                    // inactive waves still load and sync
  const int pos = Lb - a.n_q + min(i, a.n_q - 1);   // >= 0: n_q <= L_b is checked on the host
  const int lo = max(0, pos - a.window + 1);
  const int ulo = max(0, Lb - a.n_q + i0 - a.window + 1);            // the union of the bands
  const int uhi = Lb - a.n_q + min(i0 + NW, a.n_q) - 1;
  const int ntiles = (uhi - ulo + 32) / 32;

  const int head = hb * 32 + tok;                   // heads past G read head 0's row, never stored
  s16x8 qv[8];                                      // B operand: d = 16 st + 8 half
  {
    const uint16_t* qrow = (const uint16_t*)a.q + (((size_t)b * a.n_q + min(i, a.n_q - 1)) * a.H + (size_t)g * a.G + (head < a.G ? head : 0)) * D;
#pragma unroll
    for (int st = 0; st < 8; ++st) qv[st] = *(const s16x8*)(qrow + 16 * st + 8 * half);
  }
  const int64_t rs = a.row_start[b];
  const size_t rstride = (size_t)a.n_kv * SB;
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SB;
  const char* vbase = (const char*)a.v + ((size_t)rs * a.n_kv + g) * SB;
  const float sl2 = a.scale_log2;

  // piece q = tid + NT j of a tile: q < 32 PPR a K piece, else a V piece (row q' / PPR, piece q' % PPR)
  u32x4 rg[PPT];
  float rsc[PPT];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int q = tid + NT * j, isv = q >= 32 * PPR, pc = q % (32 * PPR), ptok = pc / PPR, ppc = pc % PPR;
      const int row = min(ulo + 32 * t + ptok, uhi);  // rows past the union clamp (never valid)
      rg[j] = *(const u32x4*)((isv ? vbase : kbase) + (size_t)row * rstride + 16 * ppc);
      if (FP8 && ppc == 0) rsc[j] = (isv ? a.v_scale : a.k_scale)[((size_t)rs + row) * a.n_kv + g];
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int q = tid + NT * j, isv = q >= 32 * PPR, pc = q % (32 * PPR), ptok = pc / PPR, ppc = pc % PPR;
      char* const dst = smem + buf * SBUF + (isv ? 32 * SKROW + ptok * SVROW : ptok * SKROW);
      if constexpr (FP8) {                          // 16 codes -> 16 bf16 (exact)
        uint32_t w[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) e4m3x4_to_bf16x4(rg[j][c], w[2 * c], w[2 * c + 1]);
        *(u32x4*)(dst + 32 * ppc) = u32x4{w[0], w[1], w[2], w[3]};
        *(u32x4*)(dst + 32 * ppc + 16) = u32x4{w[4], w[5], w[6], w[7]};
        if (ppc == 0) scl[buf][isv][ptok] = isv ? rsc[j] : rsc[j] * sl2;
      } else {
        *(u32x4*)(dst + 16 * ppc) = rg[j];
      }
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[4] = {};
  load_tile(0);
  store_tile(0);
  if (ntiles > 1) load_tile(1);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const char* const kt = smem + buf * SBUF;
    const char* const vt = kt + 32 * SKROW;
    const int base = ulo + 32 * t;                  // row of tile position 0
    const int first = max(lo - base, 0), last = min(pos - base, 31);
    const uint32_t mask = !active || last < first ? 0u
                        : ((last >= 31 ? ~0u : (1u << (last + 1)) - 1u) & ~((1u << first) - 1u));
    if (mask) {                                     // uniform over the wave
      // ---- S^T = K Q^T
      f32x16 s = {};
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const u32x4 ka = *(const u32x4*)(kt + tok * SKROW + 32 * st + 16 * half);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qv[st]),
                                                    s, 0, 0, 0);
      }
      // ---- online softmax (log2 units); lane: head tok, tokens crow(lane, r)
      float x[16], vs[16];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int tb = 8 * k4 + 4 * half;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float f = FP8 ? scl[buf][0][tb + r] : sl2;
          if (FP8) vs[4 * k4 + r] = scl[buf][1][tb + r];
          x[4 * k4 + r] = ((mask >> (tb + r)) & 1u) ? s[4 * k4 + r] * f : -INFINITY;
        }
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
      // ---- O^T += V^T P^T: k-step u, element e <-> p[8 u + e] <-> token 16 u + 8 (e >> 2) + 4 half + (e & 3)
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
      // A operand (d = 32 mt4 + (lane & 31)): group G = lane >> 4 reads columns 32 mt4 + 16 (G & 1) ..,
      // rows 16 u + 4 (G >> 1) + 0..3 and + 8
      const char* const vrd = vt + (4 * half + ((lane & 15) >> 2)) * SVROW + (16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
#pragma unroll
      for (int mt4 = 0; mt4 < 4; ++mt4) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const char* pv = vrd + 16 * u * SVROW + 64 * mt4;
          const u32x2 r0 = read_tr(pv), r1 = read_tr(pv + 8 * SVROW);
          const u32x4 va = {r0[0], r0[1], r1[0], r1[1]};
          acc[mt4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                             __builtin_bit_cast(bf16x8, ph[u]), acc[mt4], 0, 0, 0);
          if (SPLIT)
            acc[mt4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va),
                                                               __builtin_bit_cast(bf16x8, pl[u]), acc[mt4], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) {
      store_tile(buf ^ 1);                          // its readers finished before the last barrier
      if (t + 2 < ntiles) load_tile(t + 2);
    }
    __syncthreads();
  }
  if (!active) return;
  lsum += __shfl_xor(lsum, 32);
  const int gh = hb * 32 + tok;
  if (gh >= a.G) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float* const orow = a.out + (((size_t)b * a.n_q + i) * a.H + (size_t)g * a.G + gh) * D;
#pragma unroll
  for (int mt4 = 0; mt4 < 4; ++mt4)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 o = {acc[mt4][4 * r4], acc[mt4][4 * r4 + 1], acc[mt4][4 * r4 + 2], acc[mt4][4 * r4 + 3]};
      *(f32x4*)(orow + 32 * mt4 + crow(lane, 4 * r4)) = o * inv;
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
