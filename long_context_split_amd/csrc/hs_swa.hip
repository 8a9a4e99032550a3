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
// Two forms share the tile step (swa_tile).  bf16 caches with windows up to 154 rows take the ring
// form (swa_ring_kernel, further down): one workgroup per CU walks a range of tokens with its K/V
// tiles held in an LDS ring.  E4M3 caches and wider windows take the per-group form described here:
// one wave per query token and block of 32 query heads of one KV head, 4 waves (4 consecutive
// tokens) per workgroup and two workgroups per CU (at most 256 VGPRs per wave), so one workgroup's
// Q loads, first tiles and output stores overlap the other's tile work.  The 4 bands overlap
// almost entirely, so the workgroup walks their union
// in 32-row tiles: each tile is loaded once by all threads (next tile in registers while the
// current one is used), stored in LDS as bf16 [token][d] for K and V (E4M3 converted on the way),
// and every wave applies its own band as a mask.  S^T = K Q^T and O^T += V^T P^T run on bf16 MFMA
// with an online softmax in log2 units; the V^T operand comes from two LDS transpose reads (4 rows
// each, the token order of the P operand).
// Bands overlap between neighbouring workgroups too, so K/V rows come mostly from L2; the kernel's
// HBM traffic is Q in and O out.  O leaves through a per-wave LDS staging area as whole 128-byte pieces
// of head rows (float32, 32 d per row and round; bf16, 64 d per row and round, when the caller asks for
// a bf16 output).

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

namespace {

constexpr int SKROW = 272;                         // K tile row: 256 B + 16 B pad (16-byte operand reads)
constexpr int SVROW = 288;                         // V tile row: 256 B + 32 B pad (4-row transpose reads)
constexpr int SBUF = 32 * SKROW + 32 * SVROW;      // one tile: K then V (bf16)
constexpr int OPITCH = 36;                         // output staging: floats per head row (32 d + 4 pad)
constexpr int OPITCH2 = 68;                        // bf16 output staging: 64 d + 4 pad

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
// LDS transpose read: lane L of each 16-lane group gets column L & 15 of the 4 x 16 block whose row
// (L & 15) >> 2, columns 4 (L & 3) .. + 3 it addresses
__device__ __forceinline__ u32x2 read_tr(const char* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p)));
}

}  // namespace

// One 32-row tile of a wave's band: S^T = K Q^T from the LDS K tile, the online softmax update (log2
// units; mask bit t: tile row t is inside the band, at least one bit set), O^T += V^T P^T from two
// transpose reads of the V tile.  ksl / vsl: per-row K scale x softmax scale and V scale (E4M3), unused for bf16.
template <bool FP8>
__device__ __forceinline__ void swa_tile(const char* kt, const char* vt, uint32_t mask, const s16x8 (&qv)[8],
                                         const float* ksl, const float* vsl, float sl2, float& m, float& lsum,
                                         f32x16 (&acc)[4], int lane) {
  constexpr bool SPLIT = !FP8;                      // bf16 cache: P as bf16 hi + lo
  const int tok = lane & 31, half = lane >> 5;
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
      const float f = FP8 ? ksl[tb + r] : sl2;
      if (FP8) vs[4 * k4 + r] = vsl[tb + r];
      x[4 * k4 + r] = ((mask >> (tb + r)) & 1u) ? s[4 * k4 + r] * f : -INFINITY;
    }
  }
  float mt = x[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mt = fmaxf(mt, x[r]);
  mt = xor32_max(mt);                               // finite: the mask holds at least one row
  // lazy rescale: a head's reference m moves only when the tile's max exceeds it by more than TAU,
  // so p = 2^(x - m) <= 2^TAU and most tiles skip the rescale of acc (the first tile: m = -inf)
  constexpr float TAU = 8.f;
  const bool need = mt > m + TAU;                   // same for both lanes of a head
  if (__ballot(need)) {
    const float mn = need ? mt : m;
    const float alpha = exp2f(m - mn);
    lsum *= alpha;
#pragma unroll
    for (int mt4 = 0; mt4 < 4; ++mt4) acc[mt4] *= alpha;
    m = mn;
  }
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p[r] = exp2_fast(x[r] - m);
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

template <int KVT, int NW>
__global__ __launch_bounds__(64 * NW, 2) void swa_attn_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr int SB = (FP8 ? 1 : 2) * D;             // bytes per cache row
  constexpr int PPR = SB / 16;                      // 16-byte pieces per row
  constexpr int PPT = 2 * 32 * PPR / NT;            // 16-byte pieces per thread per tile (K and V)
  static_assert(PPT >= 1 && PPT * NT == 2 * 32 * PPR, "a tile's K and V pieces split evenly over the threads");
  constexpr int STAGE = NW * 32 * OPITCH2 * 4;               // output staging (OPITCH2 > OPITCH)
  constexpr int SMEM = 2 * SBUF > STAGE ? 2 * SBUF : STAGE;
  __shared__ __align__(16) char smem[SMEM];
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
    if (mask) swa_tile<FP8>(kt, vt, mask, qv, scl[buf][0], scl[buf][1], sl2, m, lsum, acc, lane);  // uniform over the wave
    if (t + 1 < ntiles) {
      store_tile(buf ^ 1);                          // its readers finished before the last barrier
      if (t + 2 < ntiles) load_tile(t + 2);
    }
    __syncthreads();
  }
  if (!active) return;
  lsum = xor32_add(lsum);
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  // ---- output: the wave's 32 heads go through its own LDS area (the tiles are dead after the loop's
  // last barrier) and leave as whole 128-byte pieces of head rows: 32 d per round as float32, 64 d
  // (two accumulator blocks) per round as bf16
  const int nh = min(32, a.G - hb * 32);                          // heads of this block that exist
  const size_t oel = (((size_t)b * a.n_q + i) * a.H + (size_t)g * a.G + hb * 32) * D;   // first element
  auto wave_fence = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  if (a.out_bf16) {
    float* const ob = (float*)smem + wave * (32 * OPITCH2);
    uint16_t* const obase16 = (uint16_t*)a.out + oel;
#pragma unroll
    for (int mp = 0; mp < 2; ++mp) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x16& c = acc[2 * mp + hf];
          const f32x4 o = {c[4 * r4], c[4 * r4 + 1], c[4 * r4 + 2], c[4 * r4 + 3]};
          *(f32x4*)(ob + tok * OPITCH2 + 32 * hf + crow(lane, 4 * r4)) = o * inv;
        }
      wave_fence();
#pragma unroll
      for (int k = 0; k < 4; ++k) {                               // head 8 k + lane / 8, d octet lane % 8
        const int hd = 8 * k + (lane >> 3), pc = lane & 7;
        const f32x4 x0 = *(const f32x4*)(ob + hd * OPITCH2 + 8 * pc), x1 = *(const f32x4*)(ob + hd * OPITCH2 + 8 * pc + 4);
        const u32x4 w = {pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]), pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
        if (hd < nh) *(u32x4*)(obase16 + (size_t)hd * D + 64 * mp + 8 * pc) = w;
      }
      wave_fence();                                               // reads done before the next round's writes
    }
    return;
  }
  float* const ob = (float*)smem + wave * (32 * OPITCH);
  float* const obase = a.out + oel;
#pragma unroll
  for (int mt4 = 0; mt4 < 4; ++mt4) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 o = {acc[mt4][4 * r4], acc[mt4][4 * r4 + 1], acc[mt4][4 * r4 + 2], acc[mt4][4 * r4 + 3]};
      *(f32x4*)(ob + tok * OPITCH + crow(lane, 4 * r4)) = o * inv;
    }
    wave_fence();
#pragma unroll
    for (int k = 0; k < 4; ++k) {                                 // head 8 k + lane / 8, d quad lane % 8
      const int hd = 8 * k + (lane >> 3), pc = lane & 7;
      if (hd < nh) *(f32x4*)(obase + (size_t)hd * D + 32 * mt4 + 4 * pc) = *(const f32x4*)(ob + hd * OPITCH + 4 * pc);
    }
    wave_fence();                                                 // reads done before the next block's writes
  }
}


// ---------------------------------------------------------------- ring form (bf16 caches)
//
// One workgroup of NW waves walks a contiguous range of a list's query tokens in groups of NW (one
// token per wave).  The 32-row K/V tiles sit in LDS at absolute positions (tile T holds rows 32 T ..
// 32 T + 31, in slot T mod RING): a group's bands span at most RING - 1 tiles, and the next group,
// NW rows further on, needs at most one tile more, which is loaded during the current group and
// written into the one slot the current group does not read.  So each tile is loaded once per
// workgroup, the next group's Q rows are in flight while the current group computes, and a group
// costs one barrier.  Each wave's band and online softmax are those of the per-group form above.
constexpr int RING = 7;                             // tile slots
constexpr int RING_STG = 32 * OPITCH * 4;           // per-wave output staging: 32 rows x 32 floats (or 64 bf16) + pad
constexpr int RING_NW = 8;                          // waves (query tokens per group)

template <int NW, bool OB16>
__global__ __launch_bounds__(64 * NW, 1) void swa_ring_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int PPR = 2 * D / 16;                   // 16-byte pieces per bf16 row
  constexpr int PPT = 2 * 32 * PPR / NT;            // 16-byte pieces per thread per tile (K and V)
  static_assert(PPT >= 1 && PPT * NT == 2 * 32 * PPR, "a tile's K and V pieces split evenly over the threads");
  static_assert(NW <= 32, "a group advances by at most one tile");
  __shared__ __align__(16) char smem[RING * SBUF + NW * RING_STG];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int list = blockIdx.y, hb = blockIdx.z;
  const int g = list % a.n_kv, b = list / a.n_kv;
  const int tok = lane & 31;
  const int Lb = a.seq_len[b];
  const int i0 = blockIdx.x * a.chunk;              // < n_q (grid), a.chunk a multiple of NW
  const int i1 = min(i0 + a.chunk, a.n_q);
  const int ng = (i1 - i0 + NW - 1) / NW;
  const int p0 = Lb - a.n_q;                        // cache row of query token 0 (>= 0, checked on the host)
  const int w = a.window;
  // tiles holding the bands of group j: rows max(0, first position - w + 1) .. last position
  auto t_lo = [&](int j) { return max(0, p0 + i0 + NW * j - w + 1) >> 5; };
  auto t_hi = [&](int j) { return (p0 + min(i0 + NW * j + NW, i1) - 1) >> 5; };

  const int64_t rs = a.row_start[b];
  const size_t rstride = (size_t)a.n_kv * 2 * D;
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * 2 * D;
  const char* vbase = (const char*)a.v + ((size_t)rs * a.n_kv + g) * 2 * D;
  const float sl2 = a.scale_log2;
  const int head = hb * 32 + tok;                   // heads past G read head 0's row, never stored
  const uint16_t* const qb = (const uint16_t*)a.q + ((size_t)b * a.n_q * a.H + (size_t)g * a.G + (head < a.G ? head : 0)) * D;
  auto load_q = [&](int i, s16x8 (&qr)[8]) {        // B operand: d = 16 st + 8 half
    const uint16_t* qrow = qb + (size_t)i * a.H * D;
#pragma unroll
    for (int st = 0; st < 8; ++st) qr[st] = *(const s16x8*)(qrow + 16 * st + 8 * (lane >> 5));
  };
  // piece q = tid + NT j of a tile: q < 32 PPR a K piece, else a V piece (row q' / PPR, piece q' % PPR);
  // rows past the cache clamp to its last row (never inside a band)
  auto load_tile = [&](int T, u32x4 (&r)[PPT]) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int q = tid + NT * j, isv = q >= 32 * PPR, pc = q % (32 * PPR);
      const int row = min(32 * T + pc / PPR, Lb - 1);
      r[j] = *(const u32x4*)((isv ? vbase : kbase) + (size_t)row * rstride + 16 * (pc % PPR));
    }
  };
  auto store_tile = [&](int T, const u32x4 (&r)[PPT]) {
    char* const base = smem + (T % RING) * SBUF;
#pragma unroll
    for (int j = 0; j < PPT; ++j) {
      const int q = tid + NT * j, isv = q >= 32 * PPR, pc = q % (32 * PPR), ptok = pc / PPR;
      *(u32x4*)(base + (isv ? 32 * SKROW + ptok * SVROW : ptok * SKROW) + 16 * (pc % PPR)) = r[j];
    }
  };

  {                                                 // the first group's tiles, loaded together
    const int lo0 = t_lo(0), hi0 = t_hi(0);
    u32x4 r0[RING - 1][PPT];
#pragma unroll
    for (int u = 0; u < RING - 1; ++u) load_tile(min(lo0 + u, hi0), r0[u]);
#pragma unroll
    for (int u = 0; u < RING - 1; ++u)
      if (lo0 + u <= hi0) store_tile(lo0 + u, r0[u]);
  }
  s16x8 qv[8], qn[8];
  load_q(min(i0 + wave, i1 - 1), qv);
  __syncthreads();
  // The first group's Q rows are waited for here, once: with a load still pending on the loop's entry
  // edge, the wait counts at the loop's first MFMAs would cover the previous group's output stores
  // in every later group.
#pragma unroll
  for (int st = 0; st < 8; ++st) asm volatile("" ::"v"(qv[st]));

  const int nh = min(32, a.G - hb * 32);            // heads of this block that exist
  float* const ob = (float*)(smem + RING * SBUF + wave * RING_STG);
  auto wave_fence = [] {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  u32x4 rn[PPT];
  for (int j = 0; j < ng; ++j) {
    // A wave past the range's last token computes that token again and writes the same bytes to the
    // same addresses as the wave that owns it, and lanes of heads past G write head nh - 1's bytes:
    // every wave then issues the same stores on every path, so the waits for the next group's loads
    // can be counted exactly and never include this group's output stores.
    const int i = min(i0 + NW * j + wave, i1 - 1);
    const int hi = t_hi(j);
    const int hn = j + 1 < ng ? t_hi(j + 1) : hi;
    load_tile(hn, rn);                              // the next group's new tile (a resident one otherwise)
    load_q(min(i0 + NW * (j + 1) + wave, i1 - 1), qn);   // the next group's Q rows
    const int pos = p0 + i, lo = max(0, pos - w + 1);
    float m = -INFINITY, lsum = 0.f;
    f32x16 acc[4] = {};
    for (int T = lo >> 5; T <= pos >> 5; ++T) {
      const char* const kt = smem + (T % RING) * SBUF;
      const int base = 32 * T, first = max(lo - base, 0), last = min(pos - base, 31);
      const uint32_t mask = (last >= 31 ? ~0u : (1u << (last + 1)) - 1u) & ~((1u << first) - 1u);
      swa_tile<false>(kt, kt + 32 * SKROW, mask, qv, nullptr, nullptr, sl2, m, lsum, acc, lane);
    }
    // tile hn's slot held tile hn - RING, below this group's first tile: no wave reads it now
    if (hn > hi) store_tile(hn, rn);
#pragma unroll
    for (int st = 0; st < 8; ++st) qv[st] = qn[st];
    lsum = xor32_add(lsum);
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    // output through the wave's staging area as whole 128-byte pieces of head rows: float32, 32 d
    // per round (pitch OPITCH floats); bf16, 64 d per round (pitch 72 bf16), rounded to nearest even
    const size_t oel = (((size_t)b * a.n_q + i) * a.H + (size_t)g * a.G + hb * 32) * D;
    if constexpr (OB16) {
      uint16_t* const ob16 = (uint16_t*)ob;
      uint16_t* const obase16 = (uint16_t*)a.out + oel;
#pragma unroll
      for (int mp = 0; mp < 2; ++mp) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x16& c = acc[2 * mp + hf];
            const f32x4 o = f32x4{c[4 * r4], c[4 * r4 + 1], c[4 * r4 + 2], c[4 * r4 + 3]} * inv;
            *(u32x2*)(ob16 + tok * 72 + 32 * hf + crow(lane, 4 * r4)) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          }
        wave_fence();
#pragma unroll
        for (int k = 0; k < 4; ++k) {                             // head 8 k + lane / 8, d octet lane % 8
          const int hd = min(8 * k + (lane >> 3), nh - 1), pc = lane & 7;
          *(u32x4*)(obase16 + (size_t)hd * D + 64 * mp + 8 * pc) = *(const u32x4*)(ob16 + hd * 72 + 8 * pc);
        }
        wave_fence();                                             // reads done before the next round's writes
      }
    } else {
      float* const obase = a.out + oel;
#pragma unroll
      for (int mt4 = 0; mt4 < 4; ++mt4) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 o = {acc[mt4][4 * r4], acc[mt4][4 * r4 + 1], acc[mt4][4 * r4 + 2], acc[mt4][4 * r4 + 3]};
          *(f32x4*)(ob + tok * OPITCH + crow(lane, 4 * r4)) = o * inv;
        }
        wave_fence();
#pragma unroll
        for (int k = 0; k < 4; ++k) {                             // head 8 k + lane / 8, d quad lane % 8
          const int hd = min(8 * k + (lane >> 3), nh - 1), pc = lane & 7;
          *(f32x4*)(obase + (size_t)hd * D + 32 * mt4 + 4 * pc) = *(const f32x4*)(ob + hd * OPITCH + 4 * pc);
        }
        wave_fence();
      }
    }
    __syncthreads();
  }
}

template <int KVT>
static hipError_t launch_swa_t(const AttnArgs& a, hipStream_t st) {
  constexpr int NW = 4;                             // tokens per workgroup (two workgroups per CU)
  dim3 grid((a.n_q + NW - 1) / NW, a.n_lists, (a.G + 31) / 32);
  hipLaunchKernelGGL((swa_attn_kernel<KVT, NW>), grid, dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

bool swa_ring_fits(int window) { return window >= 1 && (30 + window + RING_NW - 1) / 32 + 1 <= RING - 1; }

hipError_t launch_swa_attn(const AttnArgs& a, int kvt, hipStream_t st) {
  if (a.q_f32 || a.window < 1 || a.n_q < 1) return hipErrorInvalidValue;
  if (a.chunk > 0) {                                // ring form: a.chunk query tokens per workgroup
    if (kvt != KV_BF16 || a.chunk % RING_NW || !swa_ring_fits(a.window)) return hipErrorInvalidValue;
    dim3 grid((a.n_q + a.chunk - 1) / a.chunk, a.n_lists, (a.G + 31) / 32);
    if (a.out_bf16)
      hipLaunchKernelGGL((swa_ring_kernel<RING_NW, true>), grid, dim3(64 * RING_NW), 0, st, a);
    else
      hipLaunchKernelGGL((swa_ring_kernel<RING_NW, false>), grid, dim3(64 * RING_NW), 0, st, a);
    return hipGetLastError();
  }
  if (kvt == KV_BF16) return launch_swa_t<KV_BF16>(a, st);
  if (kvt == KV_FP8) return launch_swa_t<KV_FP8>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace hs
