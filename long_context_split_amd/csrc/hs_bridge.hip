// KV Bridging projection with fused cache-storage epilogue (gfx950 MFMA GEMM).
//
// ithome page "小米公开 MiMo-V3 核心架构 HySparse2", KV-sharing overview: each
// Cross-Decoder full-attention layer builds its own K/V from the input hidden
// state of the matching Self-Decoder full layer, with projections of its own;
// prefill runs a single full-attention layer, so every target bridges from the
// same source X (prefill early-exit paragraphs).  Per target l:
//   K_l = X W_k[l],  V_l = X W_v[l]        X bf16 [T, Dm], W bf16 [Dm, 128]
// stored at cache rows row_offset + t, as bf16 (round to nearest even) or as
// OCP E4M3FN codes with one float32 scale per row (scale = amax / 448).
//
// Workgroup tile: 256 tokens x 256 columns (one target: K's 128 columns, then V's), K-stage 64, 8 waves
// each owning 64 rows x 128 columns = one head block, so a row's amax is reduced inside one wave; one
// workgroup per CU.  Chunks too short to give every CU a 256-token tile (a prefill chunk of 8192
// tokens with 4 targets makes 128) take 128-token tiles, 32 rows per wave.  The stages are double-buffered in LDS (one barrier per stage) and the global loads
// run two stages ahead in two register buffers.  MFMA v_mfma_f32_32x32x16_bf16 with operands from LDS:
// A = rows of X (16-byte reads, 144-byte row pitch); W is kept in its own [k][column] layout (576-byte
// row pitch) and each B operand (8 consecutive k of one column) comes from two LDS transpose reads,
// which on gfx950 hand each lane of a 16-lane group one column of a 4-row x 16-column block.
// Tile order: the workgroups of one token tile (all targets) are adjacent in dispatch order and land
// on one XCD, so they share that tile's X rows through the XCD's L2.

// Epilogue in registers: the row amax by DPP and a lane swap, x / scale correctly rounded, E4M3 by the
// hardware packed conversion (equal to the software RNE conversion for
// every finite |y| < 448 that does not round to zero, the range used here; a zero magnitude is stored
// as +0), then a byte (or bf16) transpose inside each quad of lanes so that every store writes whole
// cache rows.

#include "hs_common.hpp"
#include "hs_internal.hpp"

namespace hs {

namespace {
constexpr int BN = 256, BK = 64, NT = 512;
constexpr int AROW = BK * 2 + 16;               // 144 B per X row in LDS
constexpr int WROW = 576;                       // bytes per k row of W (256 columns) in LDS
constexpr int BPT = BK * BN * 2 / 16 / NT;      // W pieces per thread per stage (4)
static_assert(BPT == 4, "load split");

__device__ __forceinline__ int crow(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ u32x2 read_tr(const char* p) {      // LDS transpose read of 4 k rows x 16 columns per 16 lanes
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p)));
}

template <int APT> struct Regs { u32x4 a[APT], b[BPT]; };
}  // namespace

// BM = 256 tokens per workgroup (8 waves of 64 rows x 128 columns), or 128 (32 rows each) when the
// 256-token tiles would leave CUs idle
template <int BM>
__global__ __launch_bounds__(NT) void bridge_kernel(BridgeArgs a) {
  constexpr int STAGE = BM * AROW + BK * WROW;
  constexpr int APT = BM * BK * 2 / 16 / NT;                     // X pieces per thread per stage (4 or 2)
  constexpr int RW = BM / 4, NI = RW / 32;                        // rows per wave, its 32-row blocks
  __shared__ __align__(16) char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // tile order: groups of 8 token tiles x all targets are consecutive in dispatch order (x fastest), and
  // dispatch id % 8 picks the XCD, so a tile's targets run together on one XCD
  const int nt = a.n_targets, ntiles = gridDim.x;
  int xt, tgt;
  {
    const int lin = blockIdx.y * ntiles + blockIdx.x;             // the hardware's dispatch order
    const int grp = 8 * nt;                                       // ids per group: 8 tiles x nt targets
    const int g = lin / grp, w = lin % grp;
    if ((g + 1) * grp <= ntiles * nt) { xt = 8 * g + (w & 7); tgt = w >> 3; }
    else { xt = lin / nt; tgt = lin % nt; }                       // the last partial group: plain order
  }
  const int64_t m0 = (int64_t)xt * BM;
  const uint16_t* wk = a.w[2 * tgt];
  const uint16_t* wv = a.w[2 * tgt + 1];
  const int Dm = a.Dm;
  const int S = Dm / BK;                                          // stages (>= 1)

  auto load = [&](Regs<APT>& r, int s) {                               // stage s; past the last: stage S - 1 again
    const int k0 = min(s, S - 1) * BK;
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int p = tid + NT * i, row = p >> 3, c = p & 7;
      const int64_t gr = min(m0 + row, a.T - 1);                  // rows past T are never stored
      r.a[i] = *(const u32x4*)(a.x + gr * Dm + k0 + c * 8);
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i) {                               // k row p >> 5, 16-byte column chunk p & 31
      const int p = tid + NT * i, kr = p >> 5, c = p & 31;
      r.b[i] = *(const u32x4*)((c < 16 ? wk : wv) + (int64_t)(k0 + kr) * D + (c & 15) * 8);
    }
  };
  auto store = [&](const Regs<APT>& r, int buf) {
    char* const As = smem + buf * STAGE;
    char* const Bs = As + BM * AROW;
#pragma unroll
    for (int i = 0; i < APT; ++i) {
      const int p = tid + NT * i;
      *(u32x4*)(As + (p >> 3) * AROW + (p & 7) * 16) = r.a[i];
    }
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int p = tid + NT * i;
      *(u32x4*)(Bs + (p >> 5) * WROW + (p & 31) * 16) = r.b[i];
    }
  };
  f32x16 acc[NI][4] = {};
  auto compute = [&](int buf) {
    const char* const As = smem + buf * STAGE;
    const char* const Bs = As + BM * AROW;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      s16x8 av[NI], bv[4];
#pragma unroll
      for (int i = 0; i < NI; ++i)
        av[i] = *(const s16x8*)(As + (RW * wm + 32 * i + (lane & 31)) * AROW + (16 * s + 8 * (lane >> 5)) * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {                               // k = 16 s + 8 (lane >> 5) + 0..7, column 128 wn + 32 j + (lane & 31)
        const char* p = Bs + (16 * s + 8 * (lane >> 5) + ((lane & 15) >> 2)) * WROW +
                        (128 * wn + 32 * j + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
        const u32x2 lo = read_tr(p), hi = read_tr(p + 4 * WROW);
        const u32x4 q = {lo[0], lo[1], hi[0], hi[1]};
        bv[j] = __builtin_bit_cast(s16x8, q);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                               __builtin_bit_cast(bf16x8, bv[j]), acc[i][j], 0, 0, 0);
    }
  };

  // Stage s is computed from LDS buffer s % 2.  Iteration s stores stage s + 1 (loaded two
  // iterations earlier) into the other buffer, loads stage s + 3 into the registers it just
  // emptied, computes stage s, and ends with the one barrier of the stage.  Register buffers R0 / R1
  // alternate (the loop handles two stages per pass, so each wait is a static count); loads past the
  // last stage re-read it; storing them (unconditionally: a branch around the store would make the
  // compiler wait for every load in flight) writes a buffer no later stage reads.
  Regs<APT> r0, r1;
  load(r0, 0);
  load(r1, 1);
  store(r0, 0);
  load(r0, 2);
  __syncthreads();
  for (int s = 0; s < S; s += 2) {
    store(r1, 1);
    load(r1, s + 3);
    compute(0);
    __syncthreads();
    if (s + 1 >= S) break;
    store(r0, 0);
    load(r0, s + 4);
    compute(1);
    __syncthreads();
  }

  // ---- epilogue: this wave holds rows RW wm + [0, RW) of head block (tgt, wn), all in registers.
  // Lane l holds, for rows 32 i + crow(l, r), the columns 32 j + (l & 31), j = 0..3.  Within a quad of
  // lanes 4 m + t, a byte (or bf16) transpose leaves lane 4 m + t with columns 32 t + 4 m .. + 3 of the
  // row, so one store per (i, r) writes two whole rows (lanes 0..31 one row, 32..63 the other).
  const int blk = 2 * tgt + wn;
  const int64_t t0 = m0 + RW * wm;                              // first token of this wave's rows
  auto orow = [&](int rl) -> int64_t { return a.rows ? a.rows[t0 + rl] : a.row_offset + t0 + rl; };
  char* const dst = (char*)a.out[blk];
  const int qt = lane & 3, qm = (lane & 31) >> 2;
  // byte selectors of v_perm_b32 {hi, lo}: byte qt of lo -> byte 0, byte qt of hi -> byte 1 (0x0C: zero)
  const uint32_t sel_lo = (uint32_t)qt | (uint32_t)(4 + qt) << 8 | 0x0C0C0000u;
  const uint32_t sel_hi = 0x00000C0Cu | (uint32_t)qt << 16 | (uint32_t)(4 + qt) << 24;
  auto quad = [](uint32_t w, int k) -> uint32_t {               // w of quad lane k (quad_perm [k, k, k, k])
    switch (k) {
      case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x00, 0xF, 0xF, false);
      case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0x55, 0xF, 0xF, false);
      case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xAA, 0xF, 0xF, false);
      default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)w, 0xFF, 0xF, 0xF, false);
    }
  };
  if (a.fp8) {
    float* const sc = a.scale[blk];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) am = fmaxf(am, fabsf(acc[i][j][r]));
        am = half_max_dpp(am);                                         // the row's 32 lanes
        float scale = am / 448.0f;                                   // correctly rounded
        if (scale == 0.f) scale = 1.f;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) y[j] = acc[i][j][r] / scale;     // correctly rounded
        // bytes j = 0..3 (|y| <= 448 (1 + 2^-24) here)
        const uint32_t w = e4m3x4_hw(y[0], y[1], y[2], y[3]);
        const uint32_t q0 = quad(w, 0), q1 = quad(w, 1), q2 = quad(w, 2), q3 = quad(w, 3);
        const uint32_t out = __builtin_amdgcn_perm(q1, q0, sel_lo) | __builtin_amdgcn_perm(q3, q2, sel_hi);
        const int rl = 32 * i + crow(lane, r);
        if (t0 + rl < a.T) {
          const int64_t orw = orow(rl);
          *(uint32_t*)(dst + orw * 128 + 32 * qt + 4 * qm) = out;
          if ((lane & 31) == 0) sc[orw] = scale;
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // p01 = bf16 of tiles (0, 1), p23 = tiles (2, 3); lane 4 m + t takes tile t of quad lanes 0..3
        const uint32_t p01 = f32_to_bf16_rne(acc[i][0][r]) | f32_to_bf16_rne(acc[i][1][r]) << 16;
        const uint32_t p23 = f32_to_bf16_rne(acc[i][2][r]) | f32_to_bf16_rne(acc[i][3][r]) << 16;
        uint32_t x[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t a01 = quad(p01, k), a23 = quad(p23, k);
          x[k] = qt >> 1 ? a23 : a01;
        }
        // half (qt & 1) of x[k] -> element k
        const uint32_t hs = (qt & 1) ? 0x07060302u : 0x05040100u;   // {hi.half, lo.half} byte pairs
        const uint32_t o0 = __builtin_amdgcn_perm(x[1], x[0], hs);
        const uint32_t o1 = __builtin_amdgcn_perm(x[3], x[2], hs);
        const int rl = 32 * i + crow(lane, r);
        if (t0 + rl < a.T) {
          uint32_t* d = (uint32_t*)(dst + orow(rl) * 256 + 64 * qt + 8 * qm);
          *(u32x2*)d = u32x2{o0, o1};
        }
      }
    }
  }
}

// Every float32 bit pattern: the bridge's E4M3 conversion (e4m3x4_hw) against f32_to_e4m3_rne on the
// finite values with |y| < 464; counts[0] += mismatches, counts[1] += values compared.
__global__ __launch_bounds__(256) void e4m3_check_kernel(unsigned long long* counts) {
  unsigned long long bad = 0, n = 0;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 4;
  for (uint64_t u0 = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; u0 < (1ull << 32); u0 += stride) {
    float y[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = __uint_as_float((uint32_t)(u0 + k));
    const uint32_t w = e4m3x4_hw(y[0], y[1], y[2], y[3]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = (uint32_t)(u0 + k) & 0x7FFFFFFFu;
      if (a >= 0x43E80000u) continue;                            // |y| >= 464, inf, NaN
      ++n;
      bad += ((w >> (8 * k)) & 0xFFu) != f32_to_e4m3_rne(y[k]);
    }
  }
  atomicAdd(counts, bad);
  atomicAdd(counts + 1, n);
}

__global__ void zero_u64_kernel(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

hipError_t launch_e4m3_check(unsigned long long* counts, hipStream_t st) {
  hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, st, counts, 2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(e4m3_check_kernel, dim3(4096), dim3(256), 0, st, counts);
  return hipGetLastError();
}

hipError_t launch_bridge(const BridgeArgs& a, hipStream_t st) {
  // 256-token tiles while they give every CU a workgroup, else 128-token tiles (twice the workgroups)
  if ((a.T + 255) / 256 * a.n_targets >= 256) {
    dim3 grid((unsigned)((a.T + 255) / 256), a.n_targets);
    hipLaunchKernelGGL(bridge_kernel<256>, grid, dim3(NT), 0, st, a);
  } else {
    dim3 grid((unsigned)((a.T + 127) / 128), a.n_targets);
    hipLaunchKernelGGL(bridge_kernel<128>, grid, dim3(NT), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace hs
