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
// workgroup per CU.  The stages are double-buffered in LDS (one barrier per stage) and the global loads
// run two stages ahead in two register buffers.  MFMA v_mfma_f32_32x32x16_bf16 with operands from LDS:
// A = rows of X (16-byte reads, 144-byte row pitch); W is kept in its own [k][column] layout (576-byte
// row pitch) and each B operand (8 consecutive k of one column) comes from two LDS transpose reads,
// which on gfx950 hand each lane of a 16-lane group one column of a 4-row x 16-column block.
// Tile order: the workgroups of one token tile (all targets) are adjacent in dispatch order and land
// on one XCD, so they share that tile's X rows through the XCD's L2.

#include "hs_common.hpp"
#include "hs_internal.hpp"

namespace hs {

namespace {
constexpr int BM = 256, BN = 256, BK = 64, NT = 512;
constexpr int AROW = BK * 2 + 16;               // 144 B per X row in LDS
constexpr int WROW = 576;                       // bytes per k row of W (256 columns) in LDS
constexpr int STAGE = BM * AROW + BK * WROW;
constexpr int EPI = 8 * 64 * 128 * 2;           // per-wave 64 x 128 bf16 staging
constexpr int SMEM = 2 * STAGE > EPI ? 2 * STAGE : EPI;
constexpr int APT = BM * BK * 2 / 16 / NT;      // X pieces per thread per stage (4)
constexpr int BPT = BK * BN * 2 / 16 / NT;      // W pieces per thread per stage (4)
static_assert(APT == 4 && BPT == 4, "load split");

__device__ __forceinline__ int crow(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
__device__ __forceinline__ u32x2 read_tr(const char* p) {      // LDS transpose read of 4 k rows x 16 columns per 16 lanes
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p)));
}

struct Regs { u32x4 a[APT], b[BPT]; };
}  // namespace

__global__ __launch_bounds__(NT) void bridge_kernel(BridgeArgs a) {
  __shared__ __align__(16) char smem[SMEM];
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

  auto load = [&](Regs& r, int s) {                               // stage s; past the last: stage S - 1 again
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
  auto store = [&](const Regs& r, int buf) {
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
  f32x16 acc[2][4] = {};
  auto compute = [&](int buf) {
    const char* const As = smem + buf * STAGE;
    const char* const Bs = As + BM * AROW;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      s16x8 av[2], bv[4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        av[i] = *(const s16x8*)(As + (64 * wm + 32 * i + (lane & 31)) * AROW + (16 * s + 8 * (lane >> 5)) * 2);
#pragma unroll
      for (int j = 0; j < 4; ++j) {                               // k = 16 s + 8 (lane >> 5) + 0..7, column 128 wn + 32 j + (lane & 31)
        const char* p = Bs + (16 * s + 8 * (lane >> 5) + ((lane & 15) >> 2)) * WROW +
                        (128 * wn + 32 * j + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;
        const u32x2 lo = read_tr(p), hi = read_tr(p + 4 * WROW);
        const u32x4 q = {lo[0], lo[1], hi[0], hi[1]};
        bv[j] = __builtin_bit_cast(s16x8, q);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
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
  Regs r0, r1;
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

  // ---- epilogue: this wave holds rows 64 wm + [0, 64) of head block (tgt, wn)
  const int blk = 2 * tgt + wn;
  char* const ep = smem + wave * (64 * 128 * 2);
  const int64_t t0 = m0 + 64 * wm;                               // first token of this wave's rows
  auto orow = [&](int rl) -> int64_t { return a.rows ? a.rows[t0 + rl] : a.row_offset + t0 + rl; };
  if (a.fp8) {
    float* sc = a.scale[blk];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) am = fmaxf(am, fabsf(acc[i][j][r]));
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
        float scale = am / 448.0f;                                   // correctly rounded
        if (scale == 0.f) scale = 1.f;
        const int rl = 32 * i + crow(lane, r);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          ep[rl * 128 + 32 * j + (lane & 31)] = (char)f32_to_e4m3_rne(acc[i][j][r] / scale);
        if ((lane & 31) == 0 && t0 + rl < a.T) sc[orow(rl)] = scale;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    char* dst = (char*)a.out[blk];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int p = lane + 64 * i, rl = p >> 3, c = p & 7;
      if (t0 + rl < a.T) *(u32x4*)(dst + orow(rl) * 128 + c * 16) = *(const u32x4*)(ep + rl * 128 + c * 16);
    }
  } else {
    uint16_t* e16 = (uint16_t*)ep;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          e16[(32 * i + crow(lane, r)) * 128 + 32 * j + (lane & 31)] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    char* dst = (char*)a.out[blk];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int p = lane + 64 * i, rl = p >> 4, c = p & 15;
      if (t0 + rl < a.T) *(u32x4*)(dst + orow(rl) * 256 + c * 16) = *(const u32x4*)(ep + rl * 256 + c * 16);
    }
  }
}

hipError_t launch_bridge(const BridgeArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.T + BM - 1) / BM), a.n_targets);
  hipLaunchKernelGGL(bridge_kernel, grid, dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs
