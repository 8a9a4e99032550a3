// Decode-time KV append through the bridge (gfx950).
//
// ithome page "小米公开 MiMo-V3 核心架构 HySparse2", KV-sharing overview and the
// prefill early-exit paragraphs: once generation starts the Cross-Decoder runs
// normally, so every new token's K and V for each target full layer are
// projected from the matching Self-Decoder hidden state with that layer's own
// weights, K_l = x W_k[l], V_l = x W_v[l], and stored in its cache.
//
// A decode step has few tokens (one per sequence), so the product is GEMV-
// shaped: the weights (n_targets x 2 x d_model x 128 bf16, 8 MB for 4 targets
// at d_model 4096) dominate the bytes.  Two kernels:
//   append_partial  split-K over d_model: workgroup (k slice of 128, head block)
//                   stages its weight slice transposed ([column][k]; each
//                   thread transposes one 8 x 8 block in registers and writes
//                   8 columns of 8 k values) and the tokens' x slice in LDS
//                   and multiplies them with
//                   v_mfma_f32_32x32x16_bf16 (32 tokens x 32 columns per wave);
//                   float32 partial sums to the workspace.
//   append_finish   one wave per (token, head block): sums the slices in a
//                   fixed order and stores the row exactly as the bridge does
//                   (bf16 round to nearest even, or E4M3 codes with the scale
//                   amax / 448) at the token's cache row.

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

namespace {

constexpr int KSL = 128;                  // d_model slice per workgroup
constexpr int PITCH = KSL * 2 + 16;       // LDS row pitch (bytes) of the staged slices
constexpr int NTOK = 32;                  // tokens per M tile

// byte offset of 8-k quad q of W^T column c: the quads are XOR-swizzled by the column's group of 8,
// which spreads the block-transposing writes (16 column groups, one quad) over the LDS banks
__device__ __forceinline__ int wq_off(int c, int q) { return c * PITCH + 16 * (q ^ ((c >> 3) & 15)); }

}  // namespace

// grid (n_slices, n_blocks, m_tiles), 256 threads: 4 waves x 32 columns of one head block
__global__ __launch_bounds__(256) void append_partial_kernel(AppendArgs a) {
  __shared__ __align__(16) char wt[128 * PITCH];                 // W slice transposed: [column][k]
  __shared__ __align__(16) char xs[NTOK * PITCH];                // x slice: [token][k]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = blockIdx.x, hb = blockIdx.y, mt = blockIdx.z;
  const int k0 = ks * KSL;
  const int kn = min(KSL, a.Dm - k0);                             // a multiple of 64
  const uint16_t* w = a.w[hb] + (size_t)k0 * 128;
  // W slice (kn rows of 128 bf16): thread (kg, cg) takes the 8 x 8 block of k rows 8 kg .. and
  // columns 8 cg .., rows past kn read as zero (clamped loads, no branch around them)
  {
    const int kg = tid >> 4, cg = tid & 15;
    u32x4 r[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = 8 * kg + i;
      r[i] = *(const u32x4*)(w + (size_t)min(k, kn - 1) * 128 + 8 * cg);
      if (k >= kn) r[i] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {                                 // column 8 cg + e: words (k, k + 1)
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t a0 = r[2 * j][e >> 1], a1 = r[2 * j + 1][e >> 1];
        o[j] = (e & 1) ? ((a0 >> 16) | (a1 & 0xFFFF0000u)) : ((a0 & 0xFFFFu) | (a1 << 16));
      }
      *(u32x4*)(wt + wq_off(8 * cg + e, kg)) = o;
    }
  }
  // x slice: NTOK tokens of this M tile (rows past n_tokens are zero)
  for (int p = tid; p < NTOK * (KSL / 8); p += 256) {
    const int t = p / (KSL / 8), k8 = (p % (KSL / 8)) * 8;
    const int64_t tok = (int64_t)mt * NTOK + t;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tok < a.T && k8 < kn) v = *(const u32x4*)(a.x + tok * a.Dm + k0 + k8);
    *(u32x4*)(xs + t * PITCH + k8 * 2) = v;
  }
  __syncthreads();
  // C[token][column] for columns 32 wave .. + 31: A = x rows, B = W^T rows (both k-contiguous)
  f32x16 c = {};
  const char* ab = xs + (lane & 31) * PITCH + (lane >> 5) * 16;
  const int bcol = 32 * wave + (lane & 31);
  for (int s = 0; s < kn / 16; ++s) {
    const s16x8 av = *(const s16x8*)(ab + 32 * s), bv = *(const s16x8*)(wt + wq_off(bcol, 2 * s + (lane >> 5)));
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
  }
  // partial [slice][block][m tile][token][128] float32: lane holds column (l & 31), tokens crow(lane, r)
  float* part = a.part + (((size_t)ks * a.n_blocks + hb) * a.m_tiles + mt) * NTOK * 128 + 32 * wave + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) part[crow(lane, r) * 128] = c[r];
}

// grid (ceil(n_tokens * n_blocks / 4)), 256 threads: one wave per (token, head block)
__global__ __launch_bounds__(256) void append_finish_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.T * a.n_blocks) return;
  const int64_t tok = item / a.n_blocks;
  const int hb = (int)(item % a.n_blocks);
  const int mt = (int)(tok / NTOK), t = (int)(tok % NTOK);
  const float* p = a.part + (((size_t)hb * a.m_tiles + mt) * NTOK + t) * 128 + 2 * lane;
  const size_t sstride = (size_t)a.n_blocks * a.m_tiles * NTOK * 128;
  float2 v = {0.f, 0.f};
  for (int s0 = 0; s0 < a.n_slices; s0 += 8) {                   // fixed order, 8 loads in flight
    float2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = *(const float2*)(p + (size_t)min(s0 + u, a.n_slices - 1) * sstride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < a.n_slices) { v.x += x[u].x; v.y += x[u].y; }
  }
  const int64_t row = a.rows[tok];
  if (a.fp8) {
    const float am = wave_max_dpp(fmaxf(fabsf(v.x), fabsf(v.y)));
    float scale = am / 448.0f;                                     // correctly rounded
    if (scale == 0.f) scale = 1.f;
    const uint32_t c0 = f32_to_e4m3_rne(v.x / scale), c1 = f32_to_e4m3_rne(v.y / scale);
    *(uint16_t*)((char*)a.out[hb] + row * 128 + 2 * lane) = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) a.scale[hb][row] = scale;
  } else {
    *(uint32_t*)((char*)a.out[hb] + row * 256 + 4 * lane) = f32_to_bf16_rne(v.x) | (f32_to_bf16_rne(v.y) << 16);
  }
}

void append_plan(int64_t n_tokens, int d_model, int n_targets, AppendArgs& a) {
  a.n_slices = (d_model + KSL - 1) / KSL;
  a.n_blocks = 2 * n_targets;
  a.m_tiles = (int)((n_tokens + NTOK - 1) / NTOK);
}

size_t append_workspace_bytes(const AppendArgs& a) {
  return (size_t)a.n_slices * a.n_blocks * a.m_tiles * NTOK * 128 * sizeof(float);
}

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(append_partial_kernel, dim3(a.n_slices, a.n_blocks, a.m_tiles), dim3(256), 0, st, a);
  const int64_t items = a.T * a.n_blocks;
  hipLaunchKernelGGL(append_finish_kernel, dim3((unsigned)((items + 3) / 4)), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs
