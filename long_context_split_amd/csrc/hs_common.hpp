// Device-side helpers shared by the libhysparse kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs {

constexpr int D = 128;          // head dimension (the only one supported)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// OCP E4M3FN code -> float32 (exact).  Normal codes move the 4-bit exponent
// (bias 7) into binary32's (bias 127) and the 3 mantissa bits to the top of
// its fraction; subnormal codes are m * 2^-9.  The two NaN codes are outside
// the cache contract and decode as 480.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t em = c & 0x7Fu;
  float v = (em >= 8u) ? __uint_as_float((em + (120u << 3)) << 20) : (float)em * 0x1p-9f;
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// Two floats -> two bf16 (round to nearest even; the conversion instruction, checked bit for bit
// against the rounding on the bits, ties and subnormals included) packed low-first in a word.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

// Four OCP E4M3FN codes (bytes of w, low first) -> four bf16 packed in two words (lo: bytes 0, 1;
// hi: bytes 2, 3), exact: every finite E4M3 value is a bf16 value.  gfx950's conversion instruction
// with unit scale (checked against the format definition on every non-NaN code).
__device__ __forceinline__ void e4m3x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// float32 -> OCP E4M3FN code: round to nearest, ties to the even mantissa,
// saturating at +-448, zero magnitude -> 0x00.  With e = max(floor(log2|y|), -6)
// the neighbours of |y| are multiples of 2^(e-3); q = rint(|y| * 2^(3-e)) is
// exact (power-of-two scaling) and the magnitude code is ((e+7)<<3) + q - 8.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float y) {
  uint32_t u = __float_as_uint(y);
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return (u >> 24 & 0x80u) | 0x7Eu;     // |y| >= 448 (inf too)
  int e = (int)(a >> 23) - 127;
  e = e < -6 ? -6 : e;
  float q = __builtin_rintf(__uint_as_float(a) * __uint_as_float((uint32_t)(127 + 3 - e) << 23));
  int mag = ((e + 7) << 3) + (int)q - 8;
  mag = mag > 0x7E ? 0x7E : mag;
  if (mag == 0) return 0u;
  return (u >> 24 & 0x80u) | (uint32_t)mag;
}

// Four float32 -> four E4M3 codes (byte k from y_k) by the hardware packed conversion
// (v_cvt_pk_fp8_f32, round to nearest even), a magnitude that rounds to zero stored as +0.  Equal to
// f32_to_e4m3_rne for every finite |y| < 464 (hs_e4m3_check compares all of them on the device);
// callers keep |y| below that.
__device__ __forceinline__ uint32_t e4m3x4_hw(float y0, float y1, float y2, float y3) {
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, (int)w, true);
  return w & ((((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u) | 0x7F7F7F7Fu);
}

// Order-preserving uint32 key of a float32 (finite values; -0 sorts below +0).
__device__ __forceinline__ uint32_t f32_key(float x) {
  uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// 2^x with the hardware instruction alone (v_exp_f32): inside the attention loops x is a logit
// minus a running maximum (<= 2^8 above it at most), and a probability below 2^-126 of the row's
// maximum may flush to zero; exp2f adds a rescaling for subnormal results that these loops do
// not need (five more instructions per element).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Orders a wave's own LDS writes before its later reads (and reads before later writes) of the
// same wave-private buffer.
// Read of cache rows that a pass streams once: a non-temporal load, so the lines do not
// displace reused data in the caches on their way (on a 2.1 GB pass: 370 -> 327 us).
__device__ __forceinline__ u32x4 load_stream(const void* p) { return __builtin_nontemporal_load((const u32x4*)p); }

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Combining v with the value of lane l ^ 32 (or l ^ 16) through v_permlane32_swap_b32
// (v_permlane16_swap_b32), vector-unit operations, instead of an LDS permute on the latency chain.
// With v in both operands the swap leaves v of lanes l and l ^ 32 (l ^ 16) in its two results, in
// an order that depends on the half, so only commutative combinations are formed: the sum equals
// v + __shfl_xor(v, 32) bit for bit.
__device__ __forceinline__ float xor32_add(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Maximum over each half of the wave (lanes 0-31, 32-63) without LDS: lane pairs, quads, half rows
// and rows of 16 by DPP, then the two rows of the half by the 16-lane swap.  Every lane gets the
// maximum of its half.
__device__ __forceinline__ float half_max_dpp(float v) {
  auto dpp = [](float x, int ctl) -> float {
    switch (ctl) {                                                // the control must be a constant
      case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // l ^ 1
      case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // l ^ 2
      case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));  // half-row mirror
      default: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, false)); // row mirror
    }
  };
#pragma unroll
  for (int c = 0; c < 4; ++c) v = fmaxf(v, dpp(v, c));
  return xor16_max(v);
}

// Maximum over the wave without LDS (every lane gets it).
__device__ __forceinline__ float wave_max_dpp(float v) { return xor32_max(half_max_dpp(v)); }

// Selection scores of the 32-token S tile a wave holds (S = Q K^T from v_mfma_f32_32x32x16_bf16:
// lane l has token l & 31 and the rows 8 (r / 4) + 4 (l >> 5) + (r & 3)): for each of the NQ query
// tokens of the 32 rows (tpw tokens of G = 32 / tpw rows each, or one token when tpw = 1), the sum
// over its rows of 2^(s f - lse2) in a fixed order.  f = softmax scale in log2 units (times the
// token's K scale for E4M3), lse2 = the row's log-sum-exp in log2 units (+inf for padding rows).
// Every pass that computes selection scores goes through here, so they agree bit for bit.
template <int NQ>
__device__ __forceinline__ void tile_scores(const f32x16& s, float f, const float (&lse2)[16], int tpw,
                                            float (&tv)[NQ]) {
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = exp2_fast(fmaf(s[r], f, -lse2[r]));
  if (tpw == 1) {
    float v = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) v += p[r];
    tv[0] = xor32_add(v);
  } else {
    float blk[4];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      blk[q4] = p[4 * q4] + p[4 * q4 + 1] + p[4 * q4 + 2] + p[4 * q4 + 3];
      blk[q4] = xor32_add(blk[q4]);
    }
#pragma unroll
    for (int t = 0; t < NQ; ++t) tv[t] = tpw == 4 ? blk[t] : blk[2 * t] + blk[2 * t + 1];
  }
}

// Clears runs of words with the whole grid (any grid shape): `lists` runs of `words` words,
// `stride` words apart.  No-op when ptr is null.
__device__ __forceinline__ void zero_words_grid(uint32_t* ptr, int64_t stride, int words, int lists) {
  if (!ptr) return;
  const int64_t total = (int64_t)lists * words;
  const int64_t nwg = (int64_t)gridDim.x * gridDim.y * gridDim.z;
  const int64_t wg = ((int64_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
  for (int64_t i = wg * blockDim.x + threadIdx.x; i < total; i += nwg * blockDim.x)
    ptr[(i / words) * stride + (i % words)] = 0u;
}

// Dense one-dimensional grids over ragged lists.  List l (sequence l / n_kv) owns
// max(min_items, ceil((L_b - min(sub, L_b)) / chunk)) consecutive items, lists in order, so a
// launch has exactly the items that have work and the hardware's round-robin spreads them evenly
// over the XCDs (a two-dimensional grid with early-exit blocks can leave one XCD a second round).
// Returns (list, index within the list) of `item`, or list = -1 past the last item.  uniform > 0:
// every list owns exactly `uniform` items (plain division, no loads).  Otherwise every thread of
// the workgroup must call it (it ends with a barrier).
__device__ inline void grid_item(const int32_t* seq_len, int n_kv, int n_lists, int chunk, int sub, int min_items,
                                 int uniform, int item, int& list, int& idx) {
  if (uniform > 0) {
    list = item / uniform < n_lists ? item / uniform : -1;
    idx = item % uniform;
    return;
  }
  __shared__ int s_li[2];
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    if (lane == 0) s_li[0] = -1;
    int base = 0;
    for (int l0 = 0; l0 < n_lists; l0 += 64) {
      const int l = l0 + lane;
      int cnt = 0;
      if (l < n_lists) {
        const int L = seq_len[l / n_kv];
        cnt = max(min_items, (L - min(sub, L) + chunk - 1) / chunk);
      }
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const int tot = __shfl(incl, 63);
      if (item < base + tot) {                                     // uniform over the wave
        const unsigned long long m = __ballot(item < base + incl);
        if (lane == __ffsll((long long)m) - 1) { s_li[0] = l; s_li[1] = item - (base + incl - cnt); }
        break;
      }
      base += tot;
    }
  }
  __syncthreads();
  list = s_li[0];
  idx = s_li[1];
}

// Split-K partials of one attention row: chunk c holds (m_c, l_c) at ml[c * mstride] (running max in
// log2 units, sum of 2^(s - m_c)) and acc_c = sum 2^(s - m_c) v at acc[c * astride].

// One wave's share of a row's partials, chunks c = c_first, c_first + step, ... < nch, combined in a
// single online pass (8 chunks in flight): running max m, l and o relative to it (lanes holding
// d = 2 lane, 2 lane + 1).  m = -inf if the wave had no chunk.  m and l are the same on every lane.
// Addresses are clamped to the first nld >= nch chunks rather than to nch, so the first loads need
// not wait for nch (a count read from memory) once c_first < nld is known: chunks past nch are
// replaced by empty parts whatever their memory holds.
struct MergePart {
  float m, l;
  float2 o;
};

__device__ inline MergePart merge_part_wave(const float* ml, size_t mstride, const float* acc, size_t astride,
                                            int c_first, int nch, int nld, int step, int lane) {
  MergePart r{-INFINITY, 0.f, make_float2(0.f, 0.f)};
  for (int c0 = c_first; c0 < nld; c0 += 8 * step) {
    float2 q[8], x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u * step, cc = min(c, nld - 1);
      q[u] = *(const float2*)(ml + (size_t)cc * mstride);
      x[u] = *(const float2*)(acc + (size_t)cc * astride + 2 * lane);
      if (c >= nch) { q[u] = make_float2(-INFINITY, 0.f); x[u] = make_float2(0.f, 0.f); }
    }
    float nm = r.m;
#pragma unroll
    for (int u = 0; u < 8; ++u) nm = fmaxf(nm, q[u].x);
    if (nm != -INFINITY) {
      const float al = exp2f(r.m - nm);
      r.l *= al;
      r.o.x *= al;
      r.o.y *= al;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float w = exp2f(q[u].x - nm);
        r.l += w * q[u].y;
        r.o.x += w * x[u].x;
        r.o.y += w * x[u].y;
      }
      r.m = nm;
    }
    if (c0 + 8 * step >= nch) break;
  }
  return r;
}

// sum_c 2^(m_c - l2) acc_c over c = c_first, c_first + step, ... < nch (l2 finite), lanes holding
// d = 2 lane and 2 lane + 1; 8 chunks in flight.
__device__ inline float2 merged_o(const float* ml, size_t mstride, const float* acc, size_t astride, int c_first,
                                  int nch, int step, float l2, int lane) {
  float2 o = make_float2(0.f, 0.f);
  for (int c0 = c_first; c0 < nch; c0 += 8 * step) {
    float m[8];
    float2 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = c0 + u * step, cc = min(c, nch - 1);
      m[u] = ml[(size_t)cc * mstride];
      x[u] = *(const float2*)(acc + (size_t)cc * astride + 2 * lane);
      if (c >= nch) m[u] = -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = exp2f(m[u] - l2);
      o.x += w * x[u].x;
      o.y += w * x[u].y;
    }
  }
  return o;
}

// The full layer's merge folded into a later pass over the same list (at most 64 dense chunks):
// every workgroup of the list derives the LSE of all R rows from the chunk partials into s_lse2
// (log2 units), and the rows r with r % nwg == cidx are merged by this workgroup: out (normalised),
// lse (natural log) and lse2 (log2), the last two nullable.  The rows this workgroup merges and the
// LSE table rows are loaded in one batch (lane = chunk), then reduced row by row.  Whole workgroup
// of NW waves; s_lse2 is complete only after a barrier.
template <int NW>
__device__ void fold_merge(const float* part_acc, const float* part_ml, int dchunk, int dmax_chunks, int R, int G,
                           int H, int n_q, int b, int g, int list, int Lb, int cidx, int nwg, float* s_lse2,
                           float* out, float* lse, float* lse2, int wave, int lane) {
  const int nchd = (Lb + dchunk - 1) / dchunk;                   // <= 64: one chunk per lane
  const size_t first = (size_t)list * dmax_chunks * R;
  constexpr int RPW = (32 + NW - 1) / NW;                        // rows per wave (R <= 32)
  auto mrow = [&](int j) { return cidx + nwg * (wave + NW * j); };
  float2 v[2 * RPW];
#pragma unroll
  for (int i = 0; i < 2 * RPW; ++i) {
    const int r = min(i < RPW ? wave + NW * i : mrow(i - RPW), R - 1);
    v[i] = *(const float2*)(part_ml + ((first + r) + (size_t)min(lane, nchd - 1) * R) * 2);
    if (lane >= nchd) v[i] = make_float2(-INFINITY, 0.f);
  }
  float l2m[RPW];
#pragma unroll
  for (int i = 0; i < 2 * RPW; ++i) {
    const int r = i < RPW ? wave + NW * i : mrow(i - RPW);
    if (r >= R) continue;                                        // uniform over the wave
    const float mx = wave_max(v[i].x);
    const float ls = mx == -INFINITY ? 0.f : wave_sum(exp2f(v[i].x - mx) * v[i].y);
    const float l2 = ls > 0.f ? mx + __log2f(ls) : -INFINITY;
    if (i < RPW) {
      if (lane == 0) s_lse2[r] = l2;
    } else {
      l2m[i - RPW] = l2;
    }
  }
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int mr = mrow(j);
    if (mr >= R) break;
    const float* ml = part_ml + (first + mr) * 2;
    const float2 o = l2m[j] == -INFINITY ? make_float2(0.f, 0.f)
                                         : merged_o(ml, (size_t)R * 2, part_acc + (first + mr) * D,
                                                    (size_t)R * D, 0, nchd, 1, l2m[j], lane);
    const size_t orow = ((size_t)b * n_q + mr / G) * H + (size_t)g * G + mr % G;
    *(float2*)(out + orow * D + 2 * lane) = o;
    if (lane == 0 && lse) lse[orow] = l2m[j] * LN2;
    if (lane == 0 && lse2) lse2[orow] = l2m[j];
  }
}

}  // namespace hs
