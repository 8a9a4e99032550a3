// MFMA tile policies shared by the attention kernels (gfx950, wave64).
#pragma once

#include "hs_common.hpp"
#include "hs_internal.hpp"

namespace hs {

// ---------------------------------------------------------------- MFMA policies

// C/D layout of every 32x32 MFMA: lane l holds column (l & 31) and the 16 rows
// 8*(r/4) + 4*(l>>5) + (r&3), r = 0..15.
__device__ __forceinline__ int crow(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int CT>
struct Mma;

// bf16 inputs, fp32 accumulate: v_mfma_f32_32x32x16_bf16.  Operand lane
// layout: lane l supplies row/column (l & 31) and 8 consecutive k values;
// the k index of element j is the same function of (l >> 5, j) for A and B,
// so only consistency between the two operands matters.
template <>
struct Mma<CT_BF16> {
  static constexpr int ROWB = 272;      // LDS bytes per token row: 256 + 16 pad (bank spread)
  static constexpr int ESZ = 2;
  struct QOp {
    s16x8 v[8];                         // k-step s: d = 16 s + 8 (l >> 5) + j
  };
  __device__ static void load_q(QOp& q, const void* row, bool q_f32, bool valid, int lane) {
    const int d0 = 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s16x8 t = {};
      if (valid) {
        if (q_f32) {
          const float* p = (const float*)row + 16 * s + d0;
#pragma unroll
          for (int j = 0; j < 8; ++j) t[j] = (short)f32_to_bf16_rne(p[j]);
        } else {
          t = *(const s16x8*)((const uint16_t*)row + 16 * s + d0);
        }
      }
      q.v[s] = t;
    }
  }
  // S^T = K Q^T for 32 tokens starting at ktile (LDS) and this wave's 32 rows.
  __device__ static f32x16 qk_t(const char* ktile, const QOp& q, int lane) {
    f32x16 acc = {};
    const char* base = ktile + (lane & 31) * ROWB + (lane >> 5) * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s16x8 a = *(const s16x8*)(base + 32 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                     __builtin_bit_cast(bf16x8, q.v[s]), acc, 0, 0, 0);
    }
    return acc;
  }
  // S = Q K^T (rows x tokens).
  __device__ static f32x16 qk(const char* ktile, const QOp& q, int lane) {
    f32x16 acc = {};
    const char* base = ktile + (lane & 31) * ROWB + (lane >> 5) * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s16x8 b = *(const s16x8*)(base + 32 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, q.v[s]),
                                                     __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
    }
    return acc;
  }
  // O^T[d x rows] += V^T[d x tok] P^T[tok x rows]; p[r] is this lane's value
  // for token crow(lane, r).  PV k-step u, element j <-> r = 8u + j.
  template <bool SPLIT>
  __device__ static void pv(f32x16 (&acc)[4], const char* vtile, const float (&p)[16], int lane) {
    s16x8 ph[2], pl[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      uint32_t hb = f32_to_bf16_rne(p[r]);
      ph[r >> 3][r & 7] = (short)hb;
      if (SPLIT) pl[r >> 3][r & 7] = (short)f32_to_bf16_rne(p[r] - bf16_to_f32(hb));
    }
    const char* vb = vtile + (lane & 31) * 2 + (lane >> 5) * 4 * ROWB;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s16x8 a;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          a[j] = *(const short*)(vb + 64 * mt + (16 * u + 8 * (j >> 2) + (j & 3)) * ROWB);
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                           __builtin_bit_cast(bf16x8, ph[u]), acc[mt], 0, 0, 0);
        if (SPLIT)
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, pl[u]), acc[mt], 0, 0, 0);
      }
    }
  }
};

// fp32 inputs: v_mfma_f32_32x32x2_f32.  Lane l supplies row/column (l & 31)
// and the single k index (l >> 5) of each step.
template <>
struct Mma<CT_F32> {
  static constexpr int ROWB = 516;      // 512 + 4: consecutive rows start one bank apart
  static constexpr int ESZ = 4;
  struct QOp {
    float v[64];                        // step s: d = 2 s + (l >> 5)
  };
  __device__ static void load_q(QOp& q, const void* row, bool q_f32, bool valid, int lane) {
    const int d0 = lane >> 5;
#pragma unroll
    for (int s = 0; s < 64; ++s) {
      float x = 0.f;
      if (valid) x = q_f32 ? ((const float*)row)[2 * s + d0] : bf16_to_f32(((const uint16_t*)row)[2 * s + d0]);
      q.v[s] = x;
    }
  }
  __device__ static f32x16 qk_t(const char* ktile, const QOp& q, int lane) {
    f32x16 acc = {};
    const float* base = (const float*)(ktile + (lane & 31) * ROWB) + (lane >> 5);
#pragma unroll
    for (int s = 0; s < 64; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(base[2 * s], q.v[s], acc, 0, 0, 0);
    return acc;
  }
  __device__ static f32x16 qk(const char* ktile, const QOp& q, int lane) {
    f32x16 acc = {};
    const float* base = (const float*)(ktile + (lane & 31) * ROWB) + (lane >> 5);
#pragma unroll
    for (int s = 0; s < 64; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(q.v[s], base[2 * s], acc, 0, 0, 0);
    return acc;
  }
  // step r pairs token crow(lane, r) of the two lane halves.
  template <bool SPLIT>
  __device__ static void pv(f32x16 (&acc)[4], const char* vtile, const float (&p)[16], int lane) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* vr = (const float*)(vtile + crow(lane, r) * ROWB) + (lane & 31);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * mt], p[r], acc[mt], 0, 0, 0);
    }
  }
};

}  // namespace hs
