// Decode kernels for at most 32 query rows per KV head (the MQA decode shapes:
// 32 heads x 1 query token, 16 heads x 2, 8 heads x 4), bf16 or FP8 caches.
//
// Every wave streams its own 32-token tiles with no workgroup barrier in the
// loop, so a CU keeps many independent tiles in flight from HBM.
//
//  attn_wave    full layer, split-K pass 1 over all L_b rows (ithome page
//               "小米公开 MiMo-V3 核心架构 HySparse2", section "KV Reuse": the full
//               layer attends to every cached row).  A workgroup whose chunk is
//               the whole sequence writes O (and LSE) itself; otherwise it writes
//               one (m, l, acc) partial that the score pass or attn_merge
//               combines.
//  scores_wave  second pass of the full layer: s_j = sum over the heads of a
//               group of exp(l_j - LSE) for the candidates outside the recent
//               window (ithome page, "KV Reuse" and recent-window paragraphs),
//               plus the first-digit histogram the selection starts from.

#include <algorithm>

#include "hs_common.hpp"
#include "hs_internal.hpp"
#include "hs_mfma.hpp"

namespace hs {

namespace {

// Clears the words the caller asked for (the selection's histograms) with the whole grid.
__device__ __forceinline__ void zero_hook(const AttnArgs& a) {
  zero_words_grid(a.zero_ptr, a.zero_stride, a.zero_words, a.zero_lists);
  zero_words_grid(a.zero2_ptr, a.zero2_words, (int)a.zero2_words, 1);
}

// First digit of a score's key in candidate mode: key bits 30..20 (8 exponent and 3 fraction bits,
// eighth-octave bins).  The score pass only produces scores >= +0, whose keys all have bit 31 set,
// so these bits order them.
__device__ __forceinline__ int cand_digit(uint32_t key) { return (int)((key >> 20) & 0x7FFu); }

// Lowest candidate-mode first digit that the kk-th largest key of a list can still have, from the
// list's histogram as it stands: the highest digit d whose bins >= d already hold kk keys (counts
// only grow while the pass runs, so the final kk-th key's digit is >= d); 0 while fewer than kk
// keys have been counted.  Scores are sums of at most 32 probabilities; the bins of values in
// [2^-55, 2^17), digits 576 .. 1151, are read, 9 per lane, with device-coherent loads (keys outside
// them could only make d lower, never wrong).  Whole wave.
__device__ int lower_digit(const uint32_t* hist, uint32_t kk, int lane) {
  constexpr int PL = 9;
  uint32_t h[PL], tot = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    h[i] = __hip_atomic_load(hist + 576 + PL * lane + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    tot += h[i];
  }
  uint32_t suf = tot;                                             // keys in this lane's bins and above
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(suf, o);
    if (lane + o < 64) suf += y;
  }
  const unsigned long long reach = __ballot(suf >= kk);           // lanes 0 .. top reach kk
  if (!reach) return 0;
  const int top = 63 - __clzll((long long)reach);                 // highest such lane
  uint32_t above = __shfl(suf - tot, top);
  int found = 0;                                                  // bins of lane `top` from its top one
#pragma unroll
  for (int i = PL - 1; i >= 0; --i) {
    above += h[i];
    found += above < kk ? 1 : 0;
  }
  return 576 + PL * top + (PL - 1) - __shfl(found, top);
}

}  // namespace

// CODES: the score filter's codes are written (a.codes set).  A template parameter rather than a
// branch: with the stores behind a branch the compiler cannot count them at the loop head, and each
// tile would then wait for the previous tile's stores as well as for its own loads.
template <int KVT, int NW, bool CODES>
__global__ __launch_bounds__(64 * NW) void attn_wave_kernel(AttnArgs a) {
  constexpr int NT = 64 * NW;
  using M = Mma<CT_BF16>;
  constexpr int ROWB = M::ROWB;
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr bool SPLIT = KVT != KV_FP8;
  constexpr int SB = (KVT == KV_BF16 ? 2 : 1) * D;               // storage bytes per row
  constexpr int PPR = SB / 16;                                   // 16-byte pieces per row
  constexpr int PPL = 32 * PPR / 64;                             // pieces per lane per tensor
  constexpr int TILES = NW * 2 * 32 * ROWB;
  constexpr int DP = D + 4;                                      // merge row pitch: 32 heads' rows on distinct banks
  constexpr int MERGE = NW * 32 * (DP + 2) * 4;
  __shared__ __align__(16) char smem[TILES > MERGE ? TILES : MERGE];
  __shared__ __align__(16) char qs[32 * ROWB];
  __shared__ float ksc[FP8 ? NW * 32 : 1], vsc[FP8 ? NW * 32 : 1];

  zero_hook(a);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int list, chunk;
  grid_item(a.seq_len, a.n_kv, a.n_lists, a.chunk, 0, 1, a.uniform_items, blockIdx.x, list, chunk);
  if (list < 0) return;
  const int g = list % a.n_kv, b = list / a.n_kv, t0 = 0;
  const int c0 = chunk * a.chunk;
  const int Lb = a.seq_len[b];
  if (c0 >= Lb) return;
  const int c1 = min(Lb, c0 + a.chunk);
  const int64_t rs = a.row_start[b];
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SB;
  const char* vbase = (const char*)a.v + ((size_t)rs * a.n_kv + g) * SB;
  const size_t rstride = (size_t)a.n_kv * SB;
  const int ntiles = (c1 - c0 + 31) / 32;

  char* const kt = smem + wave * 2 * 32 * ROWB;
  char* const vt = kt + 32 * ROWB;
  float* const wks = FP8 ? ksc + wave * 32 : nullptr;
  float* const wvs = FP8 ? vsc + wave * 32 : nullptr;

  // Cache row of a tile position, clamped into the chunk so every load stays in bounds and needs no
  // branch (a branch around a load makes the compiler wait for it at the join); positions past the
  // chunk are masked in the softmax instead.
  auto tok_row = [&](int tile, int tok) -> int { return min(c0 + tile * 32 + tok, c1 - 1); };
  u32x4 rk[PPL], rv[PPL];
  float sk = 0.f, sv = 0.f;
  auto load_rows = [&](auto row_of, int srow) {
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const size_t off = (size_t)row_of(i) * rstride + ((lane + 64 * i) % PPR) * 16;
      rk[i] = load_stream(kbase + off);
      rv[i] = load_stream(vbase + off);
    }
    if (FP8) {
      sk = a.k_scale[((size_t)rs + srow) * a.n_kv + g];
      sv = a.v_scale[((size_t)rs + srow) * a.n_kv + g];
    }
  };
  auto load = [&](int tile) {
    load_rows([&](int i) { return tok_row(tile, (lane + 64 * i) / PPR); }, FP8 ? tok_row(tile, lane & 31) : 0);
  };
  if (wave < ntiles) load(wave);                                  // first tile, before the Q barrier

  // Q rows -> LDS (row r = tt*G + hh; rows >= R are zero)
  for (int p = tid; p < 32 * 16; p += NT) {
    const int r = p >> 4, c = p & 15;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < a.R) {
      const int t = t0 + r / a.G, hh = r % a.G;
      const size_t qoff = (((size_t)b * a.n_q + t) * a.H + (size_t)g * a.G + hh) * D + c * 8;
      if (a.q_f32) {
        const float* qf = (const float*)a.q + qoff;
        for (int j = 0; j < 4; ++j) x[j] = f32_to_bf16_rne(qf[2 * j]) | (f32_to_bf16_rne(qf[2 * j + 1]) << 16);
      } else {
        x = *(const u32x4*)((const uint16_t*)a.q + qoff);
      }
    }
    *(u32x4*)(qs + r * ROWB + c * 16) = x;
  }
  __syncthreads();

  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int p = lane + 64 * i, tok = p / PPR, c = p % PPR;
      if constexpr (FP8) {                                       // 16 codes -> 16 bf16 (exact)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const u32x4 x = t2 ? rv[i] : rk[i];
          char* dst = (t2 ? vt : kt) + tok * ROWB + c * 32;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4 o;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const uint32_t word = x[2 * h + (w >> 1)];
              const uint32_t c0b = (word >> (16 * (w & 1))) & 0xFFu, c1b = (word >> (16 * (w & 1) + 8)) & 0xFFu;
              o[w] = (__float_as_uint(e4m3_to_f32(c0b)) >> 16) | (__float_as_uint(e4m3_to_f32(c1b)) & 0xFFFF0000u);
            }
            *(u32x4*)(dst + 16 * h) = o;
          }
        }
      } else {
        *(u32x4*)(kt + tok * ROWB + c * 16) = rk[i];
        *(u32x4*)(vt + tok * ROWB + c * 16) = rv[i];
      }
    }
    if (FP8 && lane < 32) { wks[lane] = sk; wvs[lane] = sv; }   // masked tokens get p = 0 below
  };

  float m = -INFINITY, lsum = 0.f;
  f32x16 acc[4] = {};
  const float sl2 = a.scale_log2;
  // Score filter: a tile's codes are held in registers and stored during the wave's next tile, just
  // before that tile's prefetch, so waiting for a prefetch never waits for younger stores.
  uint32_t hw[4] = {0u, 0u, 0u, 0u};
  float hm = 0.f;
  int htile = -1;
  auto put_codes = [&]() {
    uint32_t* rec = (uint32_t*)(a.codes + ((size_t)list * a.code_tiles + (c0 >> 5) + htile) * CODE_TILE_BYTES);
#pragma unroll
    for (int j = 0; j < 4; ++j) rec[(2 * j + (lane >> 5)) * 32 + (lane & 31)] = hw[j];
    if (lane < 32) ((float*)(rec + 256))[lane] = hm;
  };
  for (int tile = wave; tile < ntiles; tile += NW) {
    wave_sync();
    store();
    wave_sync();
    if constexpr (CODES) {
      if (htile >= 0) put_codes();
    }
    if (tile + NW < ntiles) load(tile + NW);
    f32x16 s = {};                                               // S^T = K Q^T, Q operand from LDS
    {
      const char* kb = kt + (lane & 31) * ROWB + (lane >> 5) * 16;
      const char* qb = qs + (lane & 31) * ROWB + (lane >> 5) * 16;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const s16x8 ka = *(const s16x8*)(kb + 32 * st);
        const s16x8 qa = *(const s16x8*)(qb + 32 * st);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka), __builtin_bit_cast(bf16x8, qa), s,
                                                    0, 0, 0);
      }
    }
    // Online softmax in log2 units with lazy rescaling: a row's reference m moves only when the
    // tile's max exceeds it by more than TAU, so p = 2^(l - m) <= 2^TAU and most tiles skip the
    // rescale of acc (LSE = m + log2(l) and every later combination hold for any reference).  bf16:
    // the factor is the constant sl2, so the max is taken on S and the logits are formed in exp2's
    // fma; E4M3: per-token factors, logits formed first.
    constexpr float TAU = 8.f;
    float mt = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tk = crow(lane, r);
      const bool ok = c0 + tile * 32 + tk < c1;
      const float x = FP8 ? s[r] * sl2 * wks[tk] : s[r];
      s[r] = ok ? x : -INFINITY;
      mt = fmaxf(mt, s[r]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    if (!FP8) mt *= sl2;
    const bool need = mt > m + TAU;                               // same for both lanes of a row
    if (__ballot(need)) {                                         // every wave's first tile: m = -inf
      const float mn = need ? mt : m;
      const float alpha = exp2f(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int mt4 = 0; mt4 < 4; ++mt4) acc[mt4] *= alpha;
      m = mn;
    }
    float p[16], xr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      xr[r] = FP8 ? s[r] - m : fmaf(s[r], sl2, -m);              // logit - reference, log2 units (<= 8)
      p[r] = exp2_fast(xr[r]);
      lsum += p[r];
      if (FP8) p[r] *= wvs[crow(lane, r)];
    }
    if constexpr (CODES) {
      // Score filter: one byte per (token, row), floor(8 x + 191) clamped to [0, 255] (masked
      // positions: x = -inf, code 0), four consecutive tokens per word; the tile's record holds
      // quads 2 j + (lane >> 5) of row lane & 31, then the rows' references.
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w = 0u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float y = __builtin_amdgcn_fmed3f(fmaf(xr[4 * j + i], 8.f, (float)CODE_OFFSET), 0.f, 255.f);
          w |= (uint32_t)y << (8 * i);
        }
        hw[j] = w;
      }
      hm = m;
      htile = tile;
    }
    M::template pv<SPLIT>(acc, vt, p, lane);
  }
  if constexpr (CODES) {
    if (htile >= 0) put_codes();
  }
  lsum += __shfl_xor(lsum, 32);

  // merge the NW waves (fixed order) through LDS
  __syncthreads();
  float* accb = (float*)smem;                                     // [wave][32 rows][DP]
  float* mlb = accb + NW * 32 * DP;                               // [wave][32][2]
  {
    float* mine = accb + (wave * 32 + (lane & 31)) * DP;
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
  constexpr int PER = 32 * D / NT;                                // d values per thread
  const int lin = tid * PER, row = lin / D, d0 = lin % D;
  const bool row_ok = row < a.R;
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
  const int t = t0 + (row_ok ? row / a.G : 0), hh = row_ok ? row % a.G : 0;
  const size_t orow = ((size_t)b * a.n_q + t) * a.H + (size_t)g * a.G + hh;
  if (a.direct) {                                                 // one chunk per list: final output
    if (row_ok) {
      const float inv = ls > 0.f ? 1.f / ls : 0.f;
#pragma unroll
      for (int e = 0; e < PER / 4; ++e) *(f32x4*)(a.out + orow * D + d0 + 4 * e) = o[e] * inv;
      if (d0 == 0) {
        const float l2v = ls > 0.f ? mx + __log2f(ls) : -INFINITY;
        if (a.lse) a.lse[orow] = l2v * LN2;
        if (a.lse2) a.lse2[orow] = l2v;
      }
    }
    return;
  }
  const size_t base = (size_t)list * a.max_chunks;
  if (row_ok) {
    float* pa = a.part_acc + ((base + chunk) * a.R + row) * D + d0;
#pragma unroll
    for (int e = 0; e < PER / 4; ++e) *(f32x4*)(pa + 4 * e) = o[e];
    if (d0 == 0) *(float2*)(a.part_ml + ((base + chunk) * a.R + row) * 2) = make_float2(mx, ls);
  }
}

// Score pass: each wave streams 64-token K tiles (coalesced 1 KB loads) with
// two tiles in flight in registers while the current one, staged in the
// wave's own LDS slice, feeds the MFMA B operand (S = Q K^T: lane = token, 16
// rows per lane), so the sum over a query token's heads is mostly in-lane.
//
// CAND (candidate mode, one query token): the grid holds about one workgroup per CU and each
// keeps one list, walking its items of a.chunk = 2 NW TT tokens chunk-major (item j is the list's
// chunk slot + j * nper), so every list's histogram fills early in the pass.  After each item a
// wave moves its share of the LDS histogram to the list's global one and, on its turn, derives
// from it the lowest first digit the k'-th key can still have; the scores at or above it are
// appended as (key, index) pairs for the selection, and dense scores are written only on request.
template <int KVT, int NW, int NQ, bool CAND>
__global__ __launch_bounds__(64 * NW) void scores_wave_kernel(ScoreArgs a) {
  constexpr bool FP8 = KVT == KV_FP8;
  constexpr int NT = 64 * NW;
  constexpr int TT = 64;                                         // tokens per wave tile
  constexpr int ROWB = 272;                                      // bf16 row + 16-byte pad
  constexpr int SB = (KVT == KV_BF16 ? 2 : 1) * D;
  constexpr int PPR = SB / 16;
  constexpr int PPL = TT * PPR / 64;                             // 16-byte pieces per lane per tile
  __shared__ uint32_t hist[NQ][2048];
  __shared__ __align__(16) char qs[32 * ROWB];
  __shared__ __align__(16) char ktile[NW][TT * ROWB];
  __shared__ float ksc[FP8 ? NW : 1][TT];

  __shared__ float s_lse2[32];
  __shared__ int s_kd;                                           // CAND: lowest first digit appended
  __shared__ uint32_t s_cc;                                      // CAND: pairs in this workgroup's region
  __shared__ uint32_t s_claimed;                                 // CAND: units this workgroup has taken
  static_assert(!CAND || NQ == 1, "candidate mode: one query token");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int list, cidx, slot = 0, nper = 1;                            // lists own max(fold, ceil(ncand / chunk)) items
  if constexpr (CAND) {                                           // a list's workgroups: consecutive (and XCDs)
    if (a.cand_uniform) {
      nper = (int)gridDim.x / a.n_lists;
      list = (int)blockIdx.x / nper;
      slot = (int)blockIdx.x % nper;
    } else {                                                     // prefix over the lists (n_lists <= 64)
      int acc = 0;
      list = a.n_lists - 1;
      for (int l = 0; l < a.n_lists; ++l) {
        const int L = a.seq_len[l / a.n_kv];
        const int np = cand_nper(L - min(a.window, L), a.cand_total);
        if ((int)blockIdx.x < acc + np) { list = l; nper = np; break; }
        acc += np;
      }
      slot = (int)blockIdx.x - acc;
    }
    cidx = slot;
  } else {
    grid_item(a.seq_len, a.n_kv, a.n_lists, a.chunk, a.window, a.part_ml ? 1 : 0, a.uniform_items, blockIdx.x, list,
              cidx);
    if (list < 0) return;
  }
  const int g = list % a.n_kv, b = list / a.n_kv;
  const int Lb = a.seq_len[b];
  const int w = min(a.window, Lb);
  const int ncand = Lb - w;
  const int c0 = cidx * a.chunk;
  const int c1 = min(ncand, c0 + a.chunk);
  const int64_t rs = a.row_start[b];
  const char* kbase = (const char*)a.k + ((size_t)rs * a.n_kv + g) * SB;
  const size_t rstride = (size_t)a.n_kv * SB;
  const int ntiles = c1 > c0 ? (c1 - c0 + TT - 1) / TT : 0;
  // Dense mode: this wave's tiles q = 0 .. nq - 1 of the chunk.  Candidate mode: units of UT = 2 tiles,
  // unit u = tiles u % 8 and u % 8 + 8 of the 16-tile item u / 8 (consecutive units read one item
  // together; one wave reading two adjacent tiles instead was slower), each wave's first two units
  // static (unit slot * NW + wave, then that plus nper * NW), the rest taken in order from the list's
  // counter by whichever wave of the list's workgroups is free, so slower XCDs take fewer.  Positions
  // from cend on are masked.
  constexpr int UT = 2 * TT;
  const int nq = CAND ? 0 : (wave < ntiles ? (ntiles - 1 - wave) / NW + 1 : 0);
  const int nunits = CAND ? (ncand + 8 * UT - 1) / (8 * UT) * 8 : 0;
  const int cend = CAND ? ncand : c1;
  auto tstart = [&](int q) -> int { return c0 + (wave + NW * q) * TT; };
  auto ustart = [&](int u, int h) -> int { return u < nunits ? (u >> 3) * (8 * UT) + ((u & 7) + 8 * h) * TT : cend; };
  int uk = slot * NW + wave;                                     // CAND: the unit in hand
  char* const kt = ktile[wave];
  // Two tiles in flight per wave: buffers A and B alternate (named, so every wait is a static count).
  // Loads past the wave's last tile are not skipped (no branch surrounds a load) but start at cend, so
  // every position clamps to the list's last row: one row, read again.
  u32x4 kA[PPL], kB[PPL];
  float sA = 0.f, sB = 0.f;
  auto load = [&](u32x4 (&kr)[PPL], float& ks, int ts) {        // clamped rows: no branch, in bounds
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int p = lane + 64 * i;
      const int pos = min(ts + p / PPR, cend - 1);
      kr[i] = load_stream(kbase + (size_t)pos * rstride + (p % PPR) * 16);
    }
    if (FP8) ks = a.k_scale[((size_t)rs + min(ts + lane, cend - 1)) * a.n_kv + g];
  };
  if (CAND) {                                                    // in flight during the prologue below
    if (nunits > 0) {                                            // else no row to clamp to (L_b <= window)
      load(kA, sA, ustart(uk, 0));
      load(kB, sB, ustart(uk, 1));
    }
  } else if (nq > 0) {
    load(kA, sA, tstart(0));
    load(kB, sB, nq > 1 ? tstart(1) : cend);
  }
  if (a.part_ml) {
    const int nwg = CAND ? nper : max(1, (ncand + a.chunk - 1) / a.chunk);
    if (cidx >= nwg) return;
    fold_merge<NW>(a.part_acc, a.part_ml, a.dchunk, a.dmax_chunks, a.R, a.G, a.H, a.n_q, b, g, list, Lb, cidx, nwg,
                   s_lse2, a.out, a.lse, nullptr, wave, lane);
  }
  if (!CAND && c0 >= ncand) return;
  const bool do_hist = a.hist != nullptr;
  if (do_hist)
    for (int i = tid; i < NQ * 2048; i += NT) hist[i >> 11][i & 2047] = 0u;
  const int kk = max(0, min(a.top_k, Lb - a.window));
  const bool need_cand = CAND && kk > 0 && kk < ncand;           // else the selection needs no candidates
  uint32_t* ghist = a.hist + ((size_t)b * a.n_kv + g) * a.hist_stride;   // CAND: the list's (one query token)
  if (CAND && wave == 0) {
    const int d = need_cand ? lower_digit(ghist, (uint32_t)kk, lane) : 2048;
    if (lane == 0) { s_kd = d; s_cc = 0u; s_claimed = 2u * NW; }
    if (lane == 0 && slot == 0) ghist[SELECT_NREG_WORD] = (uint32_t)nper;
  }
  uint2* const region = CAND ? (uint2*)(ghist + a.cand_off) + (size_t)slot * a.cand_region : nullptr;
  for (int p = tid; p < 32 * 16; p += NT) {
    const int r = p >> 4, c = p & 15;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (r < a.R) {
      const size_t qoff = (((size_t)b * a.n_q + r / a.G) * a.H + (size_t)g * a.G + r % a.G) * D + c * 8;
      if (a.q_f32) {
        const float* qf = (const float*)a.q + qoff;
        for (int j = 0; j < 4; ++j) x[j] = f32_to_bf16_rne(qf[2 * j]) | (f32_to_bf16_rne(qf[2 * j + 1]) << 16);
      } else {
        x = *(const u32x4*)((const uint16_t*)a.q + qoff);
      }
    }
    *(u32x4*)(qs + r * ROWB + c * 16) = x;
  }
  __syncthreads();
  s16x8 qop[8];                                                  // A = Q: row (l & 31), d = 16 s + 8 (l >> 5)
#pragma unroll
  for (int s = 0; s < 8; ++s) qop[s] = *(const s16x8*)(qs + (lane & 31) * ROWB + (16 * s + 8 * (lane >> 5)) * 2);
  float lse2[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {                                 // rows past R: p = exp2(-inf) = 0
    const int rw = crow(lane, r), rc = min(rw, a.R - 1);
    const float v = a.part_ml ? s_lse2[rc] : a.lse2[((size_t)b * a.n_q + rc / a.G) * a.H + (size_t)g * a.G + rc % a.G];
    lse2[r] = rw < a.R ? v : INFINITY;
  }
  const int tpw = a.G >= 32 ? 1 : 32 / a.G;                      // query tokens in the 32 rows
  float* sout = a.scores ? a.scores + (size_t)b * a.n_q * a.n_kv * a.s_stride : nullptr;
  // (key, index) of a score to the workgroup's region when its first digit reaches the bound; whole wave
  auto append = [&](uint32_t key, int pos) {
    const bool keep = lane < 32 && pos < cend && cand_digit(key) >= *(volatile int*)&s_kd;
    const unsigned long long mk = __ballot(keep);
    if (mk) {
      uint32_t base = 0u;
      if (lane == 0) base = atomicAdd(&s_cc, (uint32_t)__popcll(mk));
      base = __shfl(base, 0);
      if (keep) region[base + __popcll(mk & ((1ull << lane) - 1ull))] = make_uint2(key, (uint32_t)pos);
    }
  };
  // hold != null: the keys are kept (hold[half]) instead of appended
  auto process = [&](const u32x4 (&kr)[PPL], float ks, int ts, uint32_t* hold) {
    wave_sync();
#pragma unroll
    for (int i = 0; i < PPL; ++i) {                              // registers -> LDS (FP8 -> bf16)
      const int p = lane + 64 * i, tok = p / PPR, c = p % PPR;
      const u32x4 x = kr[i];
      if constexpr (FP8) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4 o;
#pragma unroll
          for (int ww = 0; ww < 4; ++ww) {
            const uint32_t word = x[2 * h + (ww >> 1)];
            const uint32_t c0b = (word >> (16 * (ww & 1))) & 0xFFu, c1b = (word >> (16 * (ww & 1) + 8)) & 0xFFu;
            o[ww] = (__float_as_uint(e4m3_to_f32(c0b)) >> 16) | (__float_as_uint(e4m3_to_f32(c1b)) & 0xFFFF0000u);
          }
          *(u32x4*)(kt + tok * ROWB + c * 32 + 16 * h) = o;
        }
      } else {
        *(u32x4*)(kt + tok * ROWB + c * 16) = x;
      }
    }
    if (FP8) ksc[wave][lane] = ks;
    wave_sync();
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x16 s = {};
      const char* kb = kt + (32 * half + (lane & 31)) * ROWB + (lane >> 5) * 16;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const s16x8 kv = *(const s16x8*)(kb + 32 * st);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qop[st]), __builtin_bit_cast(bf16x8, kv),
                                                    s, 0, 0, 0);
      }
      const float f = a.scale_log2 * (FP8 ? ksc[wave][32 * half + (lane & 31)] : 1.f);
      const int pos = ts + 32 * half + (lane & 31);
      float tv[NQ];
      tile_scores<NQ>(s, f, lse2, tpw, tv);
      if (lane < 32 && pos < cend) {
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          if (t >= a.n_q) break;
          if (sout) sout[((size_t)t * a.n_kv + g) * a.s_stride + pos] = tv[t];
          if (do_hist) atomicAdd(&hist[t][CAND ? cand_digit(f32_key(tv[t])) : (int)(f32_key(tv[t]) >> 21)], 1u);
        }
      }
      if (need_cand) {
        if (hold) hold[half] = f32_key(tv[0]);
        else append(f32_key(tv[0]), pos);
      }
    }
  };
  // this wave's share of the histogram to the list's global one (read and clear: adds that other waves
  // make meanwhile stay for a later move), only its bins at or above the current bound: the bound never
  // falls, so lower bins cannot move it (they reach the global histogram at the end)
  auto flush_share = [&]() {
    constexpr int SHARE = 2048 / NW;
    const int lo = max(wave * SHARE, *(volatile int*)&s_kd);
    for (int i = lo + lane; i < (wave + 1) * SHARE; i += 64) {
      const uint32_t v = atomicExch(&hist[0][i], 0u);
      if (v) atomicAdd(ghist + i, v);
    }
  };
  if constexpr (CAND) {
    // A workgroup takes at most cap units (its region holds cap * UT pairs); the caps of a list's
    // workgroups add up to at least twice its units, so every unit is taken.
    const uint32_t cap = (uint32_t)(a.cand_region / UT);
    uint32_t* const ctr = ghist + SELECT_CLAIM_WORD;
    // (atomicInc, not atomicAdd: the compiler turns a uniform-address add into a wave-wide one whose
    // result it broadcasts at once, which would wait for every load in flight)
    // The value is used as returned (no arithmetic next to the atomic, which would wait for it).
    auto claim = [&]() -> uint32_t {                             // lane 0: the counter's value, or ~0
      uint32_t r = ~0u;
      if (lane == 0 && atomicAdd(&s_claimed, 1u) < cap) r = atomicInc(ctr, ~0u);
      return r;
    };
    // The claim for the unit after next is issued before that unit's loads, so reading it waits for
    // nothing issued later.
    uint32_t rc = (uint32_t)((nper + slot) * NW + wave), roff = 0u;   // the second static unit
    // The first unit's keys are held until the list's histogram has the first units' counts: after
    // them every wave refreshes the bound, then appends the held keys that reach it (most of the
    // first units' scores would otherwise be appended before any bound exists).
    if (uk < nunits) {
      uint32_t hk[4];
      process(kA, sA, ustart(uk, 0), hk);
      const uint32_t raw = __builtin_amdgcn_readfirstlane(rc);
      const int un = (int)min(raw, (uint32_t)nunits);
      rc = claim();
      roff = 2u * nper * NW;
      load(kA, sA, ustart(un, 0));
      process(kB, sB, ustart(uk, 1), hk + 2);
      load(kB, sB, ustart(un, 1));
      if (need_cand) {
        flush_share();
        const int d = lower_digit(ghist, (uint32_t)kk, lane);
        if (lane == 0) atomicMax(&s_kd, d);
#pragma unroll
        for (int q = 0; q < 4; ++q) append(hk[q], ustart(uk, q >> 1) + 32 * (q & 1) + (lane & 31));
      }
      uk = un;
    }
    for (int k = 1; uk < nunits; ++k) {
      process(kA, sA, ustart(uk, 0), nullptr);
      const uint32_t raw = __builtin_amdgcn_readfirstlane(rc);
      const int un = raw == ~0u ? nunits : (int)min(raw + roff, (uint32_t)nunits);
      rc = claim();
      roff = 2u * nper * NW;                                     // counter value c is unit c + 2 nper NW
      load(kA, sA, ustart(un, 0));
      process(kB, sB, ustart(uk, 1), nullptr);
      // on this wave's turn, a fresh bound from the list's histogram (here, while kB's registers are
      // free; the next load of kB waits for it)
      if (need_cand && k % NW == wave) {
        const int d = lower_digit(ghist, (uint32_t)kk, lane);
        if (lane == 0) atomicMax(&s_kd, d);
      }
      load(kB, sB, ustart(un, 1));
      if (need_cand) flush_share();
      uk = un;
    }
  } else {
    for (int q = 0; q < nq; q += 2) {
      process(kA, sA, tstart(q), nullptr);
      load(kA, sA, q + 2 < nq ? tstart(q + 2) : cend);
      if (q + 1 >= nq) break;
      process(kB, sB, tstart(q + 1), nullptr);
      load(kB, sB, q + 3 < nq ? tstart(q + 3) : cend);
    }
  }
  if (!do_hist) return;
  __syncthreads();
  if (CAND && tid == 0) ghist[SELECT_RCOUNT_WORD + slot] = s_cc;
  for (int i = tid; i < a.n_q * 2048; i += NT) {
    const uint32_t v = hist[i >> 11][i & 2047];
    if (v) atomicAdd(a.hist + (((size_t)b * a.n_q + (i >> 11)) * a.n_kv + g) * a.hist_stride + (i & 2047), v);
  }
}

template <int KVT>
static hipError_t launch_wave_t(const AttnArgs& a, hipStream_t st) {
  constexpr int NW = 8;
  if (a.codes)
    hipLaunchKernelGGL((attn_wave_kernel<KVT, NW, true>), dim3(a.n_items), dim3(64 * NW), 0, st, a);
  else
    hipLaunchKernelGGL((attn_wave_kernel<KVT, NW, false>), dim3(a.n_items), dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_wave(const AttnArgs& a, int kvt, hipStream_t st) {
  if (a.R > 32) return hipErrorInvalidValue;
  if (kvt == KV_BF16) return launch_wave_t<KV_BF16>(a, st);
  if (kvt == KV_FP8) return launch_wave_t<KV_FP8>(a, st);
  return hipErrorInvalidValue;
}

template <int KVT, int NQ>
static void launch_scores_wave_t(const ScoreArgs& a, hipStream_t st) {
  constexpr int NW = NQ == 1 ? 8 : 6;                            // LDS: NW x 17 KB tiles + NQ x 8 KB histograms
  if constexpr (NQ == 1) {
    if (a.cand_off > 0) {
      hipLaunchKernelGGL((scores_wave_kernel<KVT, NW, NQ, true>), dim3(a.n_items), dim3(64 * NW), 0, st, a);
      return;
    }
  }
  hipLaunchKernelGGL((scores_wave_kernel<KVT, NW, NQ, false>), dim3(a.n_items), dim3(64 * NW), 0, st, a);
}

int scores_cand_chunk() { return 2 * 64; }

int64_t scores_cand_region(int64_t s_stride, int nper) {
  constexpr int NW = 8;
  const int64_t units = (s_stride + 8 * scores_cand_chunk() - 1) / (8 * scores_cand_chunk()) * 8;
  const int64_t share = (units + nper - 1) / nper;
  return std::max<int64_t>(2 * share, 2 * NW) * scores_cand_chunk();
}

hipError_t launch_scores_wave(const ScoreArgs& a, int kvt, hipStream_t st) {
  if (a.R > 32 || a.n_q > 4 || (kvt != KV_BF16 && kvt != KV_FP8)) return hipErrorInvalidValue;
  if (a.cand_off > 0 &&
      (a.n_q != 1 || !a.hist || a.chunk != scores_cand_chunk() || (a.cand_uniform && a.n_items % a.n_lists) ||
       (a.cand_uniform && a.cand_region < scores_cand_region(a.s_stride, a.n_items / a.n_lists)) ||
       (!a.cand_uniform && (a.n_lists > 64 || a.cand_total < 0))))
    return hipErrorInvalidValue;
  const int nq = a.n_q == 1 ? 1 : a.n_q == 2 ? 2 : 4;
  if (kvt == KV_BF16) {
    if (nq == 1) launch_scores_wave_t<KV_BF16, 1>(a, st);
    else if (nq == 2) launch_scores_wave_t<KV_BF16, 2>(a, st);
    else launch_scores_wave_t<KV_BF16, 4>(a, st);
  } else {
    if (nq == 1) launch_scores_wave_t<KV_FP8, 1>(a, st);
    else if (nq == 2) launch_scores_wave_t<KV_FP8, 2>(a, st);
    else launch_scores_wave_t<KV_FP8, 4>(a, st);
  }
  return hipGetLastError();
}

}  // namespace hs
