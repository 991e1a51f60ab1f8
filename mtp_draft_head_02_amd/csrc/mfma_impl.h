// The lm_head sweep + fused argmax for wide batches, on the matrix cores.
//
// At b vectors per call the VALU sweep spends, per 16-byte weight chunk, one
// decode plus b dot products and b reads of the staged vectors from LDS; from
// b of 3 to 5 (FP8) or 2 to 3 (NVFP4) that outruns HBM on gfx950 (BF16, with no
// decode and 8 elements per chunk, stays faster on the VALU sweep). Here the
// contraction runs as 16 x 16 x 32 MFMAs with the weights as the A operand
// (16 rows per tile, one per lane column) and the staged vectors as B (one
// vector per lane column; columns past b repeat vector col % b and their
// results are dropped), so a 16-byte chunk costs its decode, EPC / 8 MFMAs and
// EPC / 8 LDS reads per lane whatever b is (deepseek_v4_mtp.rs `forward_one` steps 6-7 for what
// is computed; the weight formats are those of mtp_head.rs `MtpQuantization`).
//
// Layout and schedule (gfx950, wave64, 8 waves per CU in one block):
//   - A tile is 16 consecutive rows; a unit is J = 8 loads per lane, 512
//     bytes of each of the tile's 16 rows; two register buffers keep one unit
//     in flight while the other is computed. The tiles are dealt to the
//     blocks round-robin over the grid; waves take their block's tiles from an
//     LDS counter as they need them; or (BF16, and FP8 where the partial sums
//     fit: a whole tile is too long a piece of one wave's share of the CU for
//     the launch to end evenly) the block walks its tiles in rounds, Q = 2 or
//     4 waves per tile, each summing a contiguous range of the tile's passes,
//     the Q partial sums added in LDS in wave order after a block barrier per
//     round (mfma_split_q).
//   - The MFMA wants, in lane l, row l % 16 and the k group g = l / 16, so a
//     load in that layout covers 64 bytes of each of 16 rows (a streaming
//     read in that pattern reaches ~68 % of 8 TB/s on this part, against 83 %
//     for contiguous 512-byte runs). So each load instruction instead covers
//     2 rows x 512 contiguous bytes (lanes 0-31 one row, 32-63 the next, non-
//     temporal), and the unit passes through a per-wave LDS tile
//     [16 rows][512 B + 16 B pad]: written as loaded, read back in the MFMA
//     layout (both conflict-free). Measured: FP8 b = 8 at 154,880 x 4,096,
//     128 us in the MFMA layout, 114 us through the tile.
//   - Decode: BF16 as is; FP8 to BF16 pairs (exact hardware convert), the row
//     scale applied to the finished sums; NVFP4 to F16 pairs (exact), each
//     16-element block multiplied by its E4M3 scale in F16 (exact: at most 6
//     significant bits, magnitudes within 2^-10 .. 2688), the global scale
//     applied to the finished sums. A chunk's two scale bytes come from the
//     lane of its row that loaded them (ds_bpermute).
//   - The staged vectors live in LDS row-major [b][k], the row stride padded
//     to 1 (mod 16) 16-byte chunks so the 16 columns of a read hit distinct
//     banks. For NVFP4 they are converted to F16 after a per-vector power-of-2
//     scaling that puts the vector's largest magnitude in [2^14, 2^15); the
//     power of 2 is undone on the finished sums. A BF16 value converts
//     exactly when, so scaled, it is at least 2^-17 in magnitude (or zero).
//     Every block checks that for every element of every vector (the same
//     check on the same data, so all blocks agree); if one fails, the launch
//     runs the VALU sweep instead, which takes the BF16 vectors as they are.
//   - NVFP4 block scales are loaded in the MFMA layout (64 bytes of 16 rows
//     per unit) with plain loads: a load covers half of a 128-byte line of
//     each row and the next unit the other half; non-temporal loads there
//     fetched every scale line twice.
//   - The 16 x 16 result of a tile holds, in lane l, rows 4 (l / 16) .. + 3 of
//     column l % 16; each lane keeps a running (best, lowest row) argmax and,
//     with the log-probability, an online softmax sum for its column, merged
//     per vector over the wave, the block and the grid as in the VALU sweep.
//   - The summation order of a row's logit (MFMA k-steps in k order within a
//     tile or within each half of it, the halves added in wave order) is the
//     same for every row and every b, so identical rows give identical logits.
#pragma once
#include "sweep_impl.h"

namespace mtp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// LDS budget of a launch (dynamic + the kernel's own ~4 KB within 160 KB).
constexpr int kMfmaMaxLds = 152 * 1024;
constexpr int kMfmaThreads = 512;
constexpr int kMfmaWaves = kMfmaThreads / kWave;
// Loads per lane per unit (8 KB of weights per wave per unit at J = 8, plus
// 1 KB of block scales at NVFP4).
template <int WD> constexpr int mfma_loads() { return 8; }

// Smallest batch that takes the MFMA form, per weight format: BF16 3, FP8 5,
// NVFP4 3; FP8 3 and NVFP4 2 where the VALU sweep's rows are not a whole
// number of its passes (h % 4096 != 0: that sweep then takes its slower
// clamped form). From measurements at 154,880 x 4,096 and 131,072 x 5,120.
template <int WD>
inline int mfma_min_b(int k) {
  if (WD == kBF16) return 3;
  const bool valu_ragged = (k / WT<WD>::kEPC) % (kWave * WT<WD>::kJ) != 0;
  if (WD == kFP8) return valu_ragged ? 3 : 5;
  return valu_ragged ? 2 : 3;
}

// LDS row stride of a staged vector, in 16-byte chunks: k/8 rounded up to 1 (mod 16).
__host__ __device__ inline int mfma_x_stride(int cx) { return cx + ((1 - cx) & 15); }
// Per-wave weight tile in LDS: 16 rows of a unit (4J chunks) plus one pad chunk.
template <int J> constexpr int mfma_tile_stride() { return 4 * J + 1; }
template <int J> constexpr int mfma_tile_bytes() { return kMfmaWaves * 16 * mfma_tile_stride<J>() * 16; }

template <int J>
struct MUnit {
  u32x4 w[J];
  uint32_t sd[J / 2];  // NVFP4: this lane's J/2 of its row's 2J block-scale dwords of the unit
  float rs;            // FP8: the scale of row `col` of the unit's tile (every unit)
  uint32_t mw;         // grammar-mask word of this lane's column for the tile (masked: every unit)
};

// Staged BF16 vectors -> F16 in place, each vector scaled by 2^e_b (e_b chosen
// from its largest magnitude), e_b -> xexp[b]. Returns (the same in every
// thread and every block) whether every element converts exactly: each vector
// finite, and every nonzero element at least 2^-17 once scaled (its lowest
// significant bit then lies at or above 2^-24, the F16 subnormal step). When
// it returns false the contents of xs are unspecified.
template <int B, int NT>
__device__ __forceinline__ bool stage_to_f16(u32x4 *xs, int CX, int CXP, int *xexp) {
  constexpr int kWaves = NT / kWave;
  __shared__ uint32_t smax[kWaves][B], smin[kWaves][B];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    // largest magnitude (as f32 bits) and 255 - the smallest biased exponent of a nonzero element
    uint32_t m = 0u, ne = 0u;
    for (int i = threadIdx.x; i < CX; i += NT) {
      const u32x4 v = xs[b * CXP + i];
      const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (e[q] << 16) & 0x7FFF0000u, hi = e[q] & 0x7FFF0000u;
        m = max(m, max(lo, hi));
        if (lo) ne = max(ne, 255u - (lo >> 23));
        if (hi) ne = max(ne, 255u - (hi >> 23));
      }
    }
    m = wave_max_u32(m);
    ne = wave_max_u32(ne);
    if (lane == 0) {
      smax[wave][b] = m;
      smin[wave][b] = ne;
    }
  }
  __syncthreads();
  bool exact = true;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    uint32_t m = 0u, ne = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      m = max(m, smax[w][b]);
      ne = max(ne, smin[w][b]);
    }
    // m < 2^(ef - 126) with ef its biased exponent: 2^(141 - ef) puts it in [2^14, 2^15)
    const int e = (m == 0u || m >= 0x7F800000u) ? 0 : 141 - (int)(m >> 23);
    // the smallest nonzero element scaled: biased exponent (255 - ne) + e >= 127 - 17
    exact = exact && m < 0x7F800000u && (m == 0u || (int)(255u - ne) + e >= 110);
    if (threadIdx.x == 0) xexp[b] = e;
    for (int i = threadIdx.x; i < CX; i += NT) {
      const u32x4 v = xs[b * CXP + i];
      const uint32_t ev[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const _Float16 lo = (_Float16)__builtin_ldexpf(bf16_lo(ev[q]), e);
        const _Float16 hi = (_Float16)__builtin_ldexpf(bf16_hi(ev[q]), e);
        o[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      xs[b * CXP + i] = u32x4{o[0], o[1], o[2], o[3]};
    }
  }
  return exact;
}

// The b vectors of a plain lm_head call, staged as the MFMA B operand: every
// 16-byte chunk of every vector is loaded into registers at once, and the
// first weight unit's loads (`after_loads`) go out only once they have
// arrived (issued together, the vectors' first-touch misses queued in HBM
// behind the whole grid's first weight units: ~8 us of staging at b = 8),
// then written to LDS once. For NVFP4 each vector is scaled by 2^e_b in
// registers and converted to F16 first (e_b from its largest magnitude, one
// block reduction for all vectors; the same check as stage_to_f16, whose
// result is returned).
template <int WD, int B, int NT, typename F>
__device__ __forceinline__ bool stage_x_mfma(const SweepParams &p, u32x4 *xs, int CX, int CXP, int *xexp,
                                             F &&after_loads) {
  constexpr int kWaves = NT / kWave;
  constexpr int QV = (1024 + NT - 1) / NT;  // chunks of a vector per thread (CX <= 1024)
  const u32x4 *xg = reinterpret_cast<const u32x4 *>(p.x);
  u32x4 xr[B][QV];
#pragma unroll
  for (int b = 0; b < B; ++b)
#pragma unroll
    for (int j = 0; j < QV; ++j) {
      xr[b][j] = xg[b * CX + min((int)threadIdx.x + j * NT, CX - 1)];  // unconditional (clamped; unused chunks ignored)
    }
  if constexpr (WD != kNVFP4) {
#pragma unroll
    for (int b = 0; b < B; ++b)
#pragma unroll
      for (int j = 0; j < QV; ++j) {
        const int c = (int)threadIdx.x + j * NT;
        if (c < CX) xs[b * CXP + c] = xr[b][j];
      }
    __builtin_amdgcn_sched_barrier(0);
    after_loads();
    return true;
  } else {
    __shared__ uint32_t smax[kWaves][B], smin[kWaves][B];
    const uint32_t lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    // per vector: the largest BF16 magnitude and the smallest nonzero one,
    // two elements per packed 16-bit max / min (a zero magnitude minus 1 wraps
    // to 0xFFFF, so zeros never win the min)
    uint32_t mx[B], mn[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      u16x2_t m2 = {0, 0}, z2 = {0xFFFF, 0xFFFF};
#pragma unroll
      for (int j = 0; j < QV; ++j) {
        const uint32_t e[4] = {xr[b][j].x, xr[b][j].y, xr[b][j].z, xr[b][j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u16x2_t mag = __builtin_bit_cast(u16x2_t, e[q] & 0x7FFF7FFFu);
          m2 = __builtin_elementwise_max(m2, mag);
          z2 = __builtin_elementwise_min(z2, mag - u16x2_t{1, 1});
        }
      }
      const uint32_t mmax = max((uint32_t)m2.x, (uint32_t)m2.y);
      const uint32_t zmin = min((uint32_t)z2.x, (uint32_t)z2.y);  // 0xFFFF: no nonzero element
      // as f32 bits, and 255 - the smallest biased exponent of a nonzero element (0 if none)
      mx[b] = mmax << 16;
      mn[b] = zmin == 0xFFFFu ? 0u : 255u - ((zmin + 1u) >> 7);
    }
    __builtin_amdgcn_sched_barrier(0);
    after_loads();  // the vectors have arrived: the weights may start
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < B; ++b) {
      mx[b] = wave_max_u32(mx[b]);
      mn[b] = wave_max_u32(mn[b]);
    }
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < B; ++b) {
        smax[wave][b] = mx[b];
        smin[wave][b] = mn[b];
      }
    }
    __syncthreads();
    // thread b reduces vector b over the waves, once for the block
    __shared__ int sok[B];
    if (threadIdx.x < B) {
      const int b = threadIdx.x;
      uint32_t m = 0u, ne = 0u;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        m = max(m, smax[w][b]);
        ne = max(ne, smin[w][b]);
      }
      // m < 2^(ef - 126) with ef its biased exponent: 2^(141 - ef) puts it in [2^14, 2^15)
      const int e = (m == 0u || m >= 0x7F800000u) ? 0 : 141 - (int)(m >> 23);
      // the smallest nonzero element scaled: biased exponent (255 - ne) + e >= 127 - 17
      xexp[b] = e;
      sok[b] = (m < 0x7F800000u && (m == 0u || (int)(255u - ne) + e >= 110)) ? 1 : 0;
    }
    __syncthreads();
    bool exact = true;
#pragma unroll
    for (int b = 0; b < B; ++b) {
      exact = exact && sok[b] != 0;
      const float sc = __builtin_ldexpf(1.0f, xexp[b]);  // exact power of 2
#pragma unroll
      for (int j = 0; j < QV; ++j) {
        const int c = (int)threadIdx.x + j * NT;
        if (c < CX) {
          const uint32_t ev[4] = {xr[b][j].x, xr[b][j].y, xr[b][j].z, xr[b][j].w};
          uint32_t o[4];
          // when exact, every scaled value is an F16 value: the convert does not round
#pragma unroll
          for (int q = 0; q < 4; ++q)
            o[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(ev[q]) * sc, bf16_hi(ev[q]) * sc));
          xs[b * CXP + c] = u32x4{o[0], o[1], o[2], o[3]};
        }
      }
    }
    return exact;
  }
}

// MASK: the grammar-masked argmax (p.masked), a compile-time copy of the body
// (see sweep_body).
template <int WD, int B, int J, int NT, bool MASK>
__device__ __forceinline__ void mfma_body(const SweepParams &p) {
  static_assert(J % 2 == 0 && J >= 4, "the NVFP4 scale dwords of a unit are split over the 4 lanes of a row");
  constexpr int kWaves = NT / kWave;
  constexpr int EPC = WT<WD>::kEPC;
  extern __shared__ u32x4 xs[];  // [B][CXP], then the waves' weight tiles
  __shared__ float sred[kWaves * kMaxRed];
  __shared__ int s_xexp[8];
  __shared__ unsigned s_next;
  __shared__ int s_last;

  const int k = p.k;
  const int C = k / EPC;  // weight chunks per row
  const int CX = k >> 3;  // 16-byte chunks per staged vector
  const int CXP = mfma_x_stride(CX);
  const int64_t row_bytes = (int64_t)C * 16;
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = (int)(lane & 15u);  // A: row within the tile; B and D: the vector
  const int grp = (int)(lane >> 4);   // A and B: k group; D: row quad
  static_assert(J == 8, "a load instruction covers 2 rows x 32 lanes");
  constexpr int kWS = mfma_tile_stride<J>();
  u32x4 *wtile = xs + B * CXP + wave * 16 * kWS;  // this wave's weight tile
  const int lr = (int)(lane >> 5), lc = (int)(lane & 31u);  // contiguous load: row pair half, chunk
  const bool live = col < B;
  const int64_t n = p.n;
  const int64_t ntiles = (n + 15) >> 4;
  const int npass = C / (4 * J);
  const bool want_lp = p.logprob_out != nullptr || p.conf_inout != nullptr;
  constexpr bool masked = MASK;
  float gs = 1.0f;
  if constexpr (WD == kNVFP4) gs = p.gscale[0];

  float best = -__builtin_inff(), ssum = 0.0f;
  int32_t bidx = -1;
  bool seen = false;
  // Q > 0: the block's tiles go round by round, G = W / Q tiles per round,
  // each tile's npass passes split over Q waves (wave g Q + m takes passes
  // m PQ .. m PQ + PQ - 1, PQ = npass / Q); the Q partial sums meet in LDS and
  // wave g Q adds them in wave order (with the row scale and mask word of
  // its own unit of the tile).
  const int Q = p.mfma_q;

  auto load_unit = [&](MUnit<J> &U, int64_t t, int ps) {
    int64_t row = t * 16 + col;
    row = row < n ? row : n - 1;
    // load jj: rows 2 jj and 2 jj + 1 of the tile, 512 contiguous bytes each
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      int64_t r = t * 16 + 2 * jj + lr;
      r = r < n ? r : n - 1;
      U.w[jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p.w + r * row_bytes) + ps * 4 * J + lc);
    }
    if constexpr (WD == kNVFP4) {
      // the unit's 2J scale dwords of the row: this lane takes dwords grp J/2 .. + J/2
      const uint32_t *sr = reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(p.scale) +
                                                              row * (int64_t)(k / 16)) +
                           ps * 2 * J + grp * (J / 2);
      if constexpr (J / 2 == 4) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(sr);
        U.sd[0] = v.x;
        U.sd[1] = v.y;
        U.sd[2] = v.z;
        U.sd[3] = v.w;
      } else {
#pragma unroll
        for (int i = 0; i < J / 2; ++i) U.sd[i] = sr[i];
      }
    }
    // FP8: row col's scale with every unit (one dword, unconditional, so every
    // unit leaves the same number of loads in flight and the waits before a
    // compute cover only the unit computed)
    if constexpr (WD == kFP8) U.rs = static_cast<const float *>(p.scale)[row];
    // the tile's mask word for this lane's column, with every unit (the same
    // word each pass: L2 hits; unconditional, as above): its index clamped
    // into the mask, or a weight word when the mask is empty
    if constexpr (masked) {
      int64_t wi = (t * 16) >> 5;  // the tile's 16 rows share one mask word
      wi = wi < p.mask_words ? wi : p.mask_words - 1;
      const int32_t *mp = p.mask_words > 0 ? p.mask + (int64_t)(live ? col : 0) * p.mask_words + wi
                                           : reinterpret_cast<const int32_t *>(p.w);
      const uint32_t v = (uint32_t)*mp;
      U.mw = live ? v : 0u;
    }
  };

  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // B operand rows: columns past b read a live vector's row (same address as
  // that column's lanes: a broadcast, no bank conflict) and are never reported
  const u32x4 *xb = xs + (col % B) * CXP;

  // MFMAs of the unit's chunk group jj (chunk 4 jj + grp of the unit in this
  // lane, `w`, already in the MFMA layout)
  auto mfma_group = [&](const MUnit<J> &U, const u32x4 &w, int ps, int jj) {
      const int c = ps * 4 * J + 4 * jj + grp;  // this lane's chunk of the row
      if constexpr (WD == kBF16) {
        const u32x4 bv = xb[c];
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w),
                                                      __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
      } else if constexpr (WD == kFP8) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t w0 = q ? w.z : w.x, w1 = q ? w.w : w.y;
          const u32x4 a = {fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
                           fp8x2_to_bf16x2<true>(w1)};
          const u32x4 bv = xb[2 * c + q];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                        __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
        }
      } else {
        // the chunk's two block scales: half (grp & 1) of unit dword 2 jj + grp / 2,
        // held as dword (2 jj) % (J/2) + grp / 2 by lane col + 16 ((2 jj) / (J/2))
        constexpr int H = J / 2;
        const int src = (col + 16 * ((2 * jj) / H)) * 4;
        const uint32_t v0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.sd[(2 * jj) % H]);
        const uint32_t v1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.sd[(2 * jj) % H + 1]);
        const uint32_t dw = (grp >> 1) ? v1 : v0;
        const uint32_t hw = (grp & 1) ? (dw >> 16) : dw;
        // both E4M3 scale bytes to F16 in one exact convert
        const f16x2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hw, 1.0f, false);
        const _Float16 s0 = s01[0], s1 = s01[1];
        const uint32_t wq[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const _Float16 sq = q < 2 ? s0 : s1;
          const f16x2_t sv = {sq, sq};
          const f16x2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wq[q], 1.0f, 0) * sv;
          const f16x2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wq[q], 1.0f, 1) * sv;
          const f16x2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wq[q], 1.0f, 2) * sv;
          const f16x2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(wq[q], 1.0f, 3) * sv;
          const u32x4 a = {__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                           __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)};
          const u32x4 bv = xb[4 * c + q];
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                       __builtin_bit_cast(f16x8_t, bv), acc, 0, 0, 0);
        }
      }
  };

  auto compute_unit = [&](const MUnit<J> &U, int ps) {
    // the unit in the MFMA layout: lane (row col, group grp) holds chunk 4 jj + grp of the unit
    u32x4 wa[J];
#pragma unroll
    for (int jj = 0; jj < J; ++jj) wtile[(2 * jj + lr) * kWS + lc] = U.w[jj];
#pragma unroll
    for (int jj = 0; jj < J; ++jj) wa[jj] = wtile[col * kWS + 4 * jj + grp];
#pragma unroll
    for (int jj = 0; jj < J; ++jj) mfma_group(U, wa[jj], ps, jj);
  };

  int xe = 0;  // NVFP4: the power of 2 this lane's vector was staged with
  auto finish_tile = [&](const MUnit<J> &U, int64_t t) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = t * 16 + 4 * grp + r;
      float val = acc[r];
      if constexpr (WD == kFP8)  // row 4 grp + r's scale, held by lane 4 grp + r
        val *= __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((4 * grp + r) * 4,
                                                                      __builtin_bit_cast(int, U.rs)));
      if constexpr (WD == kNVFP4) val = __builtin_ldexpf(val * gs, -xe);
      if (live && row < n) {
        if (p.logits) p.logits[(int64_t)col * n + row] = val;
        bool ok = true;
        if (masked) {
          ok = (row >> 5) < (int64_t)p.mask_words && ((U.mw >> (uint32_t)(row & 31)) & 1u);
          seen = seen || ok;
        }
        if (ok) {
          const float b0 = best;
          if (val > b0 || (val == b0 && (int32_t)row < bidx)) {
            best = val;
            bidx = (int32_t)row;
          }
          if (want_lp) {
            if (val > b0) ssum = ssum * __expf(b0 - val) + 1.0f;  // b0 = -inf: 0 * 0 + 1
            else if (val > -__builtin_inff()) ssum += __expf(val - b0);
            else if (val != val) ssum = val;  // NaN propagates
          }
        }
      }
    }
    acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  };

  // tiles of this block: i * gridDim.x + blockIdx.x for i = 0, 1, ..., wave w
  // starting with i = w and taking each next index from the LDS counter when
  // it needs that tile (at the loads of its first unit). Dealt round-robin
  // over the grid, every block gets the same number of tiles within one (in
  // rounds of W consecutive tiles per block it got a whole round more or
  // less: 32 or 40 at 154,880 rows), and the whole grid works on one window
  // of the head. Claimed when needed rather than a tile ahead (as the 8-wave
  // VALU sweep takes its short groups), no wave holds a tile in reserve while
  // others run dry: the block's last tiles go to whichever waves are free
  // (NVFP4 131,072 x 5,120: b = 4 68.1 -> 64.9 us, b = 8 70.2 -> 68.2).
  auto claim = [&]() -> unsigned {
    unsigned r = 0u;
    if (lane == 0u) r = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return r;
  };
  auto next_tile = [&]() -> int64_t {
    const unsigned i = __builtin_amdgcn_readfirstlane(claim());
    const int64_t ti = (int64_t)i * gridDim.x + blockIdx.x;
    return ti < ntiles ? ti : ntiles;
  };

  MUnit<J> ua, ub;
  int64_t t = (int64_t)wave * gridDim.x + blockIdx.x;
  int ps = 0;
  if (threadIdx.x == 0) s_next = kWaves;  // read after the staging barrier

  // the split schedule: unit u of this wave is pass m PQ + u % PQ of the
  // block's tile (u / PQ) G + g, tile i of the block being blockIdx.x + i
  // gridDim.x; units past the block's tiles load its last tile and are dropped
  const int QQ = Q > 0 ? Q : 1;
  const int G = kWaves / QQ, PQ = npass / QQ;
  const int gq = wave / QQ, mq = wave % QQ;
  const int64_t nb = (int64_t)blockIdx.x < ntiles ? (ntiles - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int64_t nunits = Q > 0 ? (nb + G - 1) / G * PQ : 0;  // the same for every wave of the block
  auto split_tile = [&](int64_t u) -> int64_t {
    const int64_t i = (u / PQ) * G + gq;
    return i < nb ? (int64_t)blockIdx.x + i * gridDim.x : -1;
  };
  auto split_load = [&](MUnit<J> &U, int64_t u) {
    const int64_t tt = split_tile(u);
    load_unit(U, tt >= 0 ? tt : (int64_t)blockIdx.x + (nb - 1) * gridDim.x, mq * PQ + (int)(u % PQ));
  };

  // the first unit's loads, issued behind the vectors' loads (they return
  // while the block stages). One unconditional call, its tile clamped into
  // the head (a wave with no tile loads one it never computes): on every path
  // the same loads are in flight behind the vectors', so the staging waits for
  // its own loads only, not for this unit as well.
  auto first_loads = [&]() {
    const int64_t i0 = gq < nb ? (int64_t)gq : nb - 1;
    int64_t t0 = Q > 0 ? (int64_t)blockIdx.x + i0 * gridDim.x : t;
    t0 = t0 < ntiles ? t0 : ntiles - 1;
    t0 = t0 > 0 ? t0 : 0;
    load_unit(ua, t0, Q > 0 ? mq * PQ : 0);
  };

  bool exact = true;
  if (p.u_in) {
    stage_final_norm<B, NT>(p, k, xs, CXP, sred, first_loads);  // the draft step: x = rms(u) per block
    if constexpr (WD == kNVFP4) {
      __syncthreads();
      exact = stage_to_f16<B, NT>(xs, CX, CXP, s_xexp);
    }
  } else {
    exact = stage_x_mfma<WD, B, NT>(p, xs, CX, CXP, s_xexp, first_loads);
  }
  if constexpr (WD == kNVFP4) {
    if (!exact) {
      // a vector F16 cannot hold exactly: the whole launch takes the VALU
      // sweep (every block reaches this branch; the weight loads issued above
      // complete unused)
      __syncthreads();
      sweep_body<WD, B, kArgmax, lm_rows<WD, B, true>(), WT<WD>::kJ, true, NT, MASK>(p);
      return;
    }
  }
  __syncthreads();
  if constexpr (WD == kNVFP4) xe = s_xexp[live ? col : 0];

  if (Q > 0) {
    // partial sums [2 rounds][W waves][64 lanes] after the weight tiles
    f32x4_t *spart = reinterpret_cast<f32x4_t *>(xs + B * CXP + kWaves * 16 * kWS);
    MUnit<J> fin;  // the adding wave's row scales and mask word for its tile
    auto split_compute = [&](const MUnit<J> &U, int64_t u) {
      const int pu = mq * PQ + (int)(u % PQ);
      compute_unit(U, pu);
      if (pu == 0) {
        fin.rs = U.rs;
        fin.mw = U.mw;
      }
      if ((int)(u % PQ) == PQ - 1) {
        // end of a round: every wave leaves its partial, then wave g Q adds
        // its tile's Q partials in wave order
        const int slot = (int)((u / PQ) & 1) * kWaves;
        spart[(slot + wave) * kWave + lane] = acc;
        acc = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        __syncthreads();
        const int64_t tt = split_tile(u);
        if (mq == 0 && tt >= 0) {
          f32x4_t sum = spart[(slot + gq * Q) * kWave + lane];
          for (int q = 1; q < Q; ++q) sum += spart[(slot + gq * Q + q) * kWave + lane];
          acc = sum;
          finish_tile(fin, tt);
        }
      }
    };
    int64_t u = 0;
    while (u < nunits) {
      if (u + 1 < nunits) {
        split_load(ub, u + 1);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the compute
        split_compute(ua, u);
      } else {
        split_compute(ua, u);
        break;
      }
      ++u;
      if (u + 1 < nunits) {
        split_load(ua, u + 1);
        __builtin_amdgcn_sched_barrier(0);
        split_compute(ub, u);
      } else {
        split_compute(ub, u);
        break;
      }
      ++u;
    }
    t = ntiles;  // the per-wave schedule below has nothing left
  }

  while (t < ntiles) {
    int64_t t1 = t;
    int ps1 = ps + 1;
    if (ps1 == npass) {
      ps1 = 0;
      t1 = next_tile();
    }
    if (t1 < ntiles) {
      load_unit(ub, t1, ps1);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the compute
      compute_unit(ua, ps);
      if (ps == npass - 1) finish_tile(ua, t);
    } else {
      compute_unit(ua, ps);
      if (ps == npass - 1) finish_tile(ua, t);
      break;
    }
    t = t1;
    ps = ps1;
    int64_t t2 = t;
    int ps2 = ps + 1;
    if (ps2 == npass) {
      ps2 = 0;
      t2 = next_tile();
    }
    if (t2 < ntiles) {
      load_unit(ua, t2, ps2);
      __builtin_amdgcn_sched_barrier(0);
      compute_unit(ub, ps);
      if (ps == npass - 1) finish_tile(ub, t);
    } else {
      compute_unit(ub, ps);
      if (ps == npass - 1) finish_tile(ub, t);
      break;
    }
    t = t2;
    ps = ps2;
  }

  argmax_publish<B, NT, true>(
      p, masked, want_lp,
      [&](int b) { return (col == b && bidx >= 0) ? argmax_key(best, (uint32_t)bidx) : 0ull; },
      [&](int b) { return col == b && seen; },
      [&](int b, float M) { return (col == b && ssum != 0.0f) ? ssum * __expf(best - M) : 0.0f; });
  // this thread's agent-coherent stores have completed before the ticket is taken
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = (__hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              gridDim.x - 1u);
  __syncthreads();
  if (!s_last) return;
  argmax_final<B, NT>(p, masked, want_lp);
  if (threadIdx.x == 0) __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int WD, int B, int J>
__global__ void __launch_bounds__(kMfmaThreads) __attribute__((amdgpu_waves_per_eu(2)))
lmhead_mfma_kernel(SweepParams p) {
  if (p.masked)
    mfma_body<WD, B, J, kMfmaThreads, true>(p);
  else
    mfma_body<WD, B, J, kMfmaThreads, false>(p);
}

// ------------------------------------------------------------------ host ----

// LDS of the split schedule's partial sums: 2 rounds x W waves x 64 lanes x 16 B.
constexpr int kMfmaPartBytes = 2 * kMfmaWaves * kWave * 16;

// Dynamic LDS of a launch: the staged vectors, the weight tiles and (q > 0)
// the partial sums, or for NVFP4 whichever of that and the VALU (fallback)
// layout is larger.
template <int WD>
inline int mfma_lds(int b, int k, int q = 0) {
  const int mf = b * mfma_x_stride(k >> 3) * 16 + mfma_tile_bytes<mfma_loads<WD>()>() +
                 (q > 0 ? kMfmaPartBytes : 0);
  const int va = b * (k * 2 + 16 * (WT<WD>::kEPC / 8));
  return (WD == kNVFP4 && va > mf) ? va : mf;
}

// Waves per tile of the split schedule for rows of k elements: 4 when the
// row's passes split evenly in 4, else for FP8 2 when they split in 2, and
// only when the partial sums fit beside 8 staged vectors (so the choice, and
// with it every row's summation order, does not depend on b); 0 keeps one
// wave per tile. Measured at 154,880 x 4,096, b = 8: FP8 one wave per tile
// 111.5 us, 2 waves 107.6 (101.1-101.2 with the current merge and staging),
// 4 waves 108.7 (100.6-100.7), 8 waves 115 (a barrier per round: the more
// waves per tile, the shorter the rounds); BF16 (128 KB tiles) 2 waves
// 196.0 us, 4 waves 185.1-185.3, 8 waves 185.3-185.7 (the VALU sweep
// 189.7-191.8); NVFP4 is slower split (66.7-67.0 us at one wave per tile,
// 73.0-73.2 with 2), its decode needing the waves free-running.
template <int WD>
inline int mfma_split_q(int k) {
  if (WD == kNVFP4) return 0;
  const int npass = (k / WT<WD>::kEPC) / (4 * mfma_loads<WD>());
  if (mfma_lds<WD>(8, k, 1) > kMfmaMaxLds) return 0;
  if (npass % 4 == 0) return 4;
  return (WD == kFP8 && npass % 2 == 0) ? 2 : 0;
}

// Whether the MFMA form takes a call: batch at least the format's threshold,
// rows a whole number of units, the staged vectors within the LDS budget.
template <int WD>
inline bool mfma_takes(int b, int k) {
  constexpr int J = mfma_loads<WD>();
  const int C = k / WT<WD>::kEPC;
  // BF16 only with the split schedule (its 16-row tiles are 16 passes long at
  // h = 4096: one wave per tile ends the launch one long tile at a time)
  if (WD == kBF16 && mfma_split_q<WD>(k) == 0) return false;
  return b >= mfma_min_b<WD>(k) && b >= 1 && b <= 8 && C > 0 && C % (4 * J) == 0 && mfma_lds<WD>(b, k) <= kMfmaMaxLds;
}

// 8 waves per CU: one 512-thread block or two 256-thread blocks (at most one
// block per W tiles).
template <int WD, int B>
static hipError_t launch_mfma_b(const SweepParams &p, hipStream_t s) {
  constexpr int J = mfma_loads<WD>();
  const void *fn = reinterpret_cast<const void *>(&lmhead_mfma_kernel<WD, B, J>);
  SweepParams ps = p;
  ps.mfma_q = mfma_split_q<WD>(p.k);
  const int lds = mfma_lds<WD>(B, p.k, ps.mfma_q);
  const int bpc = blocks_per_cu(fn, kMfmaThreads, lds);
  if (bpc <= 0) return hipErrorInvalidConfiguration;
  const int64_t tiles = (p.n + 15) / 16;
  const int64_t want = (tiles + kMfmaWaves - 1) / kMfmaWaves;
  int64_t cap = (int64_t)device_cu_count() * (512 / kMfmaThreads);
  if (cap > kSweepMaxGrid) cap = kSweepMaxGrid;
  const int grid = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL((lmhead_mfma_kernel<WD, B, J>), dim3(grid > 0 ? grid : 1), dim3(kMfmaThreads), lds, s, ps);
  return hipGetLastError();
}

template <int WD>
static hipError_t launch_mfma_wd(int b, const SweepParams &p, hipStream_t s) {
  switch (b) {
    case 1: return launch_mfma_b<WD, 1>(p, s);
    case 2: return launch_mfma_b<WD, 2>(p, s);
    case 3: return launch_mfma_b<WD, 3>(p, s);
    case 4: return launch_mfma_b<WD, 4>(p, s);
    case 5: return launch_mfma_b<WD, 5>(p, s);
    case 6: return launch_mfma_b<WD, 6>(p, s);
    case 7: return launch_mfma_b<WD, 7>(p, s);
    case 8: return launch_mfma_b<WD, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Per-format instantiations (mfma_*.hip).
hipError_t launch_mfma_bf16(int b, const SweepParams &p, hipStream_t s);
hipError_t launch_mfma_fp8(int b, const SweepParams &p, hipStream_t s);
hipError_t launch_mfma_nvfp4(int b, const SweepParams &p, hipStream_t s);

}  // namespace mtp
