// Device helpers for the MTP draft-step kernels (gfx950, wave64).
//
// Number codecs (BF16, OCP E4M3FN, E2M1), wave-wide reductions built from DPP
// row permutes and the gfx950 permlane swaps, and the packed (value, index)
// key of the fused argmax.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------- BF16 ----

// A BF16 is the upper half of an f32 (deepseek_v4_mtp.rs,
// `argmax_grammar_masked`, the bf16 -> f32 step).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// f32 -> BF16, round to nearest, ties to even (subnormals kept; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x0040u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two f32 -> a BF16 pair (lo in bits 0..15), with gfx950's packed converter
// (v_cvt_pk_bf16_f32). On every one of the 2^32 f32 bit patterns it returns
// the same bits as f32_to_bf16 above (NaN included), so the two are
// interchangeable; the packed form is one instruction per pair where many
// values are converted at once.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// --------------------------------------------------------- E4M3 / E2M1 ----

// Round-half-even of an unsigned integer shifted right by s (1 <= s <= 31).
__device__ __forceinline__ uint32_t shr_rne(uint32_t m, uint32_t s) {
  uint32_t q = m >> s;
  uint32_t rem = m & ((1u << s) - 1u);
  uint32_t half = 1u << (s - 1u);
  return q + ((rem > half) || (rem == half && (q & 1u)));
}

// f32 -> OCP E4M3FN (bias 7, largest finite 448, S.1111.111 = NaN): nearest,
// ties to the even code, saturate (also +-inf) to +-448, sign bit kept, E4M3
// subnormals kept. Integer-only, so the result does not depend on any FP mode.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // >= 448: saturate
  uint32_t E = a >> 23;
  if (E >= 121u) {  // |v| >= 2^-6: E4M3 normal, keep 3 mantissa bits
    uint32_t q = a >> 20;
    uint32_t rem = a & 0xFFFFFu;
    q += (rem > 0x80000u) || (rem == 0x80000u && (q & 1u));
    return sign | (q - (120u << 3));  // rebias 127 -> 7; a carry moves the exponent
  }
  // E4M3 subnormal: m = round(|v| / 2^-9), |v| = M * 2^(Ee - 150)
  uint32_t M = (E == 0u) ? (a & 0x7FFFFFu) : ((a & 0x7FFFFFu) | 0x800000u);
  uint32_t Ee = (E == 0u) ? 1u : E;
  uint32_t s = 141u - Ee;      // >= 21
  if (s >= 25u) return sign;   // |v| < 2^-10 (M < 2^24): rounds to zero
  return sign | shr_rne(M, s); // 0..8 (8 is the smallest normal, code 0x08)
}

// f32 -> E2M1 (bias 1; 0 0.5 1 1.5 2 3 4 6): nearest, ties to the even code,
// saturate to 6, sign bit kept.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 28) & 0x8u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x40C00000u) return sign | 0x7u;  // >= 6, inf and NaN: saturate
  uint32_t E = a >> 23;
  if (E >= 127u) {  // |v| >= 1: normal, keep 1 mantissa bit
    uint32_t q = a >> 22;
    uint32_t rem = a & 0x3FFFFFu;
    q += (rem > 0x200000u) || (rem == 0x200000u && (q & 1u));
    return sign | (q - (126u << 1));
  }
  // subnormal: m = round(|v| / 0.5)
  uint32_t M = (E == 0u) ? (a & 0x7FFFFFu) : ((a & 0x7FFFFFu) | 0x800000u);
  uint32_t Ee = (E == 0u) ? 1u : E;
  uint32_t s = 149u - Ee;  // >= 23
  if (s >= 25u) return sign;
  return sign | shr_rne(M, s);  // 0, 1 or 2 (2 is 1.0, code 0x2)
}

// E4M3 code -> f32 (exact; the NaN code is never produced by the quantizers).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  return (c & 0x80u) ? -mag : mag;
}

// --------------------------------------------------------- conversions ----

// Byte SEL of `w` as an E4M3 code -> f32 (exact, subnormals kept).
template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// Two E4M3 codes (bytes 0,1 or 2,3 of `w`) -> two BF16 (exact: every E4M3 value
// is a BF16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// Two E2M1 codes (byte SEL of `w`: low nibble -> low half) -> two BF16 (exact).
template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w) {
  bf16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, r);
}

// acc + a.lo * b.lo + a.hi * b.hi for packed BF16 pairs.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// -------------------------------------------------------- wave reduce ----

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over the 64 lanes; every lane returns the same bits. Each step adds two
// disjoint partial sums that every lane of a group holds identically (IEEE add
// is commutative), so the tree is the same for every call site and value.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kQuadXor1>(v);
  v += dpp_f32<kQuadXor2>(v);
  v += dpp_f32<kRowHalfMirror>(v);
  v += dpp_f32<kRowMirror>(v);
  {
    auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kQuadXor1>(v));
  v = max(v, dpp_u32<kQuadXor2>(v));
  v = max(v, dpp_u32<kRowHalfMirror>(v));
  v = max(v, dpp_u32<kRowMirror>(v));
  {
    auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max((uint32_t)p[0], (uint32_t)p[1]);
  }
  {
    auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = max((uint32_t)p[0], (uint32_t)p[1]);
  }
  return v;
}

// Reduce-scatter of N per-lane partial sums over the wave in one butterfly:
// pairs of values meet across the two 32-lane halves (permlane32 swap), pairs
// of those across 16-lane rows (permlane16 swap), then each 16-lane row
// finishes its own value with four DPP steps. On return out[j] holds, in every
// lane of 16-lane row q, the full 64-lane sum of value 4j + row_slot(q)
// (row_slot = {0, 2, 1, 3}); slots past N hold zero. Every value is summed by
// the same tree ((x_i + x_{i+32}) + (x_{i+16} + x_{i+48}), then the 16-lane
// DPP tree), whatever N and its position, so identical inputs give identical
// bits. Cost: N/2 + N/4 swaps and 4 DPP adds per 4 values, against 6 steps
// per value for separate reductions.
template <int N>
__device__ __forceinline__ void wave_reduce_scatter(const float (&v)[N], float (&out)[(N + 3) / 4]) {
  constexpr int N2 = (N + 1) / 2, N4 = (N + 3) / 4;
  float h2[N2];
#pragma unroll
  for (int i = 0; i < N2; ++i) {
    const float a = v[2 * i];
    const float b = (2 * i + 1 < N) ? v[2 * i + 1] : 0.0f;
    auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    h2[i] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  }
#pragma unroll
  for (int j = 0; j < N4; ++j) {
    const float a = h2[2 * j];
    const float b = (2 * j + 1 < N2) ? h2[2 * j + 1] : 0.0f;
    auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    float q = __uint_as_float(s[0]) + __uint_as_float(s[1]);
    q += dpp_f32<kQuadXor1>(q);
    q += dpp_f32<kQuadXor2>(q);
    q += dpp_f32<kRowHalfMirror>(q);
    q += dpp_f32<kRowMirror>(q);
    out[j] = q;
  }
}

// Which value of each group of 4 a 16-lane row holds after wave_reduce_scatter.
__device__ __forceinline__ int row_slot(int lane) {
  const int q = lane >> 4;
  return q == 1 ? 2 : (q == 2 ? 1 : q);
}

// Max of 64-bit values over the four 16-lane rows (lanes l, l ^ 16, l ^ 32,
// l ^ 48), returned in every lane: two cross-row swaps of both halves.
__device__ __forceinline__ unsigned long long rows_max_u64(unsigned long long v) {
  {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    auto pl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    auto ph = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const unsigned long long a = ((unsigned long long)(uint32_t)ph[0] << 32) | (uint32_t)pl[0];
    const unsigned long long b = ((unsigned long long)(uint32_t)ph[1] << 32) | (uint32_t)pl[1];
    v = a > b ? a : b;
  }
  {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    auto pl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    auto ph = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const unsigned long long a = ((unsigned long long)(uint32_t)ph[0] << 32) | (uint32_t)pl[0];
    const unsigned long long b = ((unsigned long long)(uint32_t)ph[1] << 32) | (uint32_t)pl[1];
    v = a > b ? a : b;
  }
  return v;
}

// Lane `l`'s value of a 64-bit variable (wave-uniform result).
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}

// ------------------------------------------------------- argmax key ----

// Packs (value, index) so that the unsigned max picks the largest value and,
// among equal values, the lowest index. NaN is taken as -inf (never wins over
// a number) and -0 as +0 (equal to +0, so the lower index wins). Every real
// key is > 0, so 0 means "no row".
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t idx) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) u = 0xFF800000u;
  if (u == 0x80000000u) u = 0u;
  uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)ord << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}
// Key 1 is a marker (the grammar-masked argmax: rows were allowed, none had a
// value above -inf); like 0 it gives token 0.
__device__ __forceinline__ int32_t argmax_key_index(unsigned long long k) {
  return k <= 1ull ? 0 : (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}
// The value a key carries (-inf for the markers 0 and 1).
__device__ __forceinline__ float argmax_key_value(unsigned long long k) {
  if (k <= 1ull) return -__builtin_inff();
  const uint32_t ord = (uint32_t)(k >> 32);
  const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord;
  return __uint_as_float(u);
}

}  // namespace mtp
