// The combine (embedding gather, the two input RMSNorms, concat, fc [h, 2h],
// final RMSNorm) for wide batches, with the fc on the matrix cores
// (deepseek_v4_mtp.rs `forward_one` steps 1, 2 and 6; mtp_head/new.rs
// `fc=[h, 2h]`).
//
// The VALU combine dots every 16-byte fc chunk with the b staged concat
// vectors from LDS: at b = 8 that is 8 LDS reads per chunk and the combine
// runs at a fifth of HBM speed. Here the fc [n = h rows, k = 2h] goes through
// 16 x 16 x 32 BF16 MFMAs as in the matrix-core lm_head:
//   - one block per 16-row tile of fc (h / 16 blocks, 256 at h = 4096: one per
//     CU; taken only while the tiles fit one per CU), its 8 waves splitting
//     the tile's k range into 8 equal slices, so all of fc is requested at
//     once, as in the VALU combine;
//   - lane l reads row l % 16 of the tile, the four lanes of a row consecutive
//     16-byte chunks (k group l / 16); units of 8 loads per lane, two register
//     buffers; the concat vectors [b][2h] staged in LDS (row stride 1 mod 16
//     chunks) as the B operand, columns past b reading a live row;
//   - the 8 waves' 16 x b partial sums meet in LDS and are added in wave order
//     (the same order for every row and every call), rounded to BF16 as u and
//     stored with agent-scope stores; then, as in the VALU combine, either the
//     launch ends there (the draft step: the lm_head applies the final norm) or
//     the last block to take the ticket applies the final RMSNorm.
#pragma once
#include "mfma_impl.h"

namespace mtp {

constexpr int kCmThreads = 512;
constexpr int kCmWaves = kCmThreads / kWave;
constexpr int kCmJ = 8;  // loads per lane per unit: 512 bytes of each of the tile's 16 rows

// Smallest batch that takes the MFMA combine (from measurements at h = 4096:
// b = 2 20.3 us against 23.8 us, b = 8 33.1 us against 50.7 us standalone).
constexpr int kCmMinB = 2;

template <int B>
__device__ __forceinline__ void combine_mfma_body(const SweepParams &p) {
  constexpr int NT = kCmThreads, kWaves = kCmWaves, J = kCmJ;
  extern __shared__ u32x4 xs[];  // [B][CXP] concat vectors, k = 2h BF16
  __shared__ float sred[kWaves * kMaxRed];
  __shared__ float spart[kWaves][16][B];
  __shared__ int s_last;

  const int k = p.k;      // 2h
  const int C = k >> 3;   // 16-byte BF16 chunks per fc row (= per concat vector)
  const int CXP = mfma_x_stride(C);
  const int cw = C / kWaves;  // chunks of each row in one wave's k slice
  const int nunits = cw / (4 * J);
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int col = (int)(lane & 15u), grp = (int)(lane >> 4);
  const bool live = col < B;
  const int64_t n = p.n;
  const int64_t row0 = (int64_t)blockIdx.x * 16;
  int64_t row = row0 + col;
  row = row < n ? row : n - 1;
  const u32x4 *wr = reinterpret_cast<const u32x4 *>(p.w + row * (int64_t)C * 16) + wave * cw + grp;

  struct CUnit {
    u32x4 w[J];
  };
  auto load_unit = [&](CUnit &U, int u) {
#pragma unroll
    for (int jj = 0; jj < J; ++jj) U.w[jj] = __builtin_nontemporal_load(wr + u * 4 * J + 4 * jj);
  };
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const u32x4 *xb = xs + (col % B) * CXP + wave * cw;
  auto compute_unit = [&](const CUnit &U, int u) {
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const u32x4 bv = xb[u * 4 * J + 4 * jj + grp];
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, U.w[jj]),
                                                    __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
    }
  };

  // the first unit's loads go out with the first batch of concat loads
  CUnit ua, ub;
  stage_concat<B, NT>(p, k >> 1, xs, CXP, sred, [&] { load_unit(ua, 0); });
  __syncthreads();
  for (int u = 0; u < nunits; u += 2) {
    if (u + 1 < nunits) {
      load_unit(ub, u + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    compute_unit(ua, u);
    if (u + 1 >= nunits) break;
    if (u + 2 < nunits) {
      load_unit(ua, u + 2);
      __builtin_amdgcn_sched_barrier(0);
    }
    compute_unit(ub, u + 1);
  }

  // the waves' partial sums of the tile's 16 rows, added in wave order
  if (live) {
#pragma unroll
    for (int r = 0; r < 4; ++r) spart[wave][4 * grp + r][col] = acc[r];
  }
  __syncthreads();
  if (threadIdx.x < 16 * B) {
    const int ri = threadIdx.x / B, bv = threadIdx.x - ri * B;
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) s += spart[w][ri][bv];
    const int64_t r = row0 + ri;
    if (r < n)
      __hip_atomic_store(p.y + (int64_t)bv * n + r, (uint16_t)f32_to_bf16(s), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  // this thread's agent-coherent stores have completed before the ticket is taken
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (p.no_final) return;  // the draft step: the lm_head applies the final norm
  if (threadIdx.x == 0)
    s_last = (__hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              gridDim.x - 1u);
  __syncthreads();
  if (!s_last) return;
  combine_final_norm<B, NT>(p, sred);
  if (threadIdx.x == 0) __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int B>
__global__ void __launch_bounds__(kCmThreads) __attribute__((amdgpu_waves_per_eu(2)))
combine_mfma_kernel(SweepParams p) {
  combine_mfma_body<B>(p);
}

// ------------------------------------------------------------------ host ----

// Whether the MFMA combine takes a group of b batch rows with a BF16 fc [n, k]
// (n = k / 2 = h): b at least the threshold, each wave's k slice a whole
// number of units (h % 1024 == 0), at most one 16-row tile per CU (h = 8192
// needs two rounds of blocks and measured slower than the VALU combine), the
// concat vectors within the LDS budget.
inline bool combine_mfma_ok(int b, int k) {
  const int C = k >> 3;
  const int tiles = (k / 2 + 15) / 16;
  return b >= kCmMinB && b <= 8 && C % (kCmWaves * 4 * kCmJ) == 0 && tiles <= device_cu_count() &&
         b * mfma_x_stride(C) * 16 <= kMfmaMaxLds;
}

template <int B>
static hipError_t launch_combine_mfma_b(const SweepParams &p, hipStream_t s) {
  const void *fn = reinterpret_cast<const void *>(&combine_mfma_kernel<B>);
  const int lds = B * mfma_x_stride(p.k >> 3) * 16;
  if (blocks_per_cu(fn, kCmThreads, lds) <= 0) return hipErrorInvalidConfiguration;
  const int64_t tiles = (p.n + 15) / 16;
  hipLaunchKernelGGL((combine_mfma_kernel<B>), dim3((unsigned)tiles), dim3(kCmThreads), lds, s, p);
  return hipGetLastError();
}

hipError_t launch_combine_mfma(int b, const SweepParams &p, hipStream_t s);

}  // namespace mtp
