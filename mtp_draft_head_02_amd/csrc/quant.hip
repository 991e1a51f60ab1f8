// Load-time weight quantizers: BF16 -> FP8 E4M3 with a per-row f32 scale, and
// BF16 -> NVFP4 (global absmax pass, then E2M1 codes with an E4M3 scale per 16
// elements and one f32 global scale). The pages run these as
// `quantize_bf16_to_fp8`, `nvfp4_global_absmax` and `quantize_bf16_to_nvfp4`
// (mtp_head/new.rs, `MtpHead::new`; mtp_head.rs, `quantize_proj`) without
// printing a recipe; the recipe here is this library's reading, computed with
// IEEE f32 division and multiplies and integer-only encoders so that the codes
// are reproducible bit for bit.
#include "mtp_device.h"
#include "mtp_kernels.h"

namespace mtp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kQThreads = 256;
constexpr int kQWaves = kQThreads / kWave;
constexpr int kFp8MaxChunks = 65536 / 8 / kWave;  // 16-byte chunks per lane for k <= 65536

// |bf16| bits of the larger-magnitude half of each pair, as an integer that
// orders like the magnitude (finite inputs).
__device__ __forceinline__ uint32_t absmax_pair(uint32_t v) {
  return max(v & 0x7FFFu, (v >> 16) & 0x7FFFu);
}

// FP8: one wave per row. Pass 1: exact |w| max (integer max of magnitude
// bits). s = f32(a / 448), 1 for an all-zero row. Pass 2: code = E4M3(w / s).
__global__ void __launch_bounds__(kQThreads) quant_fp8_kernel(const uint16_t *__restrict__ w,
                                                              int64_t n, int k,
                                                              uint8_t *__restrict__ codes,
                                                              float *__restrict__ scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kQWaves + threadIdx.x / kWave;
  if (row >= n) return;  // whole wave leaves; no block-wide sync below
  const u32x4 *wr = reinterpret_cast<const u32x4 *>(w + row * k);
  const int C = k >> 3;  // 8 BF16 per chunk
  uint32_t m = 0;
  for (int c = lane; c < C; c += kWave) {
    const u32x4 v = wr[c];
    m = max(m, max(max(absmax_pair(v.x), absmax_pair(v.y)), max(absmax_pair(v.z), absmax_pair(v.w))));
  }
  m = wave_max_u32(m);
  const float a = bf16_to_f32(m);
  const float sq = a / 448.0f;  // IEEE f32 division
  const float s = (m == 0u) ? 1.0f : sq;
  if (lane == 0) scale[row] = s;
  u32x2 *cr = reinterpret_cast<u32x2 *>(codes + row * k);
  for (int c = lane; c < C; c += kWave) {
    const u32x4 v = wr[c];
    const uint32_t e[4] = {v.x, v.y, v.z, v.w};
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = e4m3_encode(bf16_lo(e[i]) / s);
      const uint32_t hi = e4m3_encode(bf16_hi(e[i]) / s);
      out[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
    }
    cr[c] = u32x2{out[0], out[1]};
  }
}

__global__ void nvfp4_clear_kernel(uint32_t *ws) {
  if (threadIdx.x == 0 && blockIdx.x == 0) ws[0] = 0u;
}

// Exact global max of |w| over n*k BF16 (k % 256 == 0, so a whole number of
// 16-byte chunks), as BF16 magnitude bits, merged with atomicMax.
__global__ void __launch_bounds__(kQThreads) nvfp4_absmax_kernel(const uint16_t *__restrict__ w,
                                                                 int64_t chunks,
                                                                 uint32_t *__restrict__ ws) {
  const u32x4 *wc = reinterpret_cast<const u32x4 *>(w);
  uint32_t m = 0;
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < chunks;
       i += (int64_t)gridDim.x * kQThreads) {
    const u32x4 v = __builtin_nontemporal_load(wc + i);
    m = max(m, max(max(absmax_pair(v.x), absmax_pair(v.y)), max(absmax_pair(v.z), absmax_pair(v.w))));
  }
  m = wave_max_u32(m);
  if ((threadIdx.x & (kWave - 1)) == 0 && m) atomicMax(ws, m);
}

// One thread per 16-element block: sb = E4M3(a / d), S = e4m3(sb) * s_g,
// codes E2M1(w / S) packed low nibble first.
__global__ void __launch_bounds__(kQThreads) nvfp4_quant_kernel(const uint16_t *__restrict__ w,
                                                                int64_t nblocks, int k,
                                                                const uint32_t *__restrict__ ws,
                                                                uint8_t *__restrict__ codes,
                                                                uint8_t *__restrict__ bscale,
                                                                float *__restrict__ gscale) {
  const float G = bf16_to_f32(ws[0]);
  const float sgq = G / 2688.0f;  // 2688 = 6 * 448
  const float sg = (ws[0] == 0u) ? 1.0f : sgq;
  const float d = 6.0f * sg;
  const int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (i == 0) gscale[0] = sg;
  if (i >= nblocks) return;
  (void)k;  // blocks are contiguous in memory: block i covers elements 16i .. 16i+15
  const u32x4 *src = reinterpret_cast<const u32x4 *>(w) + 2 * i;
  const u32x4 v0 = src[0], v1 = src[1];
  const uint32_t e[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) m = max(m, absmax_pair(e[j]));
  const float a = bf16_to_f32(m);
  const uint32_t sb = e4m3_encode(a / d);
  const float S = e4m3_to_f32(sb) * sg;
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float lo = bf16_lo(e[j]), hi = bf16_hi(e[j]);
    uint32_t qlo, qhi;
    if (S == 0.0f) {
      qlo = (e[j] >> 12) & 0x8u;
      qhi = (e[j] >> 28) & 0x8u;
    } else {
      qlo = e2m1_encode(lo / S);
      qhi = e2m1_encode(hi / S);
    }
    out[j >> 2] |= (qlo | (qhi << 4)) << (8 * (j & 3));
  }
  reinterpret_cast<u32x2 *>(codes)[i] = u32x2{out[0], out[1]};
  bscale[i] = (uint8_t)sb;
}

// BF16 (codec 2) goes through the packed converter of the normalize passes:
// pattern i sits in the low half of the pair when i is even and in the high
// half when i is odd, its neighbour (or 0 past the end) in the other, so both
// halves are swept.
__global__ void __launch_bounds__(kQThreads) codec_range_kernel(int codec, uint32_t first,
                                                                int64_t count, uint8_t *out) {
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * kQThreads) {
    const float v = __uint_as_float(first + (uint32_t)i);
    if (codec == 2) {
      const int64_t i0 = i & ~(int64_t)1;
      const float lo = __uint_as_float(first + (uint32_t)i0);
      const float hi = i0 + 1 < count ? __uint_as_float(first + (uint32_t)(i0 + 1)) : 0.0f;
      const uint32_t pr = f32x2_to_bf16x2(lo, hi);
      reinterpret_cast<uint16_t *>(out)[i] = (uint16_t)((i & 1) ? (pr >> 16) : (pr & 0xFFFFu));
    } else {
      out[i] = (uint8_t)(codec == 0 ? e4m3_encode(v) : e2m1_encode(v));
    }
  }
}

static int grid_for(int64_t items, int per_block, int64_t cap) {
  int64_t g = (items + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return (int)(g > 0 ? g : 1);
}

hipError_t launch_quant_fp8(const uint16_t *w, int64_t n, int k, uint8_t *codes, float *scale,
                            hipStream_t s) {
  const int grid = (int)((n + kQWaves - 1) / kQWaves);
  hipLaunchKernelGGL(quant_fp8_kernel, dim3(grid), dim3(kQThreads), 0, s, w, n, k, codes, scale);
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4(const uint16_t *w, int64_t n, int k, uint8_t *codes,
                              uint8_t *block_scale, float *global_scale, void *ws, hipStream_t s) {
  uint32_t *amax = static_cast<uint32_t *>(ws);
  hipLaunchKernelGGL(nvfp4_clear_kernel, dim3(1), dim3(64), 0, s, amax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t chunks = n * (int64_t)k / 8;
  const int cap = device_cu_count() * 8;
  hipLaunchKernelGGL(nvfp4_absmax_kernel, dim3(grid_for(chunks, kQThreads, cap)), dim3(kQThreads), 0,
                     s, w, chunks, amax);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nblocks = n * (int64_t)k / 16;
  hipLaunchKernelGGL(nvfp4_quant_kernel, dim3(grid_for(nblocks, kQThreads, INT32_MAX)),
                     dim3(kQThreads), 0, s, w, nblocks, k, amax, codes, block_scale, global_scale);
  return hipGetLastError();
}

hipError_t launch_codec_range(int codec, uint32_t first_bits, int64_t count, uint8_t *out,
                              hipStream_t s) {
  const int cap = device_cu_count() * 16;
  hipLaunchKernelGGL(codec_range_kernel, dim3(grid_for(count, kQThreads, cap)), dim3(kQThreads), 0, s,
                     codec, first_bits, count, out);
  return hipGetLastError();
}

}  // namespace mtp
