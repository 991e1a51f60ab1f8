// Streaming GEMV sweep over row-major weight rows, for b <= 8 activation
// vectors at once, with two epilogues:
//   - argmax: the draft lm_head sweep with the fused (max, lowest index)
//     argmax (deepseek_v4_mtp.rs `forward_one` steps 6-7; the lm_head sweep is
//     most of the drafter's time per the draft-head comment in
//     glm5next_mtp_head/init.rs);
//   - store: the combine's fc GEMV (BF16 out) whose last block applies the final
//     RMSNorm (deepseek_v4_mtp.rs `forward_one` step 6; mtp_head/new.rs
//     `fc=[h, 2h]` and the fc_out / normed2 buffers).
//
// Layout and schedule (gfx950, wave64):
//   - The b activation vectors are staged once per block in LDS as 16-byte
//     chunks [b][k/8]; consecutive lanes read consecutive chunks (no bank
//     conflicts).
//   - Each wave owns groups of kR consecutive rows (grid-stride over groups).
//     For a row, lane l streams the 16-byte weight chunks l, l+64, ... with
//     non-temporal loads, kJ chunks per row per pass, all kR*kJ loads of a pass
//     issued before any use.
//   - Weights are decoded to packed BF16 in registers (FP8: exact hardware
//     convert; NVFP4: exact E2M1 convert, the E4M3 block scale applied to each
//     16-element partial sum) and multiplied with v_dot2 (f32 accumulate).
//   - One wave reduction per (row, vector) with DPP row permutes and the gfx950
//     permlane swaps; the row->lane mapping and the reduction tree are the same
//     for every row, so identical rows give bit-identical logits.
//   - Argmax: per-wave running best (strict '>' in ascending row order), then
//     per block as a packed 64-bit key; the last block to arrive (atomic
//     ticket) merges the per-block keys and writes the tokens.
//   - Cross-block hand-off without cache-wide maintenance: a block publishes
//     its partial results with agent-scope atomic stores (coherent per access
//     across the XCDs' separate L2s), waits for them to complete, then takes a
//     ticket; the last block reads the partials with agent-scope atomic loads.
//     A release/acquire fence pair per block would instead write back and
//     invalidate the block's whole L2, which on this part costs more than the
//     sweep itself.
#include "mtp_device.h"
#include "mtp_kernels.h"

namespace mtp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSweepThreads = 256;
constexpr int kSweepWaves = kSweepThreads / kWave;
constexpr int kR = 2;  // rows per wave iteration

enum SweepMode : int { kArgmax = 0, kStoreBf16 = 1 };

// Blocks per CU the sweep launches (fewer, longer-lived waves stream as fast as
// more, with less tail and merge work).
constexpr int kSweepBlocksPerCU = 2;

template <int WD> struct WT;
// kEPC: elements per 16-byte chunk; kJ: chunks per lane per row per pass.
template <> struct WT<kBF16> { static constexpr int kEPC = 8, kJ = 4; };
template <> struct WT<kFP8> { static constexpr int kEPC = 16, kJ = 4; };
template <> struct WT<kNVFP4> { static constexpr int kEPC = 32, kJ = 2; };

struct SweepParams {
  const uint16_t *x;  // [B, k] BF16
  const uint8_t *w;   // n rows of k elements
  const void *scale;  // FP8: f32 [n]; NVFP4: u8 [n, k/16]
  const float *gscale;
  int64_t n;
  int k;
  // argmax epilogue
  float *logits;  // NULL or [B, n]
  unsigned long long *partials;  // [gridDim.x][8] per-block keys
  unsigned *ticket;
  int32_t *token_out;
  // store epilogue + final norm
  uint16_t *y;  // [B, n] BF16
  const uint16_t *gamma_f;
  float eps, gamma_offset;
  uint16_t *x_out;  // [B, n]
};

template <int WD, int B>
__device__ __forceinline__ void chunk_dot(const u32x4 (&wv)[kR], const uint32_t (&sv)[kR],
                                          const u32x4 *__restrict__ xs, int CX, int c,
                                          float (&acc)[kR][B]) {
  if constexpr (WD == kBF16) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const u32x4 xv = xs[b * CX + c];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        float a = acc[r][b];
        a = dot2_bf16(wv[r].x, xv.x, a);
        a = dot2_bf16(wv[r].y, xv.y, a);
        a = dot2_bf16(wv[r].z, xv.z, a);
        a = dot2_bf16(wv[r].w, xv.w, a);
        acc[r][b] = a;
      }
    }
  } else if constexpr (WD == kFP8) {
    uint32_t d[kR][8];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      d[r][0] = fp8x2_to_bf16x2<false>(wv[r].x);
      d[r][1] = fp8x2_to_bf16x2<true>(wv[r].x);
      d[r][2] = fp8x2_to_bf16x2<false>(wv[r].y);
      d[r][3] = fp8x2_to_bf16x2<true>(wv[r].y);
      d[r][4] = fp8x2_to_bf16x2<false>(wv[r].z);
      d[r][5] = fp8x2_to_bf16x2<true>(wv[r].z);
      d[r][6] = fp8x2_to_bf16x2<false>(wv[r].w);
      d[r][7] = fp8x2_to_bf16x2<true>(wv[r].w);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const u32x4 x0 = xs[b * CX + 2 * c];
      const u32x4 x1 = xs[b * CX + 2 * c + 1];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        float a = acc[r][b];
        a = dot2_bf16(d[r][0], x0.x, a);
        a = dot2_bf16(d[r][1], x0.y, a);
        a = dot2_bf16(d[r][2], x0.z, a);
        a = dot2_bf16(d[r][3], x0.w, a);
        a = dot2_bf16(d[r][4], x1.x, a);
        a = dot2_bf16(d[r][5], x1.y, a);
        a = dot2_bf16(d[r][6], x1.z, a);
        a = dot2_bf16(d[r][7], x1.w, a);
        acc[r][b] = a;
      }
    }
  } else {
    uint32_t d[kR][16];
    float s0[kR], s1[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      d[r][0] = fp4x2_to_bf16x2<0>(wv[r].x);
      d[r][1] = fp4x2_to_bf16x2<1>(wv[r].x);
      d[r][2] = fp4x2_to_bf16x2<2>(wv[r].x);
      d[r][3] = fp4x2_to_bf16x2<3>(wv[r].x);
      d[r][4] = fp4x2_to_bf16x2<0>(wv[r].y);
      d[r][5] = fp4x2_to_bf16x2<1>(wv[r].y);
      d[r][6] = fp4x2_to_bf16x2<2>(wv[r].y);
      d[r][7] = fp4x2_to_bf16x2<3>(wv[r].y);
      d[r][8] = fp4x2_to_bf16x2<0>(wv[r].z);
      d[r][9] = fp4x2_to_bf16x2<1>(wv[r].z);
      d[r][10] = fp4x2_to_bf16x2<2>(wv[r].z);
      d[r][11] = fp4x2_to_bf16x2<3>(wv[r].z);
      d[r][12] = fp4x2_to_bf16x2<0>(wv[r].w);
      d[r][13] = fp4x2_to_bf16x2<1>(wv[r].w);
      d[r][14] = fp4x2_to_bf16x2<2>(wv[r].w);
      d[r][15] = fp4x2_to_bf16x2<3>(wv[r].w);
      s0[r] = e4m3_to_f32(sv[r] & 0xFFu);
      s1[r] = e4m3_to_f32((sv[r] >> 8) & 0xFFu);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const u32x4 x0 = xs[b * CX + 4 * c];
      const u32x4 x1 = xs[b * CX + 4 * c + 1];
      const u32x4 x2 = xs[b * CX + 4 * c + 2];
      const u32x4 x3 = xs[b * CX + 4 * c + 3];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        float p0 = dot2_bf16(d[r][0], x0.x, 0.0f);
        p0 = dot2_bf16(d[r][1], x0.y, p0);
        p0 = dot2_bf16(d[r][2], x0.z, p0);
        p0 = dot2_bf16(d[r][3], x0.w, p0);
        p0 = dot2_bf16(d[r][4], x1.x, p0);
        p0 = dot2_bf16(d[r][5], x1.y, p0);
        p0 = dot2_bf16(d[r][6], x1.z, p0);
        p0 = dot2_bf16(d[r][7], x1.w, p0);
        float p1 = dot2_bf16(d[r][8], x2.x, 0.0f);
        p1 = dot2_bf16(d[r][9], x2.y, p1);
        p1 = dot2_bf16(d[r][10], x2.z, p1);
        p1 = dot2_bf16(d[r][11], x2.w, p1);
        p1 = dot2_bf16(d[r][12], x3.x, p1);
        p1 = dot2_bf16(d[r][13], x3.y, p1);
        p1 = dot2_bf16(d[r][14], x3.z, p1);
        p1 = dot2_bf16(d[r][15], x3.w, p1);
        float a = acc[r][b];
        a = __builtin_fmaf(p0, s0[r], a);
        a = __builtin_fmaf(p1, s1[r], a);
        acc[r][b] = a;
      }
    }
  }
}

// Block-wide f32 sum (all threads get the result). `red` holds kSweepWaves floats.
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.0f;
#pragma unroll
  for (int i = 0; i < kSweepWaves; ++i) t += red[i];
  return t;
}

template <int WD, int B, int MODE>
__global__ void __launch_bounds__(kSweepThreads) sweep_kernel(SweepParams p) {
  constexpr int EPC = WT<WD>::kEPC;
  constexpr int kJ = WT<WD>::kJ;
  extern __shared__ u32x4 xs[];  // [B][k/8]
  __shared__ unsigned long long skeys[kSweepWaves][B];
  __shared__ float sred[kSweepWaves];
  __shared__ int s_last;

  const int k = p.k;
  const int CX = k >> 3;
  const int C = k / EPC;
  const int64_t row_bytes = (int64_t)C * 16;
  {
    const u32x4 *xg = reinterpret_cast<const u32x4 *>(p.x);
    for (int i = threadIdx.x; i < B * CX; i += kSweepThreads) xs[i] = xg[i];
  }
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int64_t ngroups = (p.n + kR - 1) / kR;
  const int npass = (C + kWave * kJ - 1) / (kWave * kJ);

  float best[B];
  int32_t bidx[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    best[b] = -__builtin_inff();
    bidx[b] = -1;
  }
  float gs = 1.0f;
  if constexpr (WD == kNVFP4) gs = p.gscale[0];

  for (int64_t g = (int64_t)blockIdx.x * kSweepWaves + wave; g < ngroups;
       g += (int64_t)gridDim.x * kSweepWaves) {
    const int64_t r0 = g * kR;
    float acc[kR][B];
#pragma unroll
    for (int r = 0; r < kR; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) acc[r][b] = 0.0f;

    for (int pass = 0; pass < npass; ++pass) {
      u32x4 wv[kJ][kR];
      uint32_t sv[kJ][kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int64_t row = r0 + r;
        const bool rok = row < p.n;
        const u32x4 *wr = reinterpret_cast<const u32x4 *>(p.w + (rok ? row : 0) * row_bytes);
        const uint16_t *sr = nullptr;
        if constexpr (WD == kNVFP4)
          sr = reinterpret_cast<const uint16_t *>(static_cast<const uint8_t *>(p.scale) +
                                                  (rok ? row : 0) * (int64_t)(k / 16));
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
          const int c = pass * (kWave * kJ) + j * kWave + lane;
          if (rok && c < C) {
            wv[j][r] = __builtin_nontemporal_load(wr + c);
            if constexpr (WD == kNVFP4) sv[j][r] = sr[c];
            else sv[j][r] = 0u;
          } else {
            wv[j][r] = u32x4{0u, 0u, 0u, 0u};
            sv[j][r] = 0u;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int c = pass * (kWave * kJ) + j * kWave + lane;
        const int cc = c < C ? c : 0;  // idle lanes read a valid chunk, times zero weights
        chunk_dot<WD, B>(wv[j], sv[j], xs, CX, cc, acc);
      }
    }

#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int64_t row = r0 + r;
      if (row < p.n) {
        float rs = gs;
        if constexpr (WD == kFP8) rs = static_cast<const float *>(p.scale)[row];
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float v = wave_sum(acc[r][b]);
          if constexpr (WD != kBF16) v *= rs;
          if constexpr (MODE == kArgmax) {
            if (p.logits && lane == b) p.logits[(int64_t)b * p.n + row] = v;
            if (v > best[b]) {
              best[b] = v;
              bidx[b] = (int32_t)row;
            }
          } else {
            if (lane == b)
              __hip_atomic_store(p.y + (int64_t)b * p.n + row, (uint16_t)f32_to_bf16(v), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
  }

  if constexpr (MODE == kArgmax) {
    if (lane == 0) {
#pragma unroll
      for (int b = 0; b < B; ++b)
        skeys[wave][b] = bidx[b] >= 0 ? argmax_key(best[b], (uint32_t)bidx[b]) : 0ull;
    }
    __syncthreads();
    if (threadIdx.x < B) {
      unsigned long long kmax = 0ull;
#pragma unroll
      for (int i = 0; i < kSweepWaves; ++i) kmax = max(kmax, skeys[i][threadIdx.x]);
      __hip_atomic_store(p.partials + (int64_t)blockIdx.x * 8 + threadIdx.x, kmax, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // this thread's agent-coherent stores have completed before the ticket is taken
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = (__hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              gridDim.x - 1u);
  __syncthreads();
  if (!s_last) return;

  if constexpr (MODE == kArgmax) {
    // max over the per-block keys, per batch row
    for (int b = 0; b < B; ++b) {
      unsigned long long k = 0ull;
      for (int i = threadIdx.x; i < (int)gridDim.x; i += kSweepThreads)
        k = max(k, __hip_atomic_load(p.partials + (int64_t)i * 8 + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      k = max(k, (unsigned long long)__shfl_xor(k, 1));
      k = max(k, (unsigned long long)__shfl_xor(k, 2));
      k = max(k, (unsigned long long)__shfl_xor(k, 4));
      k = max(k, (unsigned long long)__shfl_xor(k, 8));
      k = max(k, (unsigned long long)__shfl_xor(k, 16));
      k = max(k, (unsigned long long)__shfl_xor(k, 32));
      if (lane == 0) skeys[wave][b] = k;
    }
    __syncthreads();
    if (threadIdx.x < B) {
      unsigned long long k = 0ull;
#pragma unroll
      for (int i = 0; i < kSweepWaves; ++i) k = max(k, skeys[i][threadIdx.x]);
      p.token_out[threadIdx.x] = argmax_key_index(k);
    }
  } else {
    // final RMSNorm of the B fc outputs: x = bf16(u / sqrt(mean(u^2) + eps) * (g + off))
    const int n = (int)p.n;
    for (int b = 0; b < B; ++b) {
      const uint16_t *u = p.y + (int64_t)b * n;
      float ss = 0.0f;
      for (int i = threadIdx.x; i < n; i += kSweepThreads) {
        const float t = bf16_to_f32(__hip_atomic_load(u + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        ss = __builtin_fmaf(t, t, ss);
      }
      ss = block_sum(ss, sred);
      const float r = 1.0f / __builtin_sqrtf(ss / (float)n + p.eps);
      for (int i = threadIdx.x; i < n; i += kSweepThreads) {
        const float g = bf16_to_f32(p.gamma_f[i]) + p.gamma_offset;
        const float t = bf16_to_f32(__hip_atomic_load(u + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        p.x_out[(int64_t)b * n + i] = (uint16_t)f32_to_bf16((t * r) * g);
      }
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// -------------------------------------------------------- combine pre-norms ----

struct PrenormParams {
  const uint16_t *embed;
  int32_t tokens[8];
  const uint16_t *hidden;
  const uint16_t *gamma_e, *gamma_h;
  int h;
  float eps, gamma_offset;
  uint16_t *c;  // [B, 2h]: embedding half first
};

// Block (which, b): which 0 normalizes the embedding row E[t_b], which 1 the
// target hidden h_b; BF16 out into the concat buffer.
__global__ void __launch_bounds__(kSweepThreads) prenorm_kernel(PrenormParams p) {
  __shared__ float sred[kSweepWaves];
  const int which = blockIdx.x, b = blockIdx.y, h = p.h;
  const uint16_t *src = which == 0 ? p.embed + (int64_t)p.tokens[b] * h : p.hidden + (int64_t)b * h;
  const uint16_t *gam = which == 0 ? p.gamma_e : p.gamma_h;
  uint16_t *dst = p.c + (int64_t)b * 2 * h + (int64_t)which * h;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < h; i += kSweepThreads) {
    const float t = bf16_to_f32(src[i]);
    ss = __builtin_fmaf(t, t, ss);
  }
  ss = block_sum(ss, sred);
  const float r = 1.0f / __builtin_sqrtf(ss / (float)h + p.eps);
  for (int i = threadIdx.x; i < h; i += kSweepThreads) {
    const float g = bf16_to_f32(gam[i]) + p.gamma_offset;
    dst[i] = (uint16_t)f32_to_bf16((bf16_to_f32(src[i]) * r) * g);
  }
}

// ------------------------------------------------------------------ host ----

template <int WD, int B, int MODE>
static hipError_t launch_sweep_t(const SweepParams &p, hipStream_t s) {
  const void *fn = reinterpret_cast<const void *>(&sweep_kernel<WD, B, MODE>);
  const int lds = B * p.k * 2;
  const int bpc = blocks_per_cu(fn, kSweepThreads, lds);
  if (bpc <= 0) return hipErrorInvalidConfiguration;
  const int64_t groups = (p.n + kR - 1) / kR;
  const int64_t want = (groups + kSweepWaves - 1) / kSweepWaves;
  const int64_t per_cu = bpc < kSweepBlocksPerCU ? bpc : kSweepBlocksPerCU;
  int64_t cap = (int64_t)device_cu_count() * per_cu;
  if (cap > kSweepMaxGrid) cap = kSweepMaxGrid;
  const int grid = (int)(want < cap ? want : cap);
  hipLaunchKernelGGL((sweep_kernel<WD, B, MODE>), dim3(grid > 0 ? grid : 1), dim3(kSweepThreads),
                     lds, s, p);
  return hipGetLastError();
}

template <int WD, int MODE>
static hipError_t launch_sweep_b(int b, const SweepParams &p, hipStream_t s) {
  switch (b) {
    case 1: return launch_sweep_t<WD, 1, MODE>(p, s);
    case 2: return launch_sweep_t<WD, 2, MODE>(p, s);
    case 3: return launch_sweep_t<WD, 3, MODE>(p, s);
    case 4: return launch_sweep_t<WD, 4, MODE>(p, s);
    case 5: return launch_sweep_t<WD, 5, MODE>(p, s);
    case 6: return launch_sweep_t<WD, 6, MODE>(p, s);
    case 7: return launch_sweep_t<WD, 7, MODE>(p, s);
    case 8: return launch_sweep_t<WD, 8, MODE>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lmhead(const LmheadLaunch &a, hipStream_t s) {
  SweepParams p{};
  p.x = a.x;
  p.w = static_cast<const uint8_t *>(a.w);
  p.scale = a.scale;
  p.gscale = a.gscale;
  p.n = a.n;
  p.k = a.h;
  p.logits = a.logits;
  p.ticket = static_cast<unsigned *>(a.ws);
  p.partials = reinterpret_cast<unsigned long long *>(static_cast<uint8_t *>(a.ws) + 256);
  p.token_out = a.token_out;
  switch (a.wd) {
    case kBF16: return launch_sweep_b<kBF16, kArgmax>(a.b, p, s);
    case kFP8: return launch_sweep_b<kFP8, kArgmax>(a.b, p, s);
    case kNVFP4: return launch_sweep_b<kNVFP4, kArgmax>(a.b, p, s);
    default: return hipErrorInvalidValue;
  }
}

// Combine workspace: ticket u32 at 0; concat c [b, 2h] BF16 at 256; fc output
// u [b, h] BF16 after it (256-byte aligned).
size_t combine_ws_bytes(int64_t b, int64_t h) {
  const size_t c_bytes = (size_t)(b * 2 * h * 2 + 255) / 256 * 256;
  const size_t u_bytes = (size_t)(b * h * 2 + 255) / 256 * 256;
  return 256 + c_bytes + u_bytes;
}

hipError_t launch_combine(const CombineLaunch &a, hipStream_t s) {
  const int b = a.b, h = a.h;
  uint8_t *ws = static_cast<uint8_t *>(a.ws);
  unsigned *ticket = reinterpret_cast<unsigned *>(ws);
  uint16_t *c = reinterpret_cast<uint16_t *>(ws + 256);
  uint16_t *u = reinterpret_cast<uint16_t *>(ws + 256 + (size_t)(b * 2 * h * 2 + 255) / 256 * 256);

  PrenormParams pp{};
  pp.embed = a.embed;
  for (int i = 0; i < 8; ++i) pp.tokens[i] = a.tokens[i];
  pp.hidden = a.hidden;
  pp.gamma_e = a.gamma_e;
  pp.gamma_h = a.gamma_h;
  pp.h = h;
  pp.eps = a.eps;
  pp.gamma_offset = a.gamma_offset;
  pp.c = c;
  hipLaunchKernelGGL(prenorm_kernel, dim3(2, b), dim3(kSweepThreads), 0, s, pp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // fc + final norm, in groups of batch rows whose concat vectors fit in LDS
  const int k = 2 * h;
  int bp = kMaxSweepLds / (k * 2);
  if (bp > 8) bp = 8;
  if (bp < 1) return hipErrorInvalidValue;
  for (int b0 = 0; b0 < b; b0 += bp) {
    const int nb = (b - b0) < bp ? (b - b0) : bp;
    SweepParams p{};
    p.x = c + (int64_t)b0 * k;
    p.w = reinterpret_cast<const uint8_t *>(a.fc);
    p.n = h;
    p.k = k;
    p.ticket = ticket;
    p.y = u + (int64_t)b0 * h;
    p.gamma_f = a.gamma_f;
    p.eps = a.eps;
    p.gamma_offset = a.gamma_offset;
    p.x_out = a.x_out + (int64_t)b0 * h;
    e = launch_sweep_b<kBF16, kStoreBf16>(nb, p, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mtp
