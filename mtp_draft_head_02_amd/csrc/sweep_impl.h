// Streaming GEMV sweep over row-major weight rows, for b <= 8 activation
// vectors at once, with two epilogues:
//   - argmax: the draft lm_head sweep with the fused (max, lowest index)
//     argmax (deepseek_v4_mtp.rs `forward_one` steps 6-7; the lm_head sweep is
//     most of the drafter's time per the draft-head comment in
//     glm5next_mtp_head/init.rs);
//   - store: the whole combine in one launch. Every block first RMSNorms the
//     embedding row and the target hidden into its LDS concat (cheap, from L2,
//     identical bits in every block), streams its fc rows (BF16 out), and the
//     last block applies the final RMSNorm (deepseek_v4_mtp.rs `forward_one`
//     steps 1, 2 and 6; mtp_head/new.rs `fc=[h, 2h]` and the normed_embed,
//     normed_hidden, concat, fc_out, normed2 buffers).
//
// Layout and schedule (gfx950, wave64):
//   - The b activation vectors are staged once per block in LDS as 16-byte
//     chunks [b][k/8]; consecutive lanes read consecutive chunks (no bank
//     conflicts).
//   - Work comes in groups of kR consecutive rows. The combine and some
//     lm_head configurations split the groups statically (grid stride); the
//     other lm_head configurations run one 8-wave block per CU whose waves
//     take the block's groups (dealt to the blocks round-robin over the grid)
//     from an LDS counter, so faster waves take more.
//     For a row, lane l streams the 16-byte weight chunks l, l+64, ... with
//     non-temporal loads, kJ chunks per row per pass, all kR*kJ loads of a pass
//     issued before any use.
//   - Weights are decoded to packed BF16 in registers (FP8: exact hardware
//     convert; NVFP4: exact E2M1 convert, the E4M3 block scale applied to each
//     16-element partial sum) and multiplied with v_dot2 (f32 accumulate).
//   - Loads use a wave-uniform row base plus a fixed per-lane offset; the next
//     unit's loads are issued before the current unit is computed.
//   - One reduce-scatter per row group turns all kR*B per-lane partial sums
//     into full sums held by 16-lane rows (permlane32/16 swaps, then DPP); the
//     row->lane mapping and the reduction tree are the same for every row, so
//     identical rows give bit-identical logits.
//   - Argmax: each lane row keeps a running best for its (row-in-group,
//     vector) slots (larger value, then lower row), merged per vector as
//     packed 64-bit keys over the wave and the block; each block raises a
//     running maximum key per vector, and the last block to arrive (atomic
//     ticket) reads it and writes the tokens.
//   - Cross-block hand-off without cache-wide maintenance: a block publishes
//     with agent-scope atomics (coherent per access across the XCDs' separate
//     L2s: a 64-bit atomic max, or per-block stores when the log-probability
//     needs every block's own sums), waits for them to complete, then takes a
//     ticket; the last block reads with agent-scope atomics. A release/acquire
//     fence pair per block would instead write back and invalidate the
//     block's whole L2, which on this part costs more than the sweep itself.
#pragma once
#include "mtp_device.h"
#include "mtp_kernels.h"

namespace mtp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Block shapes. The lm_head runs one block per CU: either 8 waves that share
// the block's row groups at run time, or 4 waves with a static grid-stride
// split (see lm_threads); the combine runs 4-wave blocks, up to four per CU.
constexpr int kCombineThreads = 256;
constexpr int kCombineWaves = kCombineThreads / kWave;

// kStoreBf16: the concat combine (fc [h, 2h] in any weight format);
// kStoreSplit: the split combine, e_proj [h, h] and h_proj [h, h] (BF16), each
// branch's sum rounded to BF16 before the BF16 add.
enum SweepMode : int { kArgmax = 0, kStoreBf16 = 1, kStoreSplit = 2 };


template <int WD> struct WT;
// kEPC: elements per 16-byte chunk. For the lm_head sweep: kJ chunks per lane
// per row per pass (a 4 KB row pass per wave for BF16 and FP8, 2 KB of NVFP4
// codes plus their block scales).
template <> struct WT<kBF16> { static constexpr int kEPC = 8, kJ = 4; };
template <> struct WT<kFP8> { static constexpr int kEPC = 16, kJ = 4; };
template <> struct WT<kNVFP4> { static constexpr int kEPC = 32, kJ = 2; };
// (An NVFP4 pass of kJ chunks per lane has 32 kJ dwords of block scales per
// row, loaded as (kJ + 1) / 2 dwords per lane; the single-vector sweep takes
// kJ = 3 for ragged rows of 129..192 chunks, one pass per row.)

// Rows per group of the lm_head sweep (a unit is rows x kJ chunks per lane),
// from measurements at 154,880 x 4,096 and 131,072 x 5,120. Whole-pass rows at
// b = 1 (BF16: b <= 2) stream fastest in units of about 4 KB per wave: a
// plain streaming read on this part peaks near 32 KB in flight per CU (4
// waves x 8 KB or 8 waves x 4 KB) and loses up to 8 % with twice that. NVFP4
// keeps 16 decoded BF16 pairs per row in registers, so wide batches take 2
// rows; its ragged single-vector rows measured fastest with 4.
template <int WD, int B, bool RAGGED>
constexpr int lm_rows() {
  if (WD == kNVFP4) return (B == 1 && RAGGED) ? 4 : 2;
  if (!RAGGED && (B == 1 || (WD == kBF16 && B == 2))) return 1;
  return 2;
}

// The combine's fc GEMV ([h, 2h]): one row per wave, a whole 2h-long BF16 row
// (16 KB at h = 4096; FP8 8 KB) in flight per lane set in one pass (NVFP4 in
// two, the scale dword layout fixes J = 2), up to 4 blocks per CU as the
// occupancy allows (the BF16 fc at b = 1 fits 2: each wave then takes two rows
// of a 4096-row fc, the second requested after the staging).
constexpr int kFcR = 1, kFcBlocksPerCU = 4;
template <int WD>
constexpr int fc_chunks() { return WD == kBF16 ? 16 : (WD == kFP8 ? 8 : WT<kNVFP4>::kJ); }

struct SweepParams {
  const uint16_t *x;  // [B, k] BF16
  const uint8_t *w;   // n rows of k elements
  const void *scale;  // FP8: f32 [n]; NVFP4: u8 [n, k/16]
  const float *gscale;
  int64_t n;
  int k;
  // argmax epilogue
  float *logits;  // NULL or [B, n]
  unsigned long long *kmax;      // [8] running max key per vector (zero on entry and exit)
  unsigned long long *partials;  // [8][kSweepMaxGrid] per-block keys (top-1 log-probability only)
  float *psums;                  // [8][kSweepMaxGrid] per-block softmax sums (top-1 log-probability)
  unsigned *ticket;
  // lm_head options, off when NULL
  float *logprob_out;    // [B] top-1 log-probability
  float *conf_inout;     // [B] running minimum of the top-1 probability
  int masked;            // 1: only rows the mask allows take part
  const int32_t *mask;   // [B][mask_words] grammar bitmask (bit i % 32 of word i / 32 allows row i)
  int mask_words;
  int32_t *allowed_out;  // [B] 1 when the mask allowed a row, else 0
  int32_t *token_out;
  // store mode: in-block pre-norms (prologue), fc output, final norm
  const uint16_t *embed;         // [vocab, h]
  int32_t tokens[8];
  const int32_t *tokens_dev;     // NULL, or device token ids [B] (clamped into [0, vocab))
  int64_t vocab;
  const uint8_t *w2;             // split: h_proj rows (w holds e_proj rows)
  // the draft step (mtp_draft_step): the combine stops at u, each lm_head
  // block applies the final norm to u itself
  int no_final;           // combine: store u and stop (no ticket, no final norm)
  const uint16_t *u_in;   // lm_head: x = rms(u_in, gamma_f), staged per block
  int mfma_q;             // matrix-core lm_head: waves sharing a tile's passes (0: one wave per tile)
  const uint16_t *hidden;        // [B, h]
  const uint16_t *gamma_e, *gamma_h;
  uint16_t *y;  // [B, n] BF16 fc output (u)
  uint16_t *c_out;  // NULL, or [B, k] BF16: block 0 stores the concat it built (left in the workspace)
  const uint16_t *gamma_f;
  float eps, gamma_offset;
  uint16_t *x_out;  // [B, n]
};

// One 16-byte weight chunk per row of the unit (kR rows) against the B staged
// vectors: x points at the chunk's x (8 BF16 per 16 bytes, EPC/8 of them) in
// vector 0, vector b sits xstride chunks further. Accumulates into acc[r][b].
template <int WD, int B, int kR>
__device__ __forceinline__ void chunk_dot(const u32x4 (&wv)[kR], const uint32_t (&sv)[kR],
                                          const u32x4 *__restrict__ x, int xstride,
                                          float (&acc)[kR][B]) {
  if constexpr (WD == kBF16) {
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const u32x4 xv = x[b * xstride];
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
      const u32x4 x0 = x[b * xstride];
      const u32x4 x1 = x[b * xstride + 1];
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
      s0[r] = e4m3_byte_to_f32<0>(sv[r]);
      s1[r] = e4m3_byte_to_f32<1>(sv[r]);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const u32x4 x0 = x[b * xstride];
      const u32x4 x1 = x[b * xstride + 1];
      const u32x4 x2 = x[b * xstride + 2];
      const u32x4 x3 = x[b * xstride + 3];
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

// The weight bytes of one unit (kR rows x kJ chunks per lane); for NVFP4
// (kJ + 1) / 2 dwords per lane of each row's block scales for the pass (the
// pass's 2 * 64 * kJ scale bytes, in coalesced loads of one dword per lane);
// for FP8 the rows' f32 scales.
template <int kR, int kJ, int NS>
struct Unit {
  u32x4 w[kJ][kR];
  uint32_t sd[kR][(kJ + 1) / 2];
  float rs[kR];
  uint32_t mw[NS];  // grammar-mask words of this lane's (row, vector) slots (masked: every unit of a group)
};

// RMSNorm scales of N vectors from per-thread partial sums of squares:
// v[i] <- 1 / sqrt(S_i / n + eps), S_i the block-wide sum of v[i]. Each wave
// sums its lanes; the waves' partials meet in `red` (W * kMaxRed floats, W
// waves per block); lane i of every wave adds partial i over the waves in wave
// order and computes scale i, once per wave; the N scales are broadcast back
// with readlane. Every block and every thread gets the same bits.
constexpr int kMaxRed = 16;
template <int N, int W>
__device__ __forceinline__ void block_rms_scales(float (&v)[N], float *red, int n, float eps) {
  static_assert(N <= kMaxRed && N <= kWave, "one sum per lane");
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
  __syncthreads();
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) red[wave * kMaxRed + i] = v[i];
  }
  __syncthreads();
  const int li = lane < N ? lane : 0;
  float t = 0.0f;
#pragma unroll
  for (int w = 0; w < W; ++w) t += red[w * kMaxRed + li];
  const float r = 1.0f / __builtin_sqrtf(t / (float)n + eps);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(r), i));
}

__device__ __forceinline__ void sumsq_chunk(const u32x4 v, float &ss) {
  const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = bf16_lo(e[j]), hi = bf16_hi(e[j]);
    ss = __builtin_fmaf(lo, lo, ss);
    ss = __builtin_fmaf(hi, hi, ss);
  }
}

// y = bf16((v * r) * (g + off)) for the 8 BF16 of a chunk.
__device__ __forceinline__ u32x4 norm_chunk(const u32x4 v, const float (&g)[8], float r) {
  const uint32_t e[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = f32x2_to_bf16x2((bf16_lo(e[j]) * r) * g[2 * j], (bf16_hi(e[j]) * r) * g[2 * j + 1]);
  return u32x4{o[0], o[1], o[2], o[3]};
}

// The 8 gammas of a 16-byte BF16 chunk, as f32 with the offset added (g + off,
// one f32 add each, as the normalization uses them).
__device__ __forceinline__ void gamma_chunk(const u32x4 g, float off, float (&out)[8]) {
  const uint32_t gg[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = bf16_lo(gg[j]) + off;
    out[2 * j + 1] = bf16_hi(gg[j]) + off;
  }
}

// Largest h (multiple of 16, at most 8192) whose B concat vectors of 2h BF16
// (plus one zero chunk each) fit the sweep's LDS budget; the combine launch
// groups batch rows so that every group fits.
template <int B>
constexpr int combine_max_h() {
  const int h = ((kMaxSweepLds / B - 16) / 4) / 16 * 16;
  return h < 8192 ? h : 8192;
}
// Chunks of one h-long vector per thread, at most: 8 BF16 per 16-byte chunk.
template <int B, int NT = kCombineThreads>
constexpr int combine_chunks_per_thread() { return (combine_max_h<B>() / 8 + NT - 1) / NT; }

// The combine's concat, c_b = [rms(E[t_b]) (g_e + off) || rms(h_b) (g_h + off)]
// (embedding first, BF16 per element), built in the LDS vector slots. The raw
// vectors are loaded by batches of batch rows (at most 16 chunks per thread in
// flight), each thread summing the squares of what it loads; the 2B sums share
// one block reduction; each thread then normalizes its own chunks with gammas
// it loaded up front, from registers when all rows fit one batch, else from
// the raw copies it left in LDS (block 0 also stores them to p.c_out, when
// given: every block builds the same bits). `after_first` runs once the
// first batch's loads are issued (the caller issues its first weight loads
// there: loads complete in issue order, so data queued behind them would wait).
template <int B, int NT, typename F>
__device__ __forceinline__ void stage_concat(const SweepParams &p, int h, u32x4 *xs, int CXP, float *red,
                                             F &&after_first) {
  constexpr int Q = combine_chunks_per_thread<B, NT>();
  constexpr int G0 = 16 / (2 * Q) > 0 ? 16 / (2 * Q) : 1;
  constexpr int G = G0 < B ? G0 : B;  // batch rows per batch (at most 16 chunks per thread in flight)
  // All batch rows in one batch: the raw chunks stay in registers until they
  // are normalized (one LDS write each). Otherwise each batch goes to LDS raw
  // and is normalized there in place.
  constexpr bool kKeep = G == B;
  const int H8 = h >> 3;
  const u32x4 *ge = reinterpret_cast<const u32x4 *>(p.gamma_e);
  const u32x4 *gh = reinterpret_cast<const u32x4 *>(p.gamma_h);
  float ss[2 * B];
#pragma unroll
  for (int v = 0; v < 2 * B; ++v) ss[v] = 0.0f;
  u32x4 gev[Q], ghv[Q];
  u32x4 t[2 * G][Q];
#pragma unroll
  for (int b0 = 0; b0 < B; b0 += G) {
#pragma unroll
    for (int bb = 0; bb < G; ++bb) {
      const int b = b0 + bb;
      if (b < B) {
        int64_t tk = p.tokens[b];
        if (p.tokens_dev) {
          const int32_t d = p.tokens_dev[b];
          tk = d < 0 ? 0 : (d >= p.vocab ? p.vocab - 1 : d);
        }
        const u32x4 *e = reinterpret_cast<const u32x4 *>(p.embed + tk * h);
        const u32x4 *hv = reinterpret_cast<const u32x4 *>(p.hidden + (int64_t)b * h);
        // every load issued, unconditionally (indices clamped into the row;
        // chunks past it are never used), so they are in flight together
#pragma unroll
        for (int j = 0; j < Q; ++j) {
          const int c = min((int)threadIdx.x + j * NT, H8 - 1);
          t[2 * bb][j] = e[c];
          t[2 * bb + 1][j] = hv[c];
        }
      }
    }
    if (b0 == 0) {
#pragma unroll
      for (int j = 0; j < Q; ++j) {
        const int c = min((int)threadIdx.x + j * NT, H8 - 1);
        gev[j] = ge[c];
        ghv[j] = gh[c];
      }
      __builtin_amdgcn_sched_barrier(0);
      after_first();
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int bb = 0; bb < G; ++bb) {
      const int b = b0 + bb;
      if (b < B) {
#pragma unroll
        for (int j = 0; j < Q; ++j) {
          const int c = (int)threadIdx.x + j * NT;
          if (c < H8) {
            sumsq_chunk(t[2 * bb][j], ss[2 * b]);
            sumsq_chunk(t[2 * bb + 1][j], ss[2 * b + 1]);
            if constexpr (!kKeep) {
              xs[b * CXP + c] = t[2 * bb][j];
              xs[b * CXP + H8 + c] = t[2 * bb + 1][j];
            }
          }
        }
      }
    }
  }
  block_rms_scales<2 * B, NT / kWave>(ss, red, h, p.eps);
  u32x4 *cg = (p.c_out && blockIdx.x == 0) ? reinterpret_cast<u32x4 *>(p.c_out) : nullptr;
  // chunk-major, so a chunk's gammas are decoded once for all 2B vectors
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    const int c = (int)threadIdx.x + j * NT;
    if (c < H8) {
      float gef[8], ghf[8];
      gamma_chunk(gev[j], p.gamma_offset, gef);
      gamma_chunk(ghv[j], p.gamma_offset, ghf);
#pragma unroll
      for (int v = 0; v < 2 * B; ++v) {
        u32x4 *dst = xs + (v >> 1) * CXP + (v & 1) * H8;
        const u32x4 y = norm_chunk(kKeep ? t[v % (2 * G)][j] : dst[c], (v & 1) ? ghf : gef, ss[v]);
        dst[c] = y;
        if (cg) cg[(v >> 1) * 2 * H8 + (v & 1) * H8 + c] = y;
      }
    }
  }
}

// The draft step's x in the lm_head launch: x_b = rms(u_b, g_f) (BF16), with u
// written by the combine launch that ran before it on the same stream, read
// with agent-coherent 8-byte loads (all b vectors at once, one block reduction
// for the b sums), staged in the LDS vector slots; block 0 also writes x_out
// (when given). Same formula and summation order in every block, so every
// block stages the same bits. `after_loads` runs once the u and gamma loads
// are issued (the caller issues its first weight loads there, behind them).
template <int B, int NT, typename F>
__device__ __forceinline__ void stage_final_norm(const SweepParams &p, int h, u32x4 *xs, int CXP, float *red,
                                                 F &&after_loads) {
  constexpr int Q = 2 * combine_chunks_per_thread<B, NT>();  // 4-element quads per thread
  const int nq = h >> 2;
  unsigned long long q[B][Q], gq[Q];
  const unsigned long long *g = reinterpret_cast<const unsigned long long *>(p.gamma_f);
  // every load issued unconditionally (indices clamped; quads past the row are zeroed after)
#pragma unroll
  for (int j = 0; j < Q; ++j) gq[j] = g[min((int)threadIdx.x + j * NT, nq - 1)];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    const unsigned long long *u = reinterpret_cast<const unsigned long long *>(p.u_in + (int64_t)b * h);
#pragma unroll
    for (int j = 0; j < Q; ++j)
      q[b][j] = __hip_atomic_load(u + min((int)threadIdx.x + j * NT, nq - 1), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_sched_barrier(0);
  after_loads();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    if ((int)threadIdx.x + j * NT >= nq) {
      gq[j] = 0ull;
#pragma unroll
      for (int b = 0; b < B; ++b) q[b][j] = 0ull;
    }
  }
  float ss[B];
#pragma unroll
  for (int b = 0; b < B; ++b) {
    ss[b] = 0.0f;
#pragma unroll
    for (int j = 0; j < Q; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = bf16_to_f32((uint32_t)(q[b][j] >> (16 * e)) & 0xFFFFu);
        ss[b] = __builtin_fmaf(t, t, ss[b]);
      }
    }
  }
  block_rms_scales<B, NT / kWave>(ss, red, h, p.eps);
  // chunk-major, so a chunk's gammas are decoded once for all B vectors
#pragma unroll
  for (int j = 0; j < Q; ++j) {
    const int i = threadIdx.x + j * NT;
    if (i < nq) {
      float gf[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) gf[e] = bf16_to_f32((uint32_t)(gq[j] >> (16 * e)) & 0xFFFFu) + p.gamma_offset;
#pragma unroll
      for (int b = 0; b < B; ++b) {
        float t[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (bf16_to_f32((uint32_t)(q[b][j] >> (16 * e)) & 0xFFFFu) * ss[b]) * gf[e];
        const unsigned long long o = (unsigned long long)f32x2_to_bf16x2(t[0], t[1]) |
                                     ((unsigned long long)f32x2_to_bf16x2(t[2], t[3]) << 32);
        reinterpret_cast<unsigned long long *>(xs + b * CXP)[i] = o;
        if (p.x_out && blockIdx.x == 0) reinterpret_cast<unsigned long long *>(p.x_out + (int64_t)b * h)[i] = o;
      }
    }
  }
}

// The combine's final RMSNorm, in its last block: x = bf16(u / sqrt(mean(u^2)
// + eps) * (g + off)) for the B fc outputs u (p.y, [B, n]) into p.x_out. All B
// vectors of u are read at once, 4 BF16 per 8-byte agent-coherent load, and
// kept in registers; the B sums of squares share one block reduction.
template <int B, int NT>
__device__ __forceinline__ void combine_final_norm(const SweepParams &p, float *sred) {
  {
    constexpr int Q = 2 * combine_chunks_per_thread<B, NT>();  // 4-element quads per thread
    const int n = (int)p.n;
    const int nq = n >> 2;
    unsigned long long q[B][Q], gq[Q];
    const unsigned long long *g = reinterpret_cast<const unsigned long long *>(p.gamma_f);
    // every load issued unconditionally (indices clamped; quads past the row are zeroed after)
#pragma unroll
    for (int j = 0; j < Q; ++j) gq[j] = g[min((int)threadIdx.x + j * NT, nq - 1)];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const unsigned long long *u = reinterpret_cast<const unsigned long long *>(p.y + (int64_t)b * n);
#pragma unroll
      for (int j = 0; j < Q; ++j)
        q[b][j] = __hip_atomic_load(u + min((int)threadIdx.x + j * NT, nq - 1), __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      if ((int)threadIdx.x + j * NT >= nq) {
        gq[j] = 0ull;
#pragma unroll
        for (int b = 0; b < B; ++b) q[b][j] = 0ull;
      }
    }
    float ss[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      ss[b] = 0.0f;
#pragma unroll
      for (int j = 0; j < Q; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float t = bf16_to_f32((uint32_t)(q[b][j] >> (16 * e)) & 0xFFFFu);
          ss[b] = __builtin_fmaf(t, t, ss[b]);
        }
      }
    }
    block_rms_scales<B, NT / kWave>(ss, sred, n, p.eps);
#pragma unroll
    for (int j = 0; j < Q; ++j) {
      const int i = threadIdx.x + j * NT;
      if (i < nq) {
        float gf[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) gf[e] = bf16_to_f32((uint32_t)(gq[j] >> (16 * e)) & 0xFFFFu) + p.gamma_offset;
#pragma unroll
        for (int b = 0; b < B; ++b) {
          float t[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = (bf16_to_f32((uint32_t)(q[b][j] >> (16 * e)) & 0xFFFFu) * ss[b]) * gf[e];
          reinterpret_cast<unsigned long long *>(p.x_out + (int64_t)b * n)[i] =
              (unsigned long long)f32x2_to_bf16x2(t[0], t[1]) | ((unsigned long long)f32x2_to_bf16x2(t[2], t[3]) << 32);
        }
      }
    }
  }
}

// The argmax epilogue shared by the lm_head kernels, in two parts around the
// ticket. argmax_publish: per vector b, the best packed key over the wave
// (lane_key(b): this lane's best key for vector b, 0 if none; the lanes of a
// 16-lane row hold the same keys (the VALU sweep), or vector b's keys sit in
// lanes b, b + 16, b + 32, b + 48 (COLS: the matrix-core sweep), so two
// cross-row swaps give every key of the wave), raised to 1 when
// the mask allowed rows but none above -inf (lane_seen(b)); with the
// log-probability, the softmax sums rescaled to the wave's maximum M
// (lane_sum(b, M): this lane's share) and summed. Then the block's key per
// vector goes into the running maximum with one agent-scope 64-bit atomic max
// (the packed key orders by value, then lower row); with the log-probability
// the block's key and sum are instead stored per block (agent-scope atomic
// stores, [vector][block], so the last block's reads coalesce), since the sums
// need every block's own maximum.
template <int B, int NT, bool COLS, typename KeyF, typename SeenF, typename SumF>
__device__ __forceinline__ void argmax_publish(const SweepParams &p, bool masked, bool want_lp, KeyF &&lane_key,
                                               SeenF &&lane_seen, SumF &&lane_sum) {
  constexpr int kWaves = NT / kWave;
  __shared__ unsigned long long skeys[kWaves][B];
  __shared__ float sps[kWaves][B];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    unsigned long long kb = readlane_u64(rows_max_u64(lane_key(b)), COLS ? b : 0);
    if (masked && __any(lane_seen(b) ? 1 : 0)) kb = kb > 1ull ? kb : 1ull;
    if (want_lp) {
      const float sl = wave_sum(lane_sum(b, argmax_key_value(kb)));
      if (lane == 0) sps[wave][b] = sl;
    }
    if (lane == 0) skeys[wave][b] = kb;
  }
  __syncthreads();
  if (threadIdx.x < B) {
    unsigned long long kmax = 0ull;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) kmax = max(kmax, skeys[i][threadIdx.x]);
    if (!want_lp) {
      __hip_atomic_fetch_max(p.kmax + threadIdx.x, kmax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      __hip_atomic_store(p.partials + (int64_t)threadIdx.x * kSweepMaxGrid + blockIdx.x, kmax, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
      const float M = argmax_key_value(kmax);
      float S = 0.0f;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const float si = sps[i][threadIdx.x];
        if (si != 0.0f) S += si * __expf(argmax_key_value(skeys[i][threadIdx.x]) - M);
      }
      __hip_atomic_store(p.psums + (int64_t)threadIdx.x * kSweepMaxGrid + blockIdx.x, S, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// argmax_final, in the last block only: the tokens (and the mask's allowed
// flags) from the running maximum per vector, read and reset to zero for the
// next call in one atomic exchange; with the log-probability, the max over the
// per-block keys, S = the blocks' sums rescaled to that maximum, the top-1
// log-probability -log S and the running confidence.
template <int B, int NT>
__device__ __forceinline__ void argmax_final(const SweepParams &p, bool masked, bool want_lp) {
  if (!want_lp) {
    if (threadIdx.x < B) {
      const unsigned long long k =
          __hip_atomic_exchange(p.kmax + threadIdx.x, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      p.token_out[threadIdx.x] = argmax_key_index(k);
      if (masked) p.allowed_out[threadIdx.x] = k >= 1ull ? 1 : 0;
    }
    return;
  }
  constexpr int kWaves = NT / kWave;
  __shared__ unsigned long long skeys[kWaves][B];
  __shared__ float sps[kWaves][B];
  __shared__ unsigned long long sfinal[B];
  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  for (int b = 0; b < B; ++b) {
    unsigned long long k = 0ull;
    for (int i = threadIdx.x; i < (int)gridDim.x; i += NT)
      k = max(k, __hip_atomic_load(p.partials + (int64_t)b * kSweepMaxGrid + i, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT));
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
    for (int i = 0; i < kWaves; ++i) k = max(k, skeys[i][threadIdx.x]);
    p.token_out[threadIdx.x] = argmax_key_index(k);
    if (masked) p.allowed_out[threadIdx.x] = k >= 1ull ? 1 : 0;
    sfinal[threadIdx.x] = k;
  }
  if (want_lp) {
    __syncthreads();
    for (int b = 0; b < B; ++b) {
      const float M = argmax_key_value(sfinal[b]);
      float S = 0.0f;
      for (int i = threadIdx.x; i < (int)gridDim.x; i += NT) {
        const float si =
            __hip_atomic_load(p.psums + (int64_t)b * kSweepMaxGrid + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (si != 0.0f) {
          const unsigned long long ki = __hip_atomic_load(p.partials + (int64_t)b * kSweepMaxGrid + i,
                                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          S += si * __expf(argmax_key_value(ki) - M);
        }
      }
      S = wave_sum(S);
      if (lane == 0) sps[wave][b] = S;
    }
    __syncthreads();
    if (threadIdx.x < B) {
      float S = 0.0f;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) S += sps[i][threadIdx.x];
      const float lp = sfinal[threadIdx.x] > 1ull ? -logf(S) : __builtin_nanf("");
      if (p.logprob_out) p.logprob_out[threadIdx.x] = lp;
      if (p.conf_inout) p.conf_inout[threadIdx.x] = fminf(p.conf_inout[threadIdx.x], expf(lp));
    }
  }
}

// MASK: the grammar-masked argmax (p.masked), a compile-time copy of the body
// so that its per-unit mask loads do not change the unmasked loop's waits.
template <int WD, int B, int MODE, int kR, int kJ, bool RAGGED, int NT, bool MASK = false>
__device__ __forceinline__ void sweep_body(const SweepParams &p) {
  constexpr int kWaves = NT / kWave;
  constexpr int EPC = WT<WD>::kEPC;
  constexpr int XPC = EPC / 8;  // x chunks (8 BF16) per weight chunk
  constexpr int V = kR * B;     // (row, vector) sums per row group
  constexpr int NS = (V + 3) / 4;
  extern __shared__ u32x4 xs[];  // [B][k/8 + XPC]
  __shared__ float sred[kWaves * kMaxRed];
  __shared__ int s_last;

  const int k = p.k;
  const int CX = k >> 3;          // x chunks per vector
  const int CXP = CX + XPC;       // per-vector stride in LDS: x, then XPC zero chunks
  const int C = k / EPC;          // weight chunks per row
  const int64_t row_bytes = (int64_t)C * 16;

  const uint32_t lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int slot = row_slot((int)lane);
  const int64_t n = p.n;
  const int64_t ngroups = (n + kR - 1) / kR;
  const int npass = (C + kWave * kJ - 1) / (kWave * kJ);
  const int64_t gstride = (int64_t)gridDim.x * kWaves;

  // running argmax per reduce-scatter slot: this lane sees the sums of values
  // 4j + slot, i.e. of fixed (row-in-group, vector) pairs
  // and, with the log-probability on, the sum of exp(value - best) over the
  // values it took (online softmax); with a mask, whether it saw an allowed row
  float best[NS], ssum[NS];
  int32_t bidx[NS];
  bool seen[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    best[j] = -__builtin_inff();
    bidx[j] = -1;
    ssum[j] = 0.0f;
    seen[j] = false;
  }
  const bool want_lp = (MODE == kArgmax) && (p.logprob_out != nullptr || p.conf_inout != nullptr);
  constexpr bool masked = (MODE == kArgmax) && MASK;
  float gs = 1.0f;
  if constexpr (WD == kNVFP4) gs = p.gscale[0];

  // Issue the loads of unit (group g, pass ps). The row base is wave-uniform,
  // so each load is a scalar base plus the lane's fixed offset. Rows past n
  // load row n-1; for a ragged row length, chunks past C load chunk C-1: no
  // branches, so the next unit's loads stay in flight while the current one is
  // computed. Those rows are never reported and those chunks meet zero x.
  auto load_unit = [&](Unit<kR, kJ, NS> &U, int64_t g, int ps) {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      int64_t row = g * kR + r;
      row = row < n ? row : n - 1;
      const u32x4 *wr = reinterpret_cast<const u32x4 *>(p.w + row * row_bytes);
      if constexpr (WD == kNVFP4) {
        // dwords 64 s + lane of the pass's scale bytes (2 per chunk, 32 kJ
        // dwords): scales of chunks 2 (64 s + lane) and + 1 of the pass; clamped
        // to the row for ragged passes
        static_assert(kJ % 2 == 0 || RAGGED, "an odd kJ reads scale dwords past the pass: ragged rows only");
        const uint32_t *sr = reinterpret_cast<const uint32_t *>(static_cast<const uint8_t *>(p.scale) +
                                                                row * (int64_t)(k / 16));
#pragma unroll
        for (int s = 0; s < (kJ + 1) / 2; ++s) {
          uint32_t d = (uint32_t)ps * (32u * kJ) + (uint32_t)(s * kWave) + lane;
          if constexpr (RAGGED) d = d < (uint32_t)(k / 64) ? d : (uint32_t)(k / 64) - 1u;
          U.sd[r][s] = __builtin_nontemporal_load(sr + d);
        }
      } else {
#pragma unroll
        for (int s = 0; s < (kJ + 1) / 2; ++s) U.sd[r][s] = 0u;
      }
      if constexpr (WD == kFP8) U.rs[r] = static_cast<const float *>(p.scale)[row];
      else U.rs[r] = gs;
      const uint32_t c0 = (uint32_t)ps * (kWave * kJ);
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        uint32_t c = c0 + (uint32_t)(j * kWave) + lane;
        if constexpr (RAGGED) c = c < (uint32_t)C ? c : (uint32_t)C - 1u;
        if constexpr (MODE == kStoreSplit) {
          // chunks [0, C/2) from e_proj's row, [C/2, C) from h_proj's row
          const uint32_t ch = (uint32_t)C / 2u;
          const u32x4 *we = reinterpret_cast<const u32x4 *>(p.w + row * (int64_t)(ch * 16u));
          const u32x4 *wh = reinterpret_cast<const u32x4 *>(p.w2 + row * (int64_t)(ch * 16u));
          U.w[j][r] = __builtin_nontemporal_load(c < ch ? we + c : wh + (c - ch));
        } else {
          U.w[j][r] = __builtin_nontemporal_load(wr + c);
        }
      }
    }
    // the mask words this lane's slots need at the end of the group, loaded
    // with every unit of it (the same words each pass: L2 hits) so that every
    // unit leaves the same loads in flight: word indices clamped into the
    // mask, or a weight word when the mask is empty (finish_group rejects
    // rows past the mask)
    if constexpr (masked) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int t = 4 * j + slot;
        const int r = t / B, bv = t - (t / B) * B;
        int64_t wi = (g * kR + r) >> 5;
        wi = wi < p.mask_words ? wi : p.mask_words - 1;
        const int32_t *mp = p.mask_words > 0 ? p.mask + (int64_t)bv * p.mask_words + wi
                                             : reinterpret_cast<const int32_t *>(p.w);
        const uint32_t v = (uint32_t)*mp;
        U.mw[j] = (t < V) ? v : 0u;
      }
    }
  };

  float acc[kR][B], acc2[kR][B];  // acc2: the split form's h_proj branch
#pragma unroll
  for (int r = 0; r < kR; ++r)
#pragma unroll
    for (int b = 0; b < B; ++b) {
      acc[r][b] = 0.0f;
      acc2[r][b] = 0.0f;
    }

  auto compute_unit = [&](const Unit<kR, kJ, NS> &U, int ps) {
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      // a ragged row's last pass: load slots wholly past the row hold clamped
      // chunks against zero x, so their products are skipped (wave-uniform)
      if constexpr (RAGGED)
        if (ps * (kWave * kJ) + j * kWave >= C) continue;
      const int c = ps * (kWave * kJ) + j * kWave + (int)lane;
      int xi = c * XPC;
      if constexpr (RAGGED) xi = c < C ? xi : CX;  // past the row: the zero chunks
      uint32_t sv[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if constexpr (WD == kNVFP4) {
          // this lane's chunk j * 64 + lane of the pass: its two scale bytes are
          // half (lane & 1) of dword dw = 32 j + lane / 2 of the pass, held in
          // scale register dw / 64 = j / 2 by lane dw % 64
          const int src = (32 * (j & 1) + (int)(lane >> 1)) * 4;
          const uint32_t v = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)U.sd[r][j >> 1]);
          sv[r] = (lane & 1u) ? (v >> 16) : (v & 0xFFFFu);
        } else {
          sv[r] = 0u;
        }
      }
      if constexpr (MODE == kStoreSplit) {
        float t[kR][B];
#pragma unroll
        for (int r = 0; r < kR; ++r)
#pragma unroll
          for (int b = 0; b < B; ++b) t[r][b] = 0.0f;
        chunk_dot<WD, B, kR>(U.w[j], sv, xs + xi, CXP, t);
        const bool e_part = c < C / 2;
#pragma unroll
        for (int r = 0; r < kR; ++r)
#pragma unroll
          for (int b = 0; b < B; ++b) {
            acc[r][b] += e_part ? t[r][b] : 0.0f;
            acc2[r][b] += e_part ? 0.0f : t[r][b];
          }
      } else {
        chunk_dot<WD, B, kR>(U.w[j], sv, xs + xi, CXP, acc);
      }
    }
  };

  // Row epilogue of group g (its last unit in U): scale, reduce all kR*B sums
  // in one reduce-scatter, then argmax or store from the lane rows that hold them.
  auto finish_group = [&](const Unit<kR, kJ, NS> &U, int64_t g) {
    if constexpr (MODE == kStoreSplit) {
      // both branches in one reduce-scatter: value t = r B + b of the e branch
      // at t, of the h branch at V4 + t (V4 = V rounded up to 4, so both land
      // in the same lane row); u = bf16(bf16(e) + bf16(h))
      constexpr int V4 = NS * 4;
      float v2[2 * V4];
#pragma unroll
      for (int i = 0; i < 2 * V4; ++i) v2[i] = 0.0f;
#pragma unroll
      for (int r = 0; r < kR; ++r)
#pragma unroll
        for (int b = 0; b < B; ++b) {
          v2[r * B + b] = acc[r][b];
          v2[V4 + r * B + b] = acc2[r][b];
          acc[r][b] = 0.0f;
          acc2[r][b] = 0.0f;
        }
      float o2[2 * NS];
      wave_reduce_scatter<2 * V4>(v2, o2);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const int t = 4 * j + slot;
        const int r = t / B, b = t - (t / B) * B;
        const int64_t row = g * kR + r;
        if (t < V && row < n && (lane & 15u) == 0u) {
          const float ue = bf16_to_f32(f32_to_bf16(o2[j]));
          const float uh = bf16_to_f32(f32_to_bf16(o2[NS + j]));
          __hip_atomic_store(p.y + (int64_t)b * n + row, (uint16_t)f32_to_bf16(ue + uh), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      return;
    }
    float v[V];
#pragma unroll
    for (int r = 0; r < kR; ++r)
#pragma unroll
      for (int b = 0; b < B; ++b) {
        v[r * B + b] = (WD == kBF16) ? acc[r][b] : acc[r][b] * U.rs[r];
        acc[r][b] = 0.0f;
      }
    float out[NS];
    wave_reduce_scatter<V>(v, out);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int t = 4 * j + slot;
      const int r = t / B, b = t - (t / B) * B;
      const int64_t row = g * kR + r;
      if (t < V && row < n) {
        const float val = out[j];
        if constexpr (MODE == kArgmax) {
          if (p.logits && (lane & 15u) == 0u) p.logits[(int64_t)b * n + row] = val;
          bool ok = true;
          if (masked) {
            ok = (row >> 5) < (int64_t)p.mask_words && ((U.mw[j] >> (uint32_t)(row & 31)) & 1u);
            seen[j] = seen[j] || ok;
          }
          if (ok) {
            const float b0 = best[j];
            // groups arrive in any order: the larger value wins, then the lower row
            if (val > b0 || (val == b0 && (int32_t)row < bidx[j])) {
              best[j] = val;
              bidx[j] = (int32_t)row;
            }
            if (want_lp) {
              if (val > b0) ssum[j] = ssum[j] * __expf(b0 - val) + 1.0f;  // b0 = -inf: 0 * 0 + 1
              else if (val > -__builtin_inff()) ssum[j] += __expf(val - b0);
              else if (val != val) ssum[j] = val;  // NaN propagates
            }
          }
        } else {
          if ((lane & 15u) == 0u)
            __hip_atomic_store(p.y + (int64_t)b * n + row, (uint16_t)f32_to_bf16(val), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
  };

  // Which group comes next. The combine and the 4-wave lm_head blocks walk
  // their groups statically (grid stride: wave w of block b starts with group
  // b * W + w, W waves per block, and steps by the whole grid's waves). In the
  // 8-wave lm_head blocks the waves take the block's groups from a counter in
  // LDS, one group ahead, wave w starting with index w: the two waves of a
  // SIMD do not get their loads issued at the same rate, and a static split
  // leaves the slower one streaming alone at the end. Index i is group
  // i * gridDim.x + b, dealt round-robin over the grid, so every block gets
  // the same number of groups within one (dealt in rounds of W consecutive
  // groups per block, a partial last round left some blocks W groups more:
  // FP8 154,880 x 4,096, b = 4, 100-102 us then, 97-98 now). Indices map to
  // increasing groups, so the first one past the end ends every later one;
  // the argmax update does not depend on the order.
  constexpr bool kDyn = (MODE == kArgmax && NT == 512);
  __shared__ unsigned s_next;
  unsigned pend = 0u;  // lane 0: the claimed index of the group after the current one
  auto claim = [&]() -> unsigned {
    unsigned r = 0u;
    if (lane == 0u) r = __hip_atomic_fetch_add(&s_next, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return r;
  };
  auto next_group = [&](int64_t g) -> int64_t {
    if constexpr (!kDyn) {
      return g + gstride;
    } else {
      const unsigned i = __builtin_amdgcn_readfirstlane(pend);
      const int64_t gi = (int64_t)i * gridDim.x + blockIdx.x;
      if (gi >= ngroups) return ngroups;
      pend = claim();
      return gi;
    }
  };

  // Two register buffers: while one unit is computed the next one's loads are
  // in flight. Units run pass by pass through each of this wave's groups. The
  // first unit's loads are issued while the vectors are staged, behind the
  // loads of x (loads return in issue order, so x is not queued behind the
  // weights), of u for the draft step's final norm, or of the combine's first
  // batch of concat chunks. They are one unconditional call, the group clamped
  // into the head (a wave with no group loads one it never computes): on every
  // path the same loads are in flight behind the staging's, so the staging
  // waits for its own loads only, not for this unit as well.
  Unit<kR, kJ, NS> ua, ub;
  int64_t g = kDyn ? (int64_t)wave * gridDim.x + blockIdx.x : (int64_t)blockIdx.x * kWaves + wave;
  int ps = 0;
  if constexpr (kDyn)
    if (threadIdx.x == 0) s_next = kWaves;  // read after the staging barrier
  auto first_loads = [&]() { load_unit(ua, g < ngroups ? g : ngroups - 1, 0); };

  for (int b = 0; b < B; ++b)
    for (int i = threadIdx.x; i < XPC; i += NT) xs[b * CXP + CX + i] = u32x4{0u, 0u, 0u, 0u};
  if constexpr (MODE == kArgmax) {
    if (p.u_in) {
      // the draft step: x = rms(u) per block (u complete: the combine ran
      // before this launch on the same stream); the first unit's loads go
      // out behind the u loads
      stage_final_norm<B, NT>(p, k, xs, CXP, sred, first_loads);
    } else {
      // every chunk of the b vectors loaded to registers at once (CX <= 1024:
      // h <= 8192; unconditional loads, clamped, the unused ones never
      // stored), then the first unit's weight loads, then the LDS writes
      const u32x4 *xg = reinterpret_cast<const u32x4 *>(p.x);
      constexpr int QX = (1024 + NT - 1) / NT;
      u32x4 t[B][QX];
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int q = 0; q < QX; ++q) t[b][q] = xg[b * CX + min(q * NT + (int)threadIdx.x, CX - 1)];
      __builtin_amdgcn_sched_barrier(0);
      first_loads();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < B; ++b)
#pragma unroll
        for (int q = 0; q < QX; ++q) {
          const int i = q * NT + (int)threadIdx.x;
          if (i < CX) xs[b * CXP + i] = t[b][q];
        }
    }
  } else {
    stage_concat<B, NT>(p, k >> 1, xs, CXP, sred, first_loads);  // k = 2h
  }
  __syncthreads();
  if constexpr (kDyn) pend = claim();

  // Each half issues the next unit's loads only when there is one; the branch
  // is wave-uniform and both sides leave the same loads outstanding at the
  // join, so the waits before each compute cover only the unit computed.
  while (g < ngroups) {
    int64_t g1 = g;
    int ps1 = ps + 1;
    if (ps1 == npass) {
      ps1 = 0;
      g1 = next_group(g);
    }
    if (g1 < ngroups) {
      load_unit(ub, g1, ps1);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the compute
      compute_unit(ua, ps);
      if (ps == npass - 1) finish_group(ua, g);
    } else {
      compute_unit(ua, ps);
      if (ps == npass - 1) finish_group(ua, g);
      break;
    }
    g = g1;
    ps = ps1;
    int64_t g2 = g;
    int ps2 = ps + 1;
    if (ps2 == npass) {
      ps2 = 0;
      g2 = next_group(g);
    }
    if (g2 < ngroups) {
      load_unit(ua, g2, ps2);
      __builtin_amdgcn_sched_barrier(0);
      compute_unit(ub, ps);
      if (ps == npass - 1) finish_group(ub, g);
    } else {
      compute_unit(ub, ps);
      if (ps == npass - 1) finish_group(ub, g);
      break;
    }
    g = g2;
    ps = ps2;
  }

  if constexpr (MODE == kArgmax) {
    // this lane's slots of vector b (the 16-lane rows hold identical copies:
    // one lane per row counts the softmax sums)
    auto slot_of = [&](int j, int b) {
      const int t = 4 * j + slot;
      return t < V && (t - (t / B) * B) == b;
    };
    argmax_publish<B, NT, false>(
        p, masked, want_lp,
        [&](int b) {
          unsigned long long kb = 0ull;
#pragma unroll
          for (int j = 0; j < NS; ++j)
            if (slot_of(j, b) && bidx[j] >= 0) {
              const unsigned long long kk = argmax_key(best[j], (uint32_t)bidx[j]);
              kb = kk > kb ? kk : kb;
            }
          return kb;
        },
        [&](int b) {
          bool sb = false;
#pragma unroll
          for (int j = 0; j < NS; ++j) sb = sb || (slot_of(j, b) && seen[j]);
          return sb;
        },
        [&](int b, float M) {
          float sl = 0.0f;
          if ((lane & 15u) == 0u) {
#pragma unroll
            for (int j = 0; j < NS; ++j)
              if (slot_of(j, b) && ssum[j] != 0.0f) sl += ssum[j] * __expf(best[j] - M);
          }
          return sl;
        });
  }
  // this thread's agent-coherent stores have completed before the ticket is taken
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (MODE != kArgmax) {
    if (p.no_final) return;  // the draft step: u is stored, the lm_head applies the final norm
  }
  if (threadIdx.x == 0)
    s_last = (__hip_atomic_fetch_add(p.ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              gridDim.x - 1u);
  __syncthreads();
  if (!s_last) return;

  if constexpr (MODE == kArgmax) {
    argmax_final<B, NT>(p, masked, want_lp);
  } else {
    combine_final_norm<B, NT>(p, sred);
  }
  if (threadIdx.x == 0) __hip_atomic_store(p.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The two kernels, named apart so profiles and counters tell them apart. Up
// to two waves per SIMD (an 8-wave lm_head block, or the combine's four 4-wave
// blocks per CU): caps each at 256 VGPRs.
template <int WD, int B, int kR, int kJ, bool RAGGED, int NT>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2)))
lmhead_argmax_kernel(SweepParams p) {
  if (p.masked)
    sweep_body<WD, B, kArgmax, kR, kJ, RAGGED, NT, true>(p);
  else
    sweep_body<WD, B, kArgmax, kR, kJ, RAGGED, NT, false>(p);
}

template <int WD, int B, int MODE, int kR, int kJ, bool RAGGED>
__global__ void __launch_bounds__(kCombineThreads) __attribute__((amdgpu_waves_per_eu(2)))
draft_combine_kernel(SweepParams p) {
  sweep_body<WD, B, MODE, kR, kJ, RAGGED, kCombineThreads>(p);
}

// lm_head block shape (threads per block, one block per CU) per
// configuration, with lm_rows, from measurements at 154,880 x 4,096 and
// 131,072 x 5,120: a static 4-wave block (one wave per SIMD) for BF16 at
// b <= 2 and for FP8 and NVFP4 at b = 2 on whole-pass rows; otherwise 8 waves
// sharing the block's groups at run time (FP8 and NVFP4 at b = 1 hide their
// decode behind the second wave of each SIMD; b >= 3 and ragged rows).
template <int WD, int B, bool RAGGED>
constexpr int lm_threads() {
  if (RAGGED) return 512;
  if (WD == kBF16) return B <= 2 ? 256 : 512;
  return B == 2 ? 256 : 512;
}

template <int WD, int B, int MODE, int R, int J, bool RAGGED, int NT>
static const void *sweep_kernel_fn() {
  if constexpr (MODE == kArgmax)
    return reinterpret_cast<const void *>(&lmhead_argmax_kernel<WD, B, R, J, RAGGED, NT>);
  else
    return reinterpret_cast<const void *>(&draft_combine_kernel<WD, B, MODE, R, J, RAGGED>);
}

// ------------------------------------------------------------------ host ----

// Grid: one block per W groups up to blocks-per-CU x CUs (at most kSweepMaxGrid).
template <int WD, int B, int MODE, int R, int J, bool RAGGED, int NT>
static hipError_t launch_sweep_rt(const SweepParams &p, int blocks_per_cu_target, hipStream_t s) {
  const void *fn = sweep_kernel_fn<WD, B, MODE, R, J, RAGGED, NT>();
  const int lds = B * (p.k * 2 + 16 * (WT<WD>::kEPC / 8));  // x + zero chunks per vector
  const int bpc = blocks_per_cu(fn, NT, lds);
  if (bpc <= 0) return hipErrorInvalidConfiguration;
  const int64_t groups = (p.n + R - 1) / R;
  const int64_t want = (groups + NT / kWave - 1) / (NT / kWave);
  const int64_t per_cu = bpc < blocks_per_cu_target ? bpc : blocks_per_cu_target;
  int64_t cap = (int64_t)device_cu_count() * per_cu;
  if (cap > kSweepMaxGrid) cap = kSweepMaxGrid;
  const int grid = (int)(want < cap ? want : cap);
  if constexpr (MODE == kArgmax)
    hipLaunchKernelGGL((lmhead_argmax_kernel<WD, B, R, J, RAGGED, NT>), dim3(grid > 0 ? grid : 1),
                       dim3(NT), lds, s, p);
  else
    hipLaunchKernelGGL((draft_combine_kernel<WD, B, MODE, R, J, RAGGED>), dim3(grid > 0 ? grid : 1),
                       dim3(NT), lds, s, p);
  return hipGetLastError();
}

// Row lengths that are a whole number of passes need no per-chunk clamps.
template <int WD, int B, int J>
static hipError_t launch_lmhead_t(const SweepParams &p, hipStream_t s) {
  const int C = p.k / WT<WD>::kEPC;
  if (C % (kWave * J) == 0) {
    constexpr int NT = lm_threads<WD, B, false>();
    return launch_sweep_rt<WD, B, kArgmax, lm_rows<WD, B, false>(), J, false, NT>(p, 1, s);
  }
  constexpr int NT = lm_threads<WD, B, true>();
  if constexpr (WD == kNVFP4 && B == 1) {
    // rows of 129..192 chunks (h = 5,120: 160) in one pass of 3 chunks per lane
    // instead of a full pass and a quarter pass
    if (C > 2 * kWave && C <= 3 * kWave)
      return launch_sweep_rt<WD, B, kArgmax, lm_rows<WD, B, true>(), 3, true, NT>(p, 1, s);
  }
  return launch_sweep_rt<WD, B, kArgmax, lm_rows<WD, B, true>(), J, true, NT>(p, 1, s);
}

template <int WD>
static hipError_t launch_lmhead_wd(int b, const SweepParams &p, hipStream_t s) {
  constexpr int J = WT<WD>::kJ;
  switch (b) {
    case 1: return launch_lmhead_t<WD, 1, J>(p, s);
    case 2: return launch_lmhead_t<WD, 2, J>(p, s);
    case 3: return launch_lmhead_t<WD, 3, J>(p, s);
    case 4: return launch_lmhead_t<WD, 4, J>(p, s);
    case 5: return launch_lmhead_t<WD, 5, J>(p, s);
    case 6: return launch_lmhead_t<WD, 6, J>(p, s);
    case 7: return launch_lmhead_t<WD, 7, J>(p, s);
    case 8: return launch_lmhead_t<WD, 8, J>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <int WD, int MODE, int B>
static hipError_t launch_fc_b(const SweepParams &p, hipStream_t s) {
  // the concat and the final norm hold at most combine_max_h<B>() per vector
  if (p.k / 2 > combine_max_h<B>()) return hipErrorInvalidValue;
  constexpr int J = MODE == kStoreSplit ? 16 : fc_chunks<WD>();
  const int C = p.k / WT<WD>::kEPC;
  if (C % (kWave * J) == 0)
    return launch_sweep_rt<WD, B, MODE, kFcR, J, false, kCombineThreads>(p, kFcBlocksPerCU, s);
  return launch_sweep_rt<WD, B, MODE, kFcR, J, true, kCombineThreads>(p, kFcBlocksPerCU, s);
}

template <int WD, int MODE>
static hipError_t launch_fc_wd(int b, const SweepParams &p, hipStream_t s) {
  switch (b) {
    case 1: return launch_fc_b<WD, MODE, 1>(p, s);
    case 2: return launch_fc_b<WD, MODE, 2>(p, s);
    case 3: return launch_fc_b<WD, MODE, 3>(p, s);
    case 4: return launch_fc_b<WD, MODE, 4>(p, s);
    case 5: return launch_fc_b<WD, MODE, 5>(p, s);
    case 6: return launch_fc_b<WD, MODE, 6>(p, s);
    case 7: return launch_fc_b<WD, MODE, 7>(p, s);
    case 8: return launch_fc_b<WD, MODE, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

// Per-format instantiations, each in a translation unit of its own so the
// build compiles them in parallel (lm_*.hip, combine_*.hip).
hipError_t launch_lmhead_bf16(int b, const SweepParams &p, hipStream_t s);
hipError_t launch_lmhead_fp8(int b, const SweepParams &p, hipStream_t s);
hipError_t launch_lmhead_nvfp4(int b, const SweepParams &p, hipStream_t s);
hipError_t launch_fc_bf16(int b, bool split, const SweepParams &p, hipStream_t s);
hipError_t launch_fc_fp8(int b, const SweepParams &p, hipStream_t s);
hipError_t launch_fc_nvfp4(int b, const SweepParams &p, hipStream_t s);
hipError_t launch_combine_mfma(int b, const SweepParams &p, hipStream_t s);

}  // namespace mtp
