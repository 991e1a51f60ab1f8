// Internal launchers of the MTP draft-step kernels. Host code; called only by
// the C ABI layer (abi.cpp) after it has validated every argument.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

enum WDtype : int { kBF16 = 0, kFP8 = 1, kNVFP4 = 2 };

// Sizes of the workspaces (bytes).
// lm_head workspace: ticket u32 at 0; running max key per vector u64 [8] at
// 128 (its own 128-byte line); per-block keys u64 [8][kSweepMaxGrid] at 256;
// per-block softmax sums f32 [8][kSweepMaxGrid] after them. Ticket and running
// keys are zero on entry and on exit.
constexpr int kSweepMaxGrid = 4096;
constexpr size_t kLmheadKmaxOffset = 128;
constexpr size_t kLmheadPsumsOffset = 256 + (size_t)kSweepMaxGrid * 8 * 8;
constexpr size_t kLmheadWsBytes = kLmheadPsumsOffset + (size_t)kSweepMaxGrid * 8 * 4;
size_t combine_ws_bytes(int64_t b, int64_t h);
constexpr size_t kNvfp4WsBytes = 256;   // u32 global |w| max at 0

struct LmheadLaunch {
  const uint16_t *x;     // [b, h] BF16
  const void *w;         // weight rows
  const void *scale;     // FP8: f32 [n]; NVFP4: u8 [n, h/16]
  const float *gscale;   // NVFP4: f32 [1]
  int64_t n;             // rows swept (n_eff)
  int h;
  int b;
  int wd;
  int32_t *token_out;    // [b]
  float *logits;         // NULL or f32 [b, n]
  void *ws;              // kLmheadWsBytes, zero on entry, zero on exit
  // options (NULL when unused)
  float *logprob;        // [b] top-1 log-probability
  float *conf;           // [b] running minimum of the top-1 probability
  int masked;            // 1: the grammar-masked argmax
  const int32_t *mask;   // [b, mask_words] grammar bitmask (NULL when mask_words == 0)
  int mask_words;
  int32_t *allowed;      // [b] 1 if the mask allowed a row
};
hipError_t launch_lmhead(const LmheadLaunch &a, hipStream_t s);

struct CombineLaunch {
  const uint16_t *embed;         // [vocab, h]
  int64_t vocab;
  int32_t tokens[8];             // validated host token ids (when tokens_dev is NULL)
  const int32_t *tokens_dev;     // NULL, or device token ids [b], clamped into [0, vocab)
  const uint16_t *hidden;        // [b, h]
  const uint16_t *gamma_e, *gamma_h, *gamma_f;  // [h]
  int fc_wd;                     // weight format of fc (WDtype)
  const void *fc;                // [h, 2h] in fc_wd; the split form: e_proj [h, h] BF16
  const void *fc_scale;          // FP8: f32 [h]; NVFP4: u8 [h, 2h/16]; else NULL
  const float *fc_gscale;        // NVFP4: f32 [1]
  const uint16_t *h_proj;        // NULL, or the split form's h_proj [h, h] BF16
  int b, h;
  float eps, gamma_offset;
  uint16_t *x_out;               // [b, h]
  void *ws;                      // combine_ws_bytes(b, h), ticket zero on entry and exit
};
hipError_t launch_combine(const CombineLaunch &a, hipStream_t s);

// The draft step: the combine (BF16 fc) stopping at u, then the lm_head +
// argmax staging x = rms(u) per block (x_out, logprob, conf optional; no
// logits, no mask). Workspace: the lm_head's (kLmheadWsBytes, zero on entry
// and exit), 256 spare bytes, u [b, h] BF16 at kStepWsUOffset, then the
// concat c [b, 2h] BF16 at the next multiple of 256 (both left there by the
// call).
struct StepLaunch {
  CombineLaunch c;
  LmheadLaunch l;
  void *ws;
};
constexpr size_t kStepWsUOffset = kLmheadWsBytes + 256;
size_t step_ws_bytes(int64_t b, int64_t h);
hipError_t launch_step(const StepLaunch &a, hipStream_t s);

// The draft step on the library's own per-device scratch (no caller
// workspace): largest workspace it serves, and the launch.
constexpr size_t kStepScratchBytes = kStepWsUOffset + 8 * 8192 * 2 + 8 * 2 * 8192 * 2;
hipError_t launch_step_scratch(const StepLaunch &a, hipStream_t s);

hipError_t launch_quant_fp8(const uint16_t *w, int64_t n, int k, uint8_t *codes, float *scale,
                            hipStream_t s);
hipError_t launch_quant_nvfp4(const uint16_t *w, int64_t n, int k, uint8_t *codes,
                              uint8_t *block_scale, float *global_scale, void *ws, hipStream_t s);
hipError_t launch_codec_range(int codec, uint32_t first_bits, int64_t count, uint8_t *out,
                              hipStream_t s);

// Largest dynamic LDS (bytes) the sweep may use for its staged vectors (plus a
// few zero chunks; the part has 160 KB per work-group).
constexpr int kMaxSweepLds = 128 * 1024 + 8 * 64;

// Per-device cached attributes.
// Whether an lm_head call of b vectors of length k takes the matrix-core form
// (lm_fp8.hip, lm_nvfp4.hip).
bool lmhead_mfma_bf16(int b, int k);
bool lmhead_mfma_fp8(int b, int k);
bool lmhead_mfma_nvfp4(int b, int k);
// Whether a combine group of b batch rows with a BF16 fc of row length k takes
// the matrix-core fc (combine_mfma.hip).
bool combine_uses_mfma(int b, int k);

int device_cu_count();
// Blocks of `func` (block size `threads`, dynamic LDS `lds`) resident per CU;
// also raises the kernel's dynamic-LDS limit when needed. 0 on failure.
int blocks_per_cu(const void *func, int threads, int lds);

}  // namespace mtp
