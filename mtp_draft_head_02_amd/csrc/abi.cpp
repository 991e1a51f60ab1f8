// C ABI of the MTP draft-step library: argument validation on the host (no HIP
// call before every check has passed), then dispatch to the kernel launchers.
// Declarations, argument meanings and the passages each call follows are in
// include/mtp_draft.h.
#include "mtp_draft.h"  // include/ is on the include path

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <map>
#include <mutex>
#include <tuple>

#include "mtp_kernels.h"

static_assert(MTP_STEP_WS_U_OFFSET == mtp::kStepWsUOffset, "documented step workspace layout");
static_assert(MTP_COMBINE_WS_C_OFFSET == 256, "documented combine workspace layout");

namespace mtp {

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

std::mutex g_occ_mutex;
std::map<std::tuple<int, const void *, int, int>, int> g_occ;

}  // namespace

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 1;
  int v = g_cu_count[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    return 1;
  g_cu_count[dev].store(v, std::memory_order_relaxed);
  return v;
}

int blocks_per_cu(const void *func, int threads, int lds) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  const auto key = std::make_tuple(dev, func, threads, lds);
  std::lock_guard<std::mutex> lock(g_occ_mutex);
  auto it = g_occ.find(key);
  if (it != g_occ.end()) return it->second;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return 0;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, func, threads, (size_t)lds) != hipSuccess)
    return 0;
  g_occ[key] = nb;
  return nb;
}

}  // namespace mtp

namespace {

struct Range {
  const void *p;
  uint64_t bytes;
};

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Every output against every input and every other output.
bool any_overlap(const Range *outs, int nout, const Range *ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    for (int j = 0; j < nin; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < nout; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

int from_hip(hipError_t e) { return e == hipSuccess ? MTP_OK : MTP_ERR_HIP; }

constexpr int64_t kMaxRows = int64_t(1) << 40;

}  // namespace

namespace mtp {
// stream_probe.hip: the streaming-read reference (measurement only)
hipError_t launch_stream_read(const void *buf, int64_t bytes, int shape, uint32_t magic, uint32_t *sink,
                              hipStream_t s);
}  // namespace mtp

extern "C" {

int mtp_abi_version(void) { return MTP_ABI_VERSION; }

const char *mtp_status_string(int st) {
  switch (st) {
    case MTP_OK: return "ok";
    case MTP_ERR_NULL: return "a required pointer is NULL";
    case MTP_ERR_SHAPE: return "a size is out of range or not a required multiple";
    case MTP_ERR_ALIGN: return "a pointer is not aligned as required";
    case MTP_ERR_DTYPE: return "unknown weight or codec kind, or a scale pointer given/missing";
    case MTP_ERR_WORKSPACE: return "workspace NULL or smaller than required";
    case MTP_ERR_OVERLAP: return "an output range overlaps an input or another output";
    case MTP_ERR_HIP: return "the HIP runtime refused a launch";
    case MTP_ERR_RANGE: return "a token id is outside [0, vocab)";
    default: return "unknown status";
  }
}

int mtp_quantize_fp8(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes, float *row_scale,
                     void *stream) {
  if (!w || !codes || !row_scale) return MTP_ERR_NULL;
  if (n < 1 || n > kMaxRows || k < 16 || k > 65536 || k % 16 != 0) return MTP_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(row_scale, 4)) return MTP_ERR_ALIGN;
  const Range ins[] = {{w, (uint64_t)(n * k * 2)}};
  const Range outs[] = {{codes, (uint64_t)(n * k)}, {row_scale, (uint64_t)(n * 4)}};
  if (any_overlap(outs, 2, ins, 1)) return MTP_ERR_OVERLAP;
  return from_hip(mtp::launch_quant_fp8(w, n, (int)k, codes, row_scale, (hipStream_t)stream));
}

size_t mtp_quantize_nvfp4_workspace_bytes(int64_t n, int64_t k) {
  (void)n;
  (void)k;
  return mtp::kNvfp4WsBytes;
}

int mtp_quantize_nvfp4(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes,
                       uint8_t *block_scale, float *global_scale, void *ws, size_t ws_bytes,
                       void *stream) {
  if (!w || !codes || !block_scale || !global_scale) return MTP_ERR_NULL;
  if (!ws) return MTP_ERR_WORKSPACE;
  if (n < 1 || n > kMaxRows || k < 256 || k > 65536 || k % 256 != 0) return MTP_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(block_scale, 16) ||
      !aligned(global_scale, 4) || !aligned(ws, 16))
    return MTP_ERR_ALIGN;
  if (ws_bytes < mtp_quantize_nvfp4_workspace_bytes(n, k)) return MTP_ERR_WORKSPACE;
  const Range ins[] = {{w, (uint64_t)(n * k * 2)}};
  const Range outs[] = {{codes, (uint64_t)(n * k / 2)},
                        {block_scale, (uint64_t)(n * k / 16)},
                        {global_scale, 4},
                        {ws, (uint64_t)mtp_quantize_nvfp4_workspace_bytes(n, k)}};
  if (any_overlap(outs, 4, ins, 1)) return MTP_ERR_OVERLAP;
  return from_hip(mtp::launch_quant_nvfp4(w, n, (int)k, codes, block_scale, global_scale, ws,
                                          (hipStream_t)stream));
}

size_t mtp_draft_combine_workspace_bytes(int64_t b, int64_t h) {
  if (b < 1 || b > 8 || h < 16 || h > 8192) return 0;
  return mtp::combine_ws_bytes(b, h);
}

}  // extern "C"

namespace {

// Checks shared by the combine entry points (everything but the projection
// weights); fills `a` and the ranges. Host token ids are range-checked here;
// device token ids are only checked for alignment (the kernel clamps them).
int combine_common(const uint16_t *embed_table, int64_t vocab, const int32_t *token_ids,
                   bool tokens_on_device, const uint16_t *target_hidden,
                   const uint16_t *gamma_embed, const uint16_t *gamma_hidden,
                   const uint16_t *gamma_final, int64_t b, int64_t h, float eps, float gamma_offset,
                   uint16_t *x_out, void *ws, size_t ws_bytes, mtp::CombineLaunch &a, Range *ins,
                   Range *outs) {
  if (!embed_table || !token_ids || !target_hidden || !gamma_embed || !gamma_hidden ||
      !gamma_final || !x_out)
    return MTP_ERR_NULL;
  if (!ws) return MTP_ERR_WORKSPACE;
  if (b < 1 || b > 8 || h < 16 || h > 8192 || h % 16 != 0 || vocab < 1 ||
      vocab > int64_t(0x7FFFFFFF))
    return MTP_ERR_SHAPE;
  if (!(eps > 0.0f) || !std::isfinite(eps) || !std::isfinite(gamma_offset)) return MTP_ERR_SHAPE;
  if (!tokens_on_device)
    for (int64_t i = 0; i < b; ++i)
      if (token_ids[i] < 0 || token_ids[i] >= vocab) return MTP_ERR_RANGE;
  if (!aligned(embed_table, 16) || !aligned(target_hidden, 16) || !aligned(gamma_embed, 16) ||
      !aligned(gamma_hidden, 16) || !aligned(gamma_final, 16) || !aligned(x_out, 16) ||
      !aligned(ws, 16) || (tokens_on_device && !aligned(token_ids, 4)))
    return MTP_ERR_ALIGN;
  const size_t need = mtp_draft_combine_workspace_bytes(b, h);
  if (ws_bytes < need) return MTP_ERR_WORKSPACE;
  ins[0] = {embed_table, (uint64_t)(vocab * h * 2)};
  ins[1] = {target_hidden, (uint64_t)(b * h * 2)};
  ins[2] = {gamma_embed, (uint64_t)(h * 2)};
  ins[3] = {gamma_hidden, (uint64_t)(h * 2)};
  ins[4] = {gamma_final, (uint64_t)(h * 2)};
  ins[5] = {tokens_on_device ? token_ids : nullptr, tokens_on_device ? (uint64_t)(b * 4) : 0u};
  outs[0] = {x_out, (uint64_t)(b * h * 2)};
  outs[1] = {ws, (uint64_t)need};
  a = mtp::CombineLaunch{};
  a.embed = embed_table;
  a.vocab = vocab;
  if (tokens_on_device)
    a.tokens_dev = token_ids;
  else
    for (int i = 0; i < 8; ++i) a.tokens[i] = i < b ? token_ids[i] : 0;
  a.hidden = target_hidden;
  a.gamma_e = gamma_embed;
  a.gamma_h = gamma_hidden;
  a.gamma_f = gamma_final;
  a.fc_wd = MTP_W_BF16;
  a.b = (int)b;
  a.h = (int)h;
  a.eps = eps;
  a.gamma_offset = gamma_offset;
  a.x_out = x_out;
  a.ws = ws;
  return MTP_OK;
}

int combine_bf16(const uint16_t *embed_table, int64_t vocab, const int32_t *token_ids,
                 bool tokens_on_device, const uint16_t *target_hidden, const uint16_t *gamma_embed,
                 const uint16_t *gamma_hidden, const uint16_t *fc_w, const uint16_t *gamma_final,
                 int64_t b, int64_t h, float eps, float gamma_offset, uint16_t *x_out, void *ws,
                 size_t ws_bytes, void *stream) {
  mtp::CombineLaunch a;
  Range ins[7], outs[2];
  const int st = combine_common(embed_table, vocab, token_ids, tokens_on_device, target_hidden,
                                gamma_embed, gamma_hidden, gamma_final, b, h, eps, gamma_offset,
                                x_out, ws, ws_bytes, a, ins, outs);
  if (st != MTP_OK) return st;
  if (!fc_w) return MTP_ERR_NULL;
  if (!aligned(fc_w, 16)) return MTP_ERR_ALIGN;
  ins[6] = {fc_w, (uint64_t)(h * 2 * h * 2)};
  if (any_overlap(outs, 2, ins, 7)) return MTP_ERR_OVERLAP;
  a.fc = fc_w;
  return from_hip(mtp::launch_combine(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int mtp_draft_combine(const uint16_t *embed_table, int64_t vocab, const int32_t *token_ids,
                      const uint16_t *target_hidden, const uint16_t *gamma_embed,
                      const uint16_t *gamma_hidden, const uint16_t *fc_w,
                      const uint16_t *gamma_final, int64_t b, int64_t h, float eps,
                      float gamma_offset, uint16_t *x_out, void *ws, size_t ws_bytes,
                      void *stream) {
  return combine_bf16(embed_table, vocab, token_ids, false, target_hidden, gamma_embed,
                      gamma_hidden, fc_w, gamma_final, b, h, eps, gamma_offset, x_out, ws, ws_bytes,
                      stream);
}

int mtp_draft_combine_dev(const uint16_t *embed_table, int64_t vocab, const int32_t *token_ids_dev,
                          const uint16_t *target_hidden, const uint16_t *gamma_embed,
                          const uint16_t *gamma_hidden, const uint16_t *fc_w,
                          const uint16_t *gamma_final, int64_t b, int64_t h, float eps,
                          float gamma_offset, uint16_t *x_out, void *ws, size_t ws_bytes,
                          void *stream) {
  return combine_bf16(embed_table, vocab, token_ids_dev, true, target_hidden, gamma_embed,
                      gamma_hidden, fc_w, gamma_final, b, h, eps, gamma_offset, x_out, ws, ws_bytes,
                      stream);
}

int mtp_draft_combine_q(const uint16_t *embed_table, int64_t vocab, const int32_t *token_ids,
                        const uint16_t *target_hidden, const uint16_t *gamma_embed,
                        const uint16_t *gamma_hidden, int fc_wd, const void *fc,
                        const void *fc_scale, const float *fc_gscale, const uint16_t *gamma_final,
                        int64_t b, int64_t h, float eps, float gamma_offset, uint16_t *x_out,
                        void *ws, size_t ws_bytes, void *stream) {
  if (fc_wd != MTP_W_BF16 && fc_wd != MTP_W_FP8_E4M3_ROW && fc_wd != MTP_W_NVFP4) return MTP_ERR_DTYPE;
  mtp::CombineLaunch a;
  Range ins[9], outs[2];
  const int st = combine_common(embed_table, vocab, token_ids, false, target_hidden, gamma_embed,
                                gamma_hidden, gamma_final, b, h, eps, gamma_offset, x_out, ws,
                                ws_bytes, a, ins, outs);
  if (st != MTP_OK) return st;
  if (!fc) return MTP_ERR_NULL;
  if (fc_wd == MTP_W_BF16 && (fc_scale || fc_gscale)) return MTP_ERR_DTYPE;
  if (fc_wd == MTP_W_FP8_E4M3_ROW && (!fc_scale || fc_gscale)) return fc_scale ? MTP_ERR_DTYPE : MTP_ERR_NULL;
  if (fc_wd == MTP_W_NVFP4 && (!fc_scale || !fc_gscale)) return MTP_ERR_NULL;
  if (fc_wd == MTP_W_NVFP4 && (2 * h) % 256 != 0) return MTP_ERR_SHAPE;
  if (!aligned(fc, 16) || (fc_wd == MTP_W_FP8_E4M3_ROW && !aligned(fc_scale, 4)) ||
      (fc_wd == MTP_W_NVFP4 && (!aligned(fc_scale, 16) || !aligned(fc_gscale, 4))))
    return MTP_ERR_ALIGN;
  const int64_t k = 2 * h;
  const int64_t fc_bytes = fc_wd == MTP_W_BF16 ? h * k * 2 : (fc_wd == MTP_W_FP8_E4M3_ROW ? h * k : h * k / 2);
  const int64_t sc_bytes = fc_wd == MTP_W_FP8_E4M3_ROW ? 4 * h : (fc_wd == MTP_W_NVFP4 ? h * (k / 16) : 0);
  ins[6] = {fc, (uint64_t)fc_bytes};
  ins[7] = {fc_scale, (uint64_t)sc_bytes};
  ins[8] = {fc_gscale, fc_gscale ? 4u : 0u};
  if (any_overlap(outs, 2, ins, 9)) return MTP_ERR_OVERLAP;
  a.fc_wd = fc_wd;
  a.fc = fc;
  a.fc_scale = fc_scale;
  a.fc_gscale = fc_gscale;
  return from_hip(mtp::launch_combine(a, (hipStream_t)stream));
}

int mtp_draft_combine_split(const uint16_t *embed_table, int64_t vocab, const int32_t *token_ids,
                            const uint16_t *target_hidden, const uint16_t *gamma_embed,
                            const uint16_t *gamma_hidden, const uint16_t *e_proj,
                            const uint16_t *h_proj, const uint16_t *gamma_final, int64_t b,
                            int64_t h, float eps, float gamma_offset, uint16_t *x_out, void *ws,
                            size_t ws_bytes, void *stream) {
  mtp::CombineLaunch a;
  Range ins[8], outs[2];
  const int st = combine_common(embed_table, vocab, token_ids, false, target_hidden, gamma_embed,
                                gamma_hidden, gamma_final, b, h, eps, gamma_offset, x_out, ws,
                                ws_bytes, a, ins, outs);
  if (st != MTP_OK) return st;
  if (!e_proj || !h_proj) return MTP_ERR_NULL;
  if (!aligned(e_proj, 16) || !aligned(h_proj, 16)) return MTP_ERR_ALIGN;
  ins[6] = {e_proj, (uint64_t)(h * h * 2)};
  ins[7] = {h_proj, (uint64_t)(h * h * 2)};
  if (any_overlap(outs, 2, ins, 8)) return MTP_ERR_OVERLAP;
  a.fc = e_proj;
  a.h_proj = h_proj;
  return from_hip(mtp::launch_combine(a, (hipStream_t)stream));
}

int mtp_lmhead_kernel_form(int64_t b, int64_t h, int wd) {
  if (b < 1 || b > 8 || h < 16 || h > 8192 || h % 16 != 0) return -1;
  switch (wd) {
    case mtp::kBF16: return mtp::lmhead_mfma_bf16((int)b, (int)h) ? 1 : 0;
    case mtp::kFP8: return mtp::lmhead_mfma_fp8((int)b, (int)h) ? 1 : 0;
    case mtp::kNVFP4: return h % 256 != 0 ? -1 : (mtp::lmhead_mfma_nvfp4((int)b, (int)h) ? 1 : 0);
    default: return -1;
  }
}

size_t mtp_lmhead_argmax_workspace_bytes(int64_t vocab, int64_t h, int64_t b, int wd) {
  (void)vocab;
  (void)h;
  (void)b;
  (void)wd;
  return mtp::kLmheadWsBytes;
}

}  // extern "C"

namespace {

// Checks shared by the lm_head entry points; fills `a` and the input/output
// ranges (the caller appends its own before the overlap check).
int lm_common(const uint16_t *x, int64_t b, int64_t h, int wd, const void *w, const void *scale,
              const float *gscale, int64_t vocab, int64_t mtp_vocab_size, int32_t *token_out,
              float *logits_out, void *ws, size_t ws_bytes, mtp::LmheadLaunch &a, Range *ins,
              Range *outs) {
  if (wd != MTP_W_BF16 && wd != MTP_W_FP8_E4M3_ROW && wd != MTP_W_NVFP4) return MTP_ERR_DTYPE;
  if (!x || !w || !token_out) return MTP_ERR_NULL;
  if (!ws) return MTP_ERR_WORKSPACE;
  if (wd == MTP_W_BF16 && (scale || gscale)) return MTP_ERR_DTYPE;
  if (wd == MTP_W_FP8_E4M3_ROW && (!scale || gscale)) return scale ? MTP_ERR_DTYPE : MTP_ERR_NULL;
  if (wd == MTP_W_NVFP4 && (!scale || !gscale)) return MTP_ERR_NULL;
  if (b < 1 || b > 8 || vocab < 1 || vocab > int64_t(0x7FFFFFFF) || mtp_vocab_size < 0 ||
      h < 16 || h > 8192)
    return MTP_ERR_SHAPE;
  if (h % (wd == MTP_W_NVFP4 ? 256 : 16) != 0) return MTP_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(token_out, 4) || !aligned(ws, 16) ||
      (logits_out && !aligned(logits_out, 4)) ||
      (wd == MTP_W_FP8_E4M3_ROW && !aligned(scale, 4)) ||
      (wd == MTP_W_NVFP4 && (!aligned(scale, 16) || !aligned(gscale, 4))))
    return MTP_ERR_ALIGN;
  if (ws_bytes < mtp::kLmheadWsBytes) return MTP_ERR_WORKSPACE;
  const int64_t n_eff = (mtp_vocab_size > 0 && mtp_vocab_size < vocab) ? mtp_vocab_size : vocab;
  const int64_t row_bytes = wd == MTP_W_BF16 ? 2 * h : (wd == MTP_W_FP8_E4M3_ROW ? h : h / 2);
  const int64_t scale_bytes =
      wd == MTP_W_FP8_E4M3_ROW ? 4 * vocab : (wd == MTP_W_NVFP4 ? vocab * (h / 16) : 0);
  ins[0] = {x, (uint64_t)(b * h * 2)};
  ins[1] = {w, (uint64_t)(vocab * row_bytes)};
  ins[2] = {scale, (uint64_t)scale_bytes};
  ins[3] = {gscale, gscale ? 4u : 0u};
  outs[0] = {token_out, (uint64_t)(b * 4)};
  outs[1] = {logits_out, logits_out ? (uint64_t)(b * n_eff * 4) : 0u};
  outs[2] = {ws, (uint64_t)mtp::kLmheadWsBytes};
  a = mtp::LmheadLaunch{};
  a.x = x;
  a.w = w;
  a.scale = scale;
  a.gscale = gscale;
  a.n = n_eff;
  a.h = (int)h;
  a.b = (int)b;
  a.wd = wd;
  a.token_out = token_out;
  a.logits = logits_out;
  a.ws = ws;
  return MTP_OK;
}

}  // namespace

extern "C" {

int mtp_lmhead_argmax(const uint16_t *x, int64_t b, int64_t h, int wd, const void *w,
                      const void *scale, const float *gscale, int64_t vocab,
                      int64_t mtp_vocab_size, int32_t *token_out, float *logits_out, void *ws,
                      size_t ws_bytes, void *stream) {
  mtp::LmheadLaunch a;
  Range ins[4], outs[3];
  const int st = lm_common(x, b, h, wd, w, scale, gscale, vocab, mtp_vocab_size, token_out,
                           logits_out, ws, ws_bytes, a, ins, outs);
  if (st != MTP_OK) return st;
  if (any_overlap(outs, 3, ins, 4)) return MTP_ERR_OVERLAP;
  return from_hip(mtp::launch_lmhead(a, (hipStream_t)stream));
}

int mtp_lmhead_argmax_logprob(const uint16_t *x, int64_t b, int64_t h, int wd, const void *w,
                              const void *scale, const float *gscale, int64_t vocab,
                              int64_t mtp_vocab_size, int32_t *token_out, float *logprob_out,
                              float *conf_inout, void *ws, size_t ws_bytes, void *stream) {
  mtp::LmheadLaunch a;
  Range ins[5], outs[5];
  const int st = lm_common(x, b, h, wd, w, scale, gscale, vocab, mtp_vocab_size, token_out, nullptr,
                           ws, ws_bytes, a, ins, outs);
  if (st != MTP_OK) return st;
  if (!logprob_out) return MTP_ERR_NULL;
  if (!aligned(logprob_out, 4) || (conf_inout && !aligned(conf_inout, 4))) return MTP_ERR_ALIGN;
  // conf_inout is read and written: it may overlap no input and no other output
  ins[4] = {conf_inout, conf_inout ? (uint64_t)(b * 4) : 0u};
  outs[3] = {logprob_out, (uint64_t)(b * 4)};
  outs[4] = {conf_inout, conf_inout ? (uint64_t)(b * 4) : 0u};
  if (any_overlap(outs, 5, ins, 4)) return MTP_ERR_OVERLAP;
  a.logprob = logprob_out;
  a.conf = conf_inout;
  return from_hip(mtp::launch_lmhead(a, (hipStream_t)stream));
}

int mtp_lmhead_argmax_masked(const uint16_t *x, int64_t b, int64_t h, int wd, const void *w,
                             const void *scale, const float *gscale, int64_t vocab,
                             int64_t mtp_vocab_size, const int32_t *mask, int64_t mask_words,
                             int32_t *token_out, int32_t *allowed_out, void *ws, size_t ws_bytes,
                             void *stream) {
  mtp::LmheadLaunch a;
  Range ins[5], outs[4];
  const int st = lm_common(x, b, h, wd, w, scale, gscale, vocab, mtp_vocab_size, token_out, nullptr,
                           ws, ws_bytes, a, ins, outs);
  if (st != MTP_OK) return st;
  if (!allowed_out || (mask_words > 0 && !mask)) return MTP_ERR_NULL;
  if (mask_words < 0 || mask_words > (int64_t(1) << 26)) return MTP_ERR_SHAPE;
  if (!aligned(allowed_out, 4) || (mask && !aligned(mask, 4))) return MTP_ERR_ALIGN;
  ins[4] = {mask, (uint64_t)(b * mask_words * 4)};
  outs[3] = {allowed_out, (uint64_t)(b * 4)};
  if (any_overlap(outs, 4, ins, 5)) return MTP_ERR_OVERLAP;
  a.masked = 1;  // with no mask words every row is rejected and the mask is never read
  a.mask = mask_words > 0 ? mask : nullptr;
  a.mask_words = (int)mask_words;
  a.allowed = allowed_out;
  return from_hip(mtp::launch_lmhead(a, (hipStream_t)stream));
}

size_t mtp_draft_step_workspace_bytes(int64_t b, int64_t h) {
  if (b < 1 || b > 8 || h < 16 || h > 8192) return 0;
  return mtp::step_ws_bytes(b, h);
}

}  // extern "C"

namespace {

// Stand-in for the library's own scratch in the argument checks of
// mtp_draft_step_noalloc: non-null, aligned, and host memory, so no device
// buffer a caller passes can overlap it.
alignas(256) const uint8_t kScratchStandIn[256] = {};

// mtp_draft_step's checks and launch; with own_ws the workspace is the
// library's scratch (ws is the stand-in, ws_bytes the scratch size).
int draft_step_impl(const uint16_t *embed_table, int64_t embed_vocab, const int32_t *token_ids,
                    int token_ids_on_device, const uint16_t *target_hidden,
                    const uint16_t *gamma_embed, const uint16_t *gamma_hidden, const uint16_t *fc_w,
                    const uint16_t *gamma_final, int64_t b, int64_t h, float eps, float gamma_offset,
                    int wd, const void *w, const void *scale, const float *gscale, int64_t vocab,
                    int64_t mtp_vocab_size, int32_t *token_out, uint16_t *x_out, float *logprob_out,
                    float *conf_inout, void *ws, size_t ws_bytes, bool own_ws, void *stream) {
  // the combine's checks (x_out is optional here: a stand-in passes the null check)
  mtp::CombineLaunch c;
  Range cins[7], couts[2];
  int st = combine_common(embed_table, embed_vocab, token_ids, token_ids_on_device != 0,
                          target_hidden, gamma_embed, gamma_hidden, gamma_final, b, h, eps,
                          gamma_offset, x_out ? x_out : const_cast<uint16_t *>(target_hidden), ws,
                          mtp_draft_combine_workspace_bytes(b, h), c, cins, couts);
  if (st != MTP_OK) return st;
  // the lm_head's checks (its x is internal: the hidden stands in for the check)
  mtp::LmheadLaunch l;
  Range lins[4], louts[3];
  st = lm_common(target_hidden, b, h, wd, w, scale, gscale, vocab, mtp_vocab_size, token_out, nullptr,
                 ws, ws_bytes, l, lins, louts);
  if (st != MTP_OK) return st;
  if (!fc_w) return MTP_ERR_NULL;
  if (!aligned(fc_w, 16) || (logprob_out && !aligned(logprob_out, 4)) ||
      (conf_inout && !aligned(conf_inout, 4)))
    return MTP_ERR_ALIGN;
  if (b * (4 * h + 16) > mtp::kMaxSweepLds) return MTP_ERR_SHAPE;  // concat vectors in LDS
  const size_t need = mtp_draft_step_workspace_bytes(b, h);
  if (ws_bytes < need) return MTP_ERR_WORKSPACE;
  // conf_inout is read and written: as an output it may overlap no input and no other output
  const Range ins[] = {cins[0], cins[1], cins[2], cins[3], cins[4], cins[5],
                       {fc_w, (uint64_t)(h * 2 * h * 2)}, lins[1], lins[2], lins[3]};
  const Range outs[] = {{token_out, (uint64_t)(b * 4)},
                        {x_out, x_out ? (uint64_t)(b * h * 2) : 0u},
                        {logprob_out, logprob_out ? (uint64_t)(b * 4) : 0u},
                        {conf_inout, conf_inout ? (uint64_t)(b * 4) : 0u},
                        {ws, (uint64_t)need}};
  if (any_overlap(outs, 5, ins, 10)) return MTP_ERR_OVERLAP;
  c.fc = fc_w;
  c.x_out = x_out;
  l.logprob = logprob_out;
  l.conf = conf_inout;
  mtp::StepLaunch a{c, l, ws};
  if (own_ws) return from_hip(mtp::launch_step_scratch(a, (hipStream_t)stream));
  return from_hip(mtp::launch_step(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int mtp_draft_step(const uint16_t *embed_table, int64_t embed_vocab, const int32_t *token_ids,
                   int token_ids_on_device, const uint16_t *target_hidden,
                   const uint16_t *gamma_embed, const uint16_t *gamma_hidden, const uint16_t *fc_w,
                   const uint16_t *gamma_final, int64_t b, int64_t h, float eps, float gamma_offset,
                   int wd, const void *w, const void *scale, const float *gscale, int64_t vocab,
                   int64_t mtp_vocab_size, int32_t *token_out, uint16_t *x_out, float *logprob_out,
                   float *conf_inout, void *ws, size_t ws_bytes, void *stream) {
  return draft_step_impl(embed_table, embed_vocab, token_ids, token_ids_on_device, target_hidden,
                         gamma_embed, gamma_hidden, fc_w, gamma_final, b, h, eps, gamma_offset, wd, w,
                         scale, gscale, vocab, mtp_vocab_size, token_out, x_out, logprob_out,
                         conf_inout, ws, ws_bytes, false, stream);
}

int mtp_draft_step_noalloc(const uint16_t *embed_table, int64_t embed_vocab,
                           const int32_t *token_ids, int token_ids_on_device,
                           const uint16_t *target_hidden, const uint16_t *gamma_embed,
                           const uint16_t *gamma_hidden, const uint16_t *fc_w,
                           const uint16_t *gamma_final, int64_t b, int64_t h, float eps,
                           float gamma_offset, int wd, const void *w, const void *scale,
                           const float *gscale, int64_t vocab, int64_t mtp_vocab_size,
                           int32_t *token_out, uint16_t *x_out, float *logprob_out,
                           float *conf_inout, void *stream) {
  return draft_step_impl(embed_table, embed_vocab, token_ids, token_ids_on_device, target_hidden,
                         gamma_embed, gamma_hidden, fc_w, gamma_final, b, h, eps, gamma_offset, wd, w,
                         scale, gscale, vocab, mtp_vocab_size, token_out, x_out, logprob_out,
                         conf_inout, const_cast<uint8_t *>(kScratchStandIn), mtp::kStepScratchBytes, true,
                         stream);
}

int mtp_codec_encode_range(int codec, uint32_t first_bits, int64_t count, uint8_t *out,
                           void *stream) {
  if (codec != MTP_CODEC_E4M3 && codec != MTP_CODEC_E2M1 && codec != MTP_CODEC_BF16) return MTP_ERR_DTYPE;
  if (!out) return MTP_ERR_NULL;
  if (count < 1 || (uint64_t)first_bits + (uint64_t)count > (uint64_t(1) << 32)) return MTP_ERR_SHAPE;
  if (!aligned(out, 16)) return MTP_ERR_ALIGN;
  return from_hip(mtp::launch_codec_range(codec, first_bits, count, out, (hipStream_t)stream));
}

int mtp_stream_read(const void *buf, int64_t bytes, int shape, uint32_t magic, uint32_t *sink, void *stream) {
  if (!buf || !sink) return MTP_ERR_NULL;
  if (bytes < 8192 || shape < 0 || shape > 5) return MTP_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return MTP_ERR_ALIGN;
  return from_hip(mtp::launch_stream_read(buf, bytes, shape, magic, sink, (hipStream_t)stream));
}

}  // extern "C"
