// Host entry points of the sweep kernels: argument packing and dispatch to the
// per-format instantiations (the kernels and their templates: sweep_impl.h).
#include "sweep_impl.h"

namespace mtp {

static hipError_t launch_fc(int wd, bool split, int b, const SweepParams &p, hipStream_t s) {
  if (split) return wd == kBF16 ? launch_fc_bf16(b, true, p, s) : hipErrorInvalidValue;
  if (wd == kBF16 && combine_uses_mfma(b, p.k)) return launch_combine_mfma(b, p, s);
  switch (wd) {
    case kBF16: return launch_fc_bf16(b, false, p, s);
    case kFP8: return launch_fc_fp8(b, p, s);
    case kNVFP4: return launch_fc_nvfp4(b, p, s);
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
  p.kmax = reinterpret_cast<unsigned long long *>(static_cast<uint8_t *>(a.ws) + kLmheadKmaxOffset);
  p.partials = reinterpret_cast<unsigned long long *>(static_cast<uint8_t *>(a.ws) + 256);
  p.psums = reinterpret_cast<float *>(static_cast<uint8_t *>(a.ws) + kLmheadPsumsOffset);
  p.token_out = a.token_out;
  p.logprob_out = a.logprob;
  p.conf_inout = a.conf;
  p.masked = a.masked;
  p.mask = a.mask;
  p.mask_words = a.mask_words;
  p.allowed_out = a.allowed;
  switch (a.wd) {
    case kBF16: return launch_lmhead_bf16(a.b, p, s);
    case kFP8: return launch_lmhead_fp8(a.b, p, s);
    case kNVFP4: return launch_lmhead_nvfp4(a.b, p, s);
    default: return hipErrorInvalidValue;
  }
}

size_t step_ws_bytes(int64_t b, int64_t h) {
  return kStepWsUOffset + (size_t)(b * h * 2 + 255) / 256 * 256 + (size_t)(b * 2 * h * 2 + 255) / 256 * 256;
}

// The draft step in two launches on one stream: the combine stops after
// storing u (no ticket, no last-block final norm); every lm_head block then
// stages x = rms(u, g_f) itself (block 0 also writes x_out) while its first
// weight units are in flight, and sweeps as usual.
hipError_t launch_step(const StepLaunch &a, hipStream_t s) {
  const CombineLaunch &c = a.c;
  const LmheadLaunch &l = a.l;
  uint8_t *ws = static_cast<uint8_t *>(a.ws);
  uint16_t *u = reinterpret_cast<uint16_t *>(ws + kStepWsUOffset);
  uint16_t *cc = reinterpret_cast<uint16_t *>(ws + kStepWsUOffset + (size_t)(c.b * c.h * 2 + 255) / 256 * 256);
  if (c.b * (4 * c.h + 16) > kMaxSweepLds) return hipErrorInvalidValue;  // concat vectors in LDS
  SweepParams pc{};
  pc.w = static_cast<const uint8_t *>(c.fc);
  pc.n = c.h;
  pc.k = 2 * c.h;
  pc.embed = c.embed;
  for (int i = 0; i < 8; ++i) pc.tokens[i] = i < c.b ? c.tokens[i] : 0;
  pc.tokens_dev = c.tokens_dev;
  pc.vocab = c.vocab;
  pc.hidden = c.hidden;
  pc.gamma_e = c.gamma_e;
  pc.gamma_h = c.gamma_h;
  pc.eps = c.eps;
  pc.gamma_offset = c.gamma_offset;
  pc.y = u;
  pc.c_out = cc;
  pc.no_final = 1;
  hipError_t e = launch_fc(kBF16, false, c.b, pc, s);
  if (e != hipSuccess) return e;
  SweepParams pl{};
  pl.w = static_cast<const uint8_t *>(l.w);
  pl.scale = l.scale;
  pl.gscale = l.gscale;
  pl.n = l.n;
  pl.k = l.h;
  pl.ticket = static_cast<unsigned *>(a.ws);
  pl.kmax = reinterpret_cast<unsigned long long *>(ws + kLmheadKmaxOffset);
  pl.partials = reinterpret_cast<unsigned long long *>(ws + 256);
  pl.psums = reinterpret_cast<float *>(ws + kLmheadPsumsOffset);
  pl.token_out = l.token_out;
  pl.logprob_out = l.logprob;
  pl.conf_inout = l.conf;
  pl.u_in = u;
  pl.gamma_f = c.gamma_f;
  pl.eps = c.eps;
  pl.gamma_offset = c.gamma_offset;
  pl.x_out = c.x_out;
  switch (l.wd) {
    case kBF16: return launch_lmhead_bf16(c.b, pl, s);
    case kFP8: return launch_lmhead_fp8(c.b, pl, s);
    case kNVFP4: return launch_lmhead_nvfp4(c.b, pl, s);
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
  uint16_t *cc = reinterpret_cast<uint16_t *>(ws + 256);
  uint16_t *u = reinterpret_cast<uint16_t *>(ws + 256 + (size_t)(b * 2 * h * 2 + 255) / 256 * 256);
  // one launch per group of batch rows whose concat vectors fit in LDS
  const int k = 2 * h;
  int bp = kMaxSweepLds / (k * 2 + 16);
  if (bp > 8) bp = 8;
  if (bp < 1) return hipErrorInvalidValue;
  for (int b0 = 0; b0 < b; b0 += bp) {
    const int nb = (b - b0) < bp ? (b - b0) : bp;
    SweepParams p{};
    p.w = static_cast<const uint8_t *>(a.fc);
    p.scale = a.fc_scale;
    p.gscale = a.fc_gscale;
    p.w2 = reinterpret_cast<const uint8_t *>(a.h_proj);
    p.n = h;
    p.k = k;
    p.ticket = ticket;
    p.embed = a.embed;
    for (int i = 0; i < 8; ++i) p.tokens[i] = (b0 + i < b) ? a.tokens[b0 + i] : 0;
    p.tokens_dev = a.tokens_dev ? a.tokens_dev + b0 : nullptr;
    p.vocab = a.vocab;
    p.hidden = a.hidden + (int64_t)b0 * h;
    p.gamma_e = a.gamma_e;
    p.gamma_h = a.gamma_h;
    p.y = u + (int64_t)b0 * h;
    p.c_out = cc + (int64_t)b0 * 2 * h;
    p.gamma_f = a.gamma_f;
    p.eps = a.eps;
    p.gamma_offset = a.gamma_offset;
    p.x_out = a.x_out + (int64_t)b0 * h;
    const hipError_t e = launch_fc(a.fc_wd, a.h_proj != nullptr, nb, p, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mtp
