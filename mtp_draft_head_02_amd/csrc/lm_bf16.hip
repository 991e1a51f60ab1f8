// lm_head sweep + argmax: the BF16 instantiations (a translation unit of its own so the build
// compiles the formats in parallel).
#include "mfma_impl.h"

namespace mtp {

bool lmhead_mfma_bf16(int b, int k) { return mfma_takes<kBF16>(b, k); }

hipError_t launch_lmhead_bf16(int b, const SweepParams &p, hipStream_t s) {
  if (lmhead_mfma_bf16(b, p.k)) return launch_mfma_bf16(b, p, s);
  return launch_lmhead_wd<kBF16>(b, p, s);
}

}  // namespace mtp
