// lm_head sweep + argmax: the FP8 instantiations (a translation unit of its own so the build
// compiles the formats in parallel).
#include "mfma_impl.h"

namespace mtp {

bool lmhead_mfma_fp8(int b, int k) { return mfma_takes<kFP8>(b, k); }

hipError_t launch_lmhead_fp8(int b, const SweepParams &p, hipStream_t s) {
  if (lmhead_mfma_fp8(b, p.k)) return launch_mfma_fp8(b, p, s);
  return launch_lmhead_wd<kFP8>(b, p, s);
}

}  // namespace mtp
