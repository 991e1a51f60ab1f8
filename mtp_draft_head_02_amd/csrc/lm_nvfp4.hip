// lm_head sweep + argmax: the NVFP4 instantiations (a translation unit of its own so the build
// compiles the formats in parallel).
#include "mfma_impl.h"

namespace mtp {

bool lmhead_mfma_nvfp4(int b, int k) { return mfma_takes<kNVFP4>(b, k); }

hipError_t launch_lmhead_nvfp4(int b, const SweepParams &p, hipStream_t s) {
  if (lmhead_mfma_nvfp4(b, p.k)) return launch_mfma_nvfp4(b, p, s);
  return launch_lmhead_wd<kNVFP4>(b, p, s);
}

}  // namespace mtp
