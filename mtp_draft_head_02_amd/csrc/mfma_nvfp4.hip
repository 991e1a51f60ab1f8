// lm_head sweep + argmax on the matrix cores: the NVFP4 instantiations (a translation
// unit of its own so the build compiles the formats in parallel).
#include "mfma_impl.h"

namespace mtp {

hipError_t launch_mfma_nvfp4(int b, const SweepParams &p, hipStream_t s) {
  return launch_mfma_wd<kNVFP4>(b, p, s);
}

}  // namespace mtp
