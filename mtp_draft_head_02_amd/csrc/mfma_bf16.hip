// lm_head sweep + argmax on the matrix cores: the BF16 instantiations (a translation
// unit of its own so the build compiles the formats in parallel).
#include "mfma_impl.h"

namespace mtp {

hipError_t launch_mfma_bf16(int b, const SweepParams &p, hipStream_t s) {
  return launch_mfma_wd<kBF16>(b, p, s);
}

}  // namespace mtp
