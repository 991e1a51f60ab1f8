// lm_head sweep + argmax: the NVFP4 instantiations (a translation unit of its own so the build
// compiles the formats in parallel).
#include "sweep_impl.h"

namespace mtp {

hipError_t launch_lmhead_nvfp4(int b, const SweepParams &p, hipStream_t s) {
  return launch_lmhead_wd<kNVFP4>(b, p, s);
}

}  // namespace mtp
