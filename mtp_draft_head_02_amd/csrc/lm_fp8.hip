// lm_head sweep + argmax: the FP8 instantiations (a translation unit of its own so the build
// compiles the formats in parallel).
#include "sweep_impl.h"

namespace mtp {

hipError_t launch_lmhead_fp8(int b, const SweepParams &p, hipStream_t s) {
  return launch_lmhead_wd<kFP8>(b, p, s);
}

}  // namespace mtp
