// The combine: the FP8 fc instantiations (a translation unit of its own so the build
// compiles the formats in parallel).
#include "sweep_impl.h"

namespace mtp {

hipError_t launch_fc_fp8(int b, const SweepParams &p, hipStream_t s) {
  return launch_fc_wd<kFP8, kStoreBf16>(b, p, s);
}

}  // namespace mtp
