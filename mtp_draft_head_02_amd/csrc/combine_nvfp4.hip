// The combine: the NVFP4 fc instantiations (a translation unit of its own so the build
// compiles the formats in parallel).
#include "sweep_impl.h"

namespace mtp {

hipError_t launch_fc_nvfp4(int b, const SweepParams &p, hipStream_t s) {
  return launch_fc_wd<kNVFP4, kStoreBf16>(b, p, s);
}

}  // namespace mtp
