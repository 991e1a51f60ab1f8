// The combine: the BF16 fc (concat and split forms) instantiations (a translation unit of its own so the build
// compiles the formats in parallel).
#include "sweep_impl.h"

namespace mtp {

hipError_t launch_fc_bf16(int b, bool split, const SweepParams &p, hipStream_t s) {
  return split ? launch_fc_wd<kBF16, kStoreSplit>(b, p, s) : launch_fc_wd<kBF16, kStoreBf16>(b, p, s);
}

}  // namespace mtp
