// The combine with its fc on the matrix cores (wide batches, BF16 fc): the
// instantiations (a translation unit of its own so the build compiles it in
// parallel with the others).
#include "combine_mfma_impl.h"

namespace mtp {

bool combine_uses_mfma(int b, int k) { return combine_mfma_ok(b, k); }

hipError_t launch_combine_mfma(int b, const SweepParams &p, hipStream_t s) {
  switch (b) {
    case 1: return launch_combine_mfma_b<1>(p, s);
    case 2: return launch_combine_mfma_b<2>(p, s);
    case 3: return launch_combine_mfma_b<3>(p, s);
    case 4: return launch_combine_mfma_b<4>(p, s);
    case 5: return launch_combine_mfma_b<5>(p, s);
    case 6: return launch_combine_mfma_b<6>(p, s);
    case 7: return launch_combine_mfma_b<7>(p, s);
    case 8: return launch_combine_mfma_b<8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mtp
