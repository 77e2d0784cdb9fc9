// k_mfma_f32_mask.hip -- instantiates the fused MFMA kernels (mfma_kernel.h) for
// fp32 storage with a modulation mask.
#include "mfma_kernel.h"

namespace dc1d {

hipError_t launch_mfma_f32_mask(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    return launch_for<TrF32, true>(p, pl, stream);
}

}  // namespace dc1d
