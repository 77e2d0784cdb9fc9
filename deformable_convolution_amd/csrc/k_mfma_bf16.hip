// k_mfma_bf16.hip -- instantiates the fused MFMA kernels (mfma_kernel.h) for
// bfloat16 storage, no mask.
#include "mfma_kernel.h"

namespace dc1d {

hipError_t launch_mfma_bf16(const Params &p, const MfmaPlan &pl, hipStream_t stream) {
    return launch_for<TrBF16, false>(p, pl, stream);
}

}  // namespace dc1d
