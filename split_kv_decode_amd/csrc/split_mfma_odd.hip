// Matrix-core split kernel for head dims that are not multiples of 8 (any
// tile width; element loads and stores).
#include "mfma_kernel.h"

namespace mxfa {

hipError_t launch_split_mfma_odd(const KernelArgs &a, int dtype, dim3 grid, hipStream_t stream) {
    int dk, dv;
    mfma_tile_dims(a.Dk, a.Dv, &dk, &dv);
    if (dk == 64 && dv == 64) return mfma::launch_odd_dims<64, 64>(a, dtype, grid, stream);
    if (dk == 128 && dv == 128) return mfma::launch_odd_dims<128, 128>(a, dtype, grid, stream);
    if (dk == 192 && dv == 128) return mfma::launch_odd_dims<192, 128>(a, dtype, grid, stream);
    if (dk == 256 && dv == 256) return mfma::launch_odd_dims<256, 256>(a, dtype, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace mxfa
