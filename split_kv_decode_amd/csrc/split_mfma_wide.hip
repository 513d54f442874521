// Matrix-core split kernel, wide heads (tile widths 192 x 128 and 256 x 256).
#include "mfma_kernel.h"

namespace mxfa {

hipError_t launch_split_mfma_wide(const KernelArgs &a, int dtype, dim3 grid,
                                  hipStream_t stream) {
    int dk, dv;
    mfma_tile_dims(a.Dk, a.Dv, &dk, &dv);
    if (dk == 192 && dv == 128) return mfma::launch_dims<192, 128>(a, dtype, grid, stream);
    if (dk == 256 && dv == 256) return mfma::launch_dims<256, 256>(a, dtype, grid, stream);
    return hipErrorInvalidValue;
}

}  // namespace mxfa
