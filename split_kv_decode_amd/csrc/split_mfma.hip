// Matrix-core split kernel, head dims up to 128 (tile widths 64 and 128).
#include "mfma_kernel.h"

namespace mxfa {

hipError_t launch_split_mfma(const KernelArgs &a, int dtype, dim3 grid, hipStream_t stream) {
    if (odd_head_dims(a.Dk, a.Dv)) return launch_split_mfma_odd(a, dtype, grid, stream);
    int dk, dv;
    mfma_tile_dims(a.Dk, a.Dv, &dk, &dv);
    if (dk == 64 && dv == 64) return mfma::launch_dims<64, 64>(a, dtype, grid, stream);
    if (dk == 128 && dv == 128) return mfma::launch_dims<128, 128>(a, dtype, grid, stream);
    return launch_split_mfma_wide(a, dtype, grid, stream);
}

}  // namespace mxfa
