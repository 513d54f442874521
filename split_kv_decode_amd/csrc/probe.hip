// Streaming-read probe: the practical HBM read ceiling that the attention
// kernels' bandwidth is set against.  Each workgroup streams its own
// contiguous share of the source (consecutive lanes read consecutive 16-byte
// chunks, UNR loads in flight per thread) through a buffer descriptor that
// ends with the share, and folds the data into one xor so the loads stay
// live.  Nothing is written unless the fold hits a fixed 32-bit pattern, so
// the write traffic is nil.  Contiguous shares per workgroup read faster
// than a grid-wide strided walk on this GPU, so this is the pattern measured.
#include "device_common.h"
#include "mxfa.h"

namespace mxfa {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocksPerCu = 2;
constexpr int kProbeUnroll = 8;
constexpr uint32_t kProbeMarker = 0x9e3779b9u;

template <int POLICY>
__global__ __launch_bounds__(kProbeThreads)
void read_probe_kernel(const void *__restrict__ src, uint32_t bytes, uint32_t *sink) {
    const uint32_t n16 = bytes / 16;
    const uint32_t share = (n16 + gridDim.x - 1) / gridDim.x;
    const uint32_t lo = min((uint32_t)blockIdx.x * share, n16);
    const uint32_t len = min(share, n16 - lo);
    const __amdgpu_buffer_rsrc_t r = make_rsrc((const uint8_t *)src + (size_t)lo * 16, len * 16);
    uint32_t acc = 0;
    for (uint32_t i = threadIdx.x; i < len; i += kProbeThreads * kProbeUnroll) {
        u32x4 x[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u)   // chunks past the share read as 0
            x[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (i + u * kProbeThreads) * 16, 0, POLICY);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
    }
    if (acc == kProbeMarker) *sink = acc;
}

}  // namespace
}  // namespace mxfa

extern "C" {

MXFA_API mxfa_status mxfa_read_probe(const void *src, size_t bytes, int nontemporal,
                                     uint32_t *sink, int num_cus, void *stream) {
    using namespace mxfa;
    if (src == nullptr || sink == nullptr || bytes == 0) return MXFA_ERR_INVALID_ARG;
    if (((uintptr_t)src & 15) != 0 || ((uintptr_t)sink & 3) != 0 || bytes % 16 != 0 ||
        bytes > ((size_t)1 << 31) || (nontemporal != 0 && nontemporal != 1) ||
        num_cus > 4096)
        return MXFA_ERR_INVALID_ARG;
    const int cus = num_cus > 0 ? num_cus : 256;
    const unsigned blocks = (unsigned)cus * kProbeBlocksPerCu;
    const uint32_t nb = (uint32_t)bytes;
    void *args[] = {(void *)&src, (void *)&nb, (void *)&sink};
    const void *fn = nontemporal ? (const void *)&read_probe_kernel<2>
                                 : (const void *)&read_probe_kernel<0>;
    if (hipLaunchKernel(fn, dim3(blocks), dim3(kProbeThreads), args, 0,
                        (hipStream_t)stream) != hipSuccess)
        return MXFA_ERR_HIP;
    return MXFA_OK;
}

}  // extern "C"
