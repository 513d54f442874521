// Merge of the per-partition results of the split-KV kernels.
//
// Each KV partition s of a sequence left, for every query row, a normalised
// output O_s and the log2-sum-exp lse_s of its scaled scores (log2 units).
// The exact result over the union of the partitions is the log-sum-exp
// combination (the running-max / running-sum recurrence of online softmax,
// ops-transformer articles, applied once across partitions):
//     M = max_s lse_s,  w_s = 2^(lse_s - M),  L = sum_s w_s,
//     O = sum_s w_s O_s / L,  lse = (M + log2 L) * ln 2   (natural log).
// A row whose partitions all saw no key (M = -inf) gets O = 0, lse = -inf.
//
// One wave per output row (b, h, i); lanes split the D channels.  Only the
// n_s = ceil(n_b / chunk) partitions that exist for sequence b are read.
#include "device_common.h"
#include "launch.h"

namespace mxfa {
namespace {

template <int DT, int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    constexpr int PER = D / 64;                 // channels per lane (1 or 2)
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const long long nrows = (long long)a.B * a.Hq * a.qLen;
    if (row >= nrows) return;
    const int i = (int)(row % a.qLen);
    const int h = (int)((row / a.qLen) % a.Hq);
    const int b = (int)(row / ((long long)a.qLen * a.Hq));

    const int n = clampi(a.seqlens ? a.seqlens[b] : a.kv_cap, 0, a.kv_cap);
    const int ns = clampi((n + a.chunk - 1) / a.chunk, 1, a.S);
    const float *lrow = a.ws_lse + (size_t)row * a.S;   // row = (b*Hq + h)*qLen + i
    const float *orow = a.ws_o + (size_t)row * a.S * D;

    float M = kNegInf;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, lrow[s]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));

    float acc[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] = 0.f;
    float L = 0.f;
    if (M != kNegInf) {
        for (int s = 0; s < ns; ++s) {
            const float w = fast_exp2(lrow[s] - M);   // -inf partitions weigh 0
            L += w;
            const float *op = orow + (size_t)s * D + lane * PER;
            if constexpr (PER == 2) {
                const f32x2 x = *(const f32x2 *)op;
                acc[0] = fmaf(w, x[0], acc[0]);
                acc[1] = fmaf(w, x[1], acc[1]);
            } else {
                acc[0] = fmaf(w, op[0], acc[0]);
            }
        }
    }
    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    uint16_t *outp = (uint16_t *)a.out + (((size_t)b * a.qLen + i) * a.Hq + h) * D + lane * PER;
    if constexpr (PER == 2)
        *(uint32_t *)outp = pack2<DT>(acc[0] * inv, acc[1] * inv);
    else
        *outp = (uint16_t)to16<DT>(acc[0] * inv);
    if (lane == 0 && a.lse) a.lse[row] = empty ? kNegInf : (M + fast_log2(L)) * kLn2;
}

template <int DT, int D>
hipError_t launch_t(const CombineArgs &a, hipStream_t stream) {
    CombineArgs args = a;
    void *kargs[] = {&args};
    const long long nrows = (long long)a.B * a.Hq * a.qLen;
    const unsigned blocks = (unsigned)((nrows + 3) / 4);
    return hipLaunchKernel((const void *)&combine_kernel<DT, D>, dim3(blocks), dim3(256),
                           kargs, 0, stream);
}

}  // namespace

hipError_t launch_combine(const CombineArgs &a, int dtype, int D, hipStream_t stream) {
    if (dtype == kFp16) {
        if (D == 128) return launch_t<kFp16, 128>(a, stream);
        if (D == 64) return launch_t<kFp16, 64>(a, stream);
    } else {
        if (D == 128) return launch_t<kBf16, 128>(a, stream);
        if (D == 64) return launch_t<kBf16, 64>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mxfa
