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
// One wave per output row (b, h, i).  The row belongs to the stream of its
// (sequence, head block, row block); the slots that hold the stream's
// partials are consecutive (see launch.h): with fixed partitions the
// ceil(n_b / chunk) partitions of the stream, with the balanced schedule the
// workgroups whose share of the concatenated streams overlaps it.  A stream
// served by one workgroup was written directly by the split kernel and is
// skipped; a stream with no token at all gets O = 0, lse = -inf here.  The
// weights are computed
// with one partition per lane and kept in LDS; the weighted sum then splits
// the wave into NG groups of D/4 lanes (4 channels per lane, 16-byte loads),
// each group taking every NG-th partition with UNR loads in flight, and the
// groups are summed with cross-lane exchanges.  D here is the channel count
// of a partial row (the head dim, or the matrix-core kernel's padded V tile);
// only the first Dv channels are written out.
#include "device_common.h"
#include "launch.h"

namespace mxfa {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kMaxStaged = 256;     // weights staged in LDS per pass

template <int DT, int D>
__global__ __launch_bounds__(kRowsPerBlock * 64) void combine_kernel(KernelArgs a) {
    constexpr int LPG = D / 4;                  // lanes per group
    constexpr int NG = 64 / LPG;                // groups per wave (2 or 4)
    constexpr int UNR = 4;
    __shared__ float lds_w[kRowsPerBlock][kMaxStaged];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const long long row = (long long)blockIdx.x * kRowsPerBlock + wave;
    const long long nrows = (long long)a.B * a.Hq * a.qLen;
    if (row >= nrows) return;                   // whole wave exits together
    const int i = (int)(row % a.qLen);
    const int h = (int)((row / a.qLen) % a.Hq);
    const int b = (int)(row / ((long long)a.qLen * a.Hq));
    if (i >= q_count(a, b)) return;             // past a packed sequence's queries
    const int kvh = h / a.G;
    const int rg = i * a.G + h % a.G;           // row index within the kv head
    const int hb = kvh / a.head_block, hx = kvh % a.head_block;
    const int rb = rg / a.row_block, r = rg % a.row_block;
    const int HR = a.head_blocks * a.row_blocks;
    const int jst = hb * a.row_blocks + rb;     // stream index within sequence b
    const int st = b * HR + jst;

    const int n = seq_len(a, b);
    long long first;
    int count;
    if (a.schedule == kFixed) {
        count = (n + a.chunk - 1) / a.chunk;
        first = (long long)st * a.S;
    } else if (n > 0) {
        const long long *cw = (const long long *)a.ws_cum;
        const long long W = cw[a.B + 1];
        const long long c0 = cw[b] * HR + (long long)jst * n;   // stream start
        const long long w_lo = c0 / W, w_hi = (c0 + n - 1) / W;
        count = (int)(w_hi - w_lo + 1);
        first = w_lo + st;
    } else {
        count = 0;
        first = 0;
    }
    if (count == 1) return;                     // written by the split kernel

    const size_t stride = (size_t)a.head_block * a.row_block;   // entries per slot
    const size_t e0 = ((size_t)first * a.head_block + hx) * a.row_block + r;
    const float *lrow = a.ws_lse + e0;           // entry of slot k at lrow[k * stride]
    const float *orow = a.ws_o + e0 * D;         // row of slot k at orow[k * stride * D]

    float M = kNegInf;
    for (int s = lane; s < count; s += 64) M = fmaxf(M, lrow[(size_t)s * stride]);
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));

    const int g = lane / LPG;
    const int d0 = (lane % LPG) * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != kNegInf) {
        for (int s0 = 0; s0 < count; s0 += kMaxStaged) {
            const int cnt = min(count - s0, kMaxStaged);
            for (int s = lane; s < cnt; s += 64) {
                const float w = fast_exp2(lrow[(size_t)(s0 + s) * stride] - M);
                lds_w[wave][s] = w;                     // -inf partials weigh 0
                L += w;
            }
            wave_lds_sync();
            int s = g;
            for (; s + (UNR - 1) * NG < cnt; s += UNR * NG) {
                f32x4 x[UNR];
#pragma unroll
                for (int u = 0; u < UNR; ++u)
                    x[u] = *(const f32x4 *)(orow + (size_t)(s0 + s + u * NG) * stride * D + d0);
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const float w = lds_w[wave][s + u * NG];
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[j] = fmaf(w, x[u][j], acc[j]);
                }
            }
            for (; s < cnt; s += NG) {
                const f32x4 x = *(const f32x4 *)(orow + (size_t)(s0 + s) * stride * D + d0);
                const float w = lds_w[wave][s];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = fmaf(w, x[j], acc[j]);
            }
            wave_lds_sync();
        }
    }
#pragma unroll
    for (int x = 32; x >= 1; x >>= 1) L += __shfl_xor(L, x);
#pragma unroll
    for (int x = LPG; x < 64; x <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], x);

    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    if (g == 0 && d0 < a.Dv) {
        uint16_t *outp = (uint16_t *)a.out + (q_token(a, b, i) * a.Hq + h) * a.Dv + d0;
        *(u32x2 *)outp = u32x2{pack2<DT>(acc[0] * inv, acc[1] * inv),
                               pack2<DT>(acc[2] * inv, acc[3] * inv)};
    }
    if (lane == 0 && a.lse) a.lse[lse_index(a, b, h, i)] = empty ? kNegInf : (M + fast_log2(L)) * kLn2;
}

template <int DT, int D>
hipError_t launch_t(const KernelArgs &a, hipStream_t stream) {
    KernelArgs args = a;
    void *kargs[] = {&args};
    const long long nrows = (long long)a.B * a.Hq * a.qLen;
    const unsigned blocks = (unsigned)((nrows + kRowsPerBlock - 1) / kRowsPerBlock);
    return hipLaunchKernel((const void *)&combine_kernel<DT, D>, dim3(blocks),
                           dim3(kRowsPerBlock * 64), kargs, 0, stream);
}

}  // namespace

hipError_t launch_combine(const KernelArgs &a, int dtype, hipStream_t stream) {
    if (dtype == kFp16) {
        if (a.dv_tile == 128) return launch_t<kFp16, 128>(a, stream);
        if (a.dv_tile == 64) return launch_t<kFp16, 64>(a, stream);
        if (a.dv_tile == 256) return launch_t<kFp16, 256>(a, stream);
    } else {
        if (a.dv_tile == 128) return launch_t<kBf16, 128>(a, stream);
        if (a.dv_tile == 64) return launch_t<kBf16, 64>(a, stream);
        if (a.dv_tile == 256) return launch_t<kBf16, 256>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mxfa
