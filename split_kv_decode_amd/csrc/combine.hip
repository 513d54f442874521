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
// wave splits into NG groups of D/4 lanes (4 channels per lane, 16-byte
// loads), each group taking every NG-th partition; the lse values of the
// first 128 partitions (two per lane) and the first 16 partition rows per
// lane are loaded together, so the maximum and the weights cost no extra
// memory round trip (with 4 waves per row that covers 128 partitions).
// A partition's weight travels from its lane by a cross-lane read, and the
// groups are summed with cross-lane exchanges.  D here is the channel count
// of a partial row (the head dim, or the matrix-core kernel's padded V tile);
// only the first Dv channels are written out.
#include "device_common.h"
#include "launch.h"
#include "schedule.h"

namespace mxfa {
namespace {

constexpr int kWaves = 4;                    // waves per workgroup

// WPR waves per output row: 1 when rows have few partials, 4 (one workgroup
// per row) when they have many, so that the partial rows of one output row
// are read by 4 waves at once.  MANY (with WPR = 4): rows with more than 64
// partials; each lane then holds two lse values and 16 partial rows in
// flight, so up to 128 partials cost one memory round trip.
template <int DT, int D, int WPR, bool MANY>
__global__ __launch_bounds__(kWaves * 64) void combine_kernel(KernelArgs a) {
    constexpr int LPG = D / 4;                  // lanes per group
    constexpr int NG = 64 / LPG;                // groups per wave (1, 2 or 4)
    constexpr int UNR = (WPR == 1 || MANY) ? 16 : 8;   // partial rows in flight per lane
    constexpr int NLSE = MANY ? 128 : 64;       // partials whose lse the lanes hold
    constexpr int RPB = kWaves / WPR;           // rows per workgroup
    constexpr int STEP = WPR * NG;              // partials between a lane's loads
    __shared__ f32x4 lds_acc[WPR > 1 ? WPR : 1][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = wave % WPR;                 // this wave's share of the partials
    // rows in XCD order (schedule.h): a row is merged on the XCD whose
    // workgroups wrote most of its partials (its reads still miss that XCD's
    // L2, which the split kernel's end has written back)
    const long long row = (long long)xcd_order(blockIdx.x, gridDim.x) * RPB + wave / WPR;
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
        // the prefix sums and the share size the split kernel used; without
        // per-sequence lengths every sequence holds n keys and both follow
        // directly, with no load of what the split kernel stored
        const bool uniform = a.seqlens == nullptr && a.cu_k == nullptr;
        if (uniform && a.uni_spw > 0) {
            count = a.uni_spw;                  // shares st * spw + i, slots + st
            first = (long long)st * (a.uni_spw + 1);
        } else {
            long long cb, W;
            if (uniform) {
                cb = (long long)b * n;
                W = a.uni_w;
            } else {
                const long long *cw = (const long long *)a.ws_cum;
                cb = cw[b];
                W = cw[a.B + 1];
            }
            const long long c0 = cb * HR + (long long)jst * n;   // stream start
            const long long w_lo = c0 / W, w_hi = (c0 + n - 1) / W;
            count = (int)(w_hi - w_lo + 1);
            first = w_lo + st;
        }
    } else {
        count = 0;
        first = 0;
    }
    if (count == 1) return;                     // written by the split kernel

    const size_t stride = (size_t)a.head_block * a.row_block;   // entries per slot
    const size_t e0 = ((size_t)first * a.head_block + hx) * a.row_block + r;
    const float *lrow = a.ws_lse + e0;           // entry of slot k at lrow[k * stride]
    const float *orow = a.ws_o + e0 * D;         // row of slot k at orow[k * stride * D]
    const int g = sub * NG + lane / LPG;        // first partial of this lane
    const int d0 = (lane % LPG) * 4;
    auto orow_of = [&](int s) { return *(const f32x4 *)(orow + (size_t)s * stride * D + d0); };

    // the partials' lse (lane s holds partial s, and 64 + s with MANY) and the
    // first UNR * STEP partial rows are loaded together, before the maximum
    // is known
    const float lv0 = lane < count ? lrow[(size_t)lane * stride] : kNegInf;
    const float lv1 = MANY && lane + 64 < count ? lrow[(size_t)(lane + 64) * stride] : kNegInf;
    f32x4 x[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
        const int sp = g + u * STEP;
        x[u] = sp < count ? orow_of(sp) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float M = fmaxf(lv0, lv1);
    for (int sp = lane + NLSE; sp < count; sp += 64) M = fmaxf(M, lrow[(size_t)sp * stride]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m));

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    if (M != kNegInf) {
        // weights of partials s < NLSE sit in lane s % 64; -inf partials weigh 0
        const float w0 = fast_exp2(lv0 - M);
        const float w1 = MANY ? fast_exp2(lv1 - M) : 0.f;
        L = w0 + w1;
        for (int sp = lane + NLSE; sp < count; sp += 64) L += fast_exp2(lrow[(size_t)sp * stride] - M);
        // every lane takes part in the cross-lane reads
        auto add = [&](int sp, const f32x4 &xs) {
            const float wa = __shfl(w0, sp & 63);
            const float wb = MANY ? __shfl(w1, sp & 63) : 0.f;
            if (sp < count) {
                const float w = sp < 64 ? wa
                                        : (sp < NLSE ? wb : fast_exp2(lrow[(size_t)sp * stride] - M));
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[j] = fmaf(w, xs[j], acc[j]);
            }
        };
#pragma unroll
        for (int u = 0; u < UNR; ++u) add(g + u * STEP, x[u]);
        // more partials than the first batch holds
        for (int s0 = UNR * STEP; s0 < count; s0 += UNR * STEP) {
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int sp = s0 + g + u * STEP;
                x[u] = sp < count ? orow_of(sp) : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) add(s0 + g + u * STEP, x[u]);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) L += __shfl_xor(L, m);
#pragma unroll
    for (int m = LPG; m < 64; m <<= 1)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], m);
    if constexpr (WPR > 1) {
        // the waves of the row sum their shares through LDS; wave 0 writes
        lds_acc[sub][lane] = acc;
        __syncthreads();
        if (sub != 0) return;
#pragma unroll
        for (int w = 1; w < WPR; ++w) {
            const f32x4 y = lds_acc[w][lane];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += y[j];
        }
    }

    const bool empty = !(L > 0.f);
    const float inv = empty ? 0.f : 1.f / L;
    if (lane < LPG && d0 < a.Dv) {
        uint16_t *outp = (uint16_t *)a.out + (q_token(a, b, i) * a.Hq + h) * a.Dv + d0;
        if (a.Dv % 4 == 0) {
            *(u32x2 *)outp = u32x2{pack2<DT>(acc[0] * inv, acc[1] * inv),
                                   pack2<DT>(acc[2] * inv, acc[3] * inv)};
        } else {
            // rows only 2-byte aligned: element stores, none past the head
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (d0 + j < a.Dv) outp[j] = (uint16_t)to16<DT>(acc[j] * inv);
        }
    }
    if (lane == 0 && a.lse) a.lse[lse_index(a, b, h, i)] = empty ? kNegInf : (M + fast_log2(L)) * kLn2;
}

template <int DT, int D>
hipError_t launch_t(const KernelArgs &a, hipStream_t stream) {
    KernelArgs args = a;
    void *kargs[] = {&args};
    const long long nrows = (long long)a.B * a.Hq * a.qLen;
    // partials per output row: the partitions of a fixed schedule, about
    // grid / streams (+ 1) for the balanced one
    const long long streams = (long long)a.B * a.head_blocks * a.row_blocks;
    const long long per_row = a.schedule == kFixed ? a.S : a.S / (streams > 0 ? streams : 1) + 1;
    // the balanced schedule's busy shares are at most the grid and at most
    // the largest total the lengths allow over the share floor
    long long busy = a.S;
    if (a.schedule != kFixed && a.min_share > 0) {
        const long long most = (streams * a.kv_cap + a.min_share - 1) / a.min_share;
        if (most < busy) busy = most;
    }
    const long long most_per_row = a.schedule == kFixed ? a.S : busy / (streams > 0 ? streams : 1) + 1;
    // the grid-based count also decides when few rows need more workgroups:
    // one workgroup per row above 24 partials, or above 12 when there are at
    // most 1024 rows (the Qwen3-4B-shaped batch, 512 rows of 17 partials:
    // 156.0 against 156.4 us per call; the Llama-70B MTP batch, 2048 rows of
    // 17, keeps one wave per row: 96.1 against 98.7 us; the exact count of
    // stream-aligned shares, 16 for SmallQ q8 kv1023, measured 0.5 us slower
    // than this estimate's choice of one workgroup per row there)
    const bool wide = per_row > 24 || (per_row > 12 && nrows <= 1024);
    const int rpb = wide ? 1 : kWaves;
    const unsigned blocks = (unsigned)((nrows + rpb - 1) / rpb);
    const void *fn = !wide               ? (const void *)&combine_kernel<DT, D, 1, false>
                     : most_per_row > 64 ? (const void *)&combine_kernel<DT, D, kWaves, true>
                                         : (const void *)&combine_kernel<DT, D, kWaves, false>;
    return hipLaunchKernel(fn, dim3(blocks), dim3(kWaves * 64), kargs, 0, stream);
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
