// Split-KV decode attention, vector-ALU path (gfx950).
//
// Used when a kv head carries few query rows (R = (Hq/Hkv) * qLen small), where
// Q K^T is too thin to be worth the matrix cores and the kernel is bound by
// streaming K and V from HBM.
//
// Work decomposition.  A workgroup (4 waves) owns one KV partition
// [split * chunk, (split + 1) * chunk) of one (batch b, kv head) pair for a
// block of RB query rows -- the split-KV decomposition of the MXFlashAttn
// package page (M1 split-KV decode), with the K-outer loop and resident Q of
// the SmallQ FlashAttention README (algorithm notes).  Row r of a block is
// query position i = r / G and head h = kvh * G + r % G.
//
// Lane layout.  A token's head slice (D 16-bit values) is read by LPT = D/8
// lanes, 16 contiguous bytes each (one global_load_dwordx4 per lane, fully
// coalesced); a wave therefore covers TPW = 64 / LPT tokens per load, one per
// "token slot" of LPT lanes.  Each lane loads U tokens of K and U of V per
// step and computes partial dot products over its 8 channels for its U
// tokens x RB rows (N = U * RB partials, v_dot2 with fp32 accumulation).
//
// Reduce-scatter.  The N partials are summed across the LPT lanes of the
// slot with DPP exchanges inside a 16-lane row (xor 8 = row_ror:8, xor 7 =
// half-row mirror, xor 2 / xor 1 = quad permutations).  Each halving step
// keeps the lower half of the register array; to make that valid without
// per-lane selects, lane sl's register k holds the partial for value index
// j = k ^ phi(sl), where phi is chosen so that the partner of every step holds
// the same value index in the upper half (phi = g(sl) >> (LB - H) with
// g(sl) = sl ^ (bit2(sl) ? 3 : 0)).  The lane-dependent XOR is applied for
// free when loading: lane sl keeps q row (r ^ phi_r) in its register r and
// K token (u ^ phi_u) in its register u.  After log2(N) halving steps the lane
// holds one complete score, for (token u*, row r*) = (phi_u, phi_r).
//
// Online softmax (ops-transformer articles: running max m and sum l, with
// the accumulated output rescaled by exp(m_old - m_new)).  Per token slot and
// row, in log2 units (Q K^T is scaled by log2(e)/sqrt(D) so exp2 replaces
// exp): row max over the slot's U tokens by DPP, p = exp2(s - m_new),
// alpha = exp2(m_old - m_new), l = alpha * l + sum p.  p and alpha are shared
// within the slot through a small LDS array; the rescale of O is skipped when
// no row's maximum moved anywhere in the wave.  O += p V in fp32 with V
// converted from 16 bits (the SmallQ README's fp32 PV accumulation).
//
// Epilogue.  The TPW slots of a wave and the 4 waves of the workgroup hold
// independent (m, l, O) states; they are merged with the same log-sum-exp
// rule, then written either as the final output (single partition) or as a
// normalised partial O plus its log2-sum-exp for the combine kernel.
#include "device_common.h"
#include "launch.h"

namespace mxfa {
namespace {

constexpr int kWaves = 4;

// DPP lane mask used at step t of the reduce sequence for a slot of 2^LB lanes.
constexpr int step_mask(int LB, int t) {
    return LB == 4 ? (t == 0 ? 8 : t == 1 ? 7 : t == 2 ? 2 : 1)
                   : (t == 0 ? 7 : t == 1 ? 2 : 1);
}

template <int LB, int T, int END>
struct AllReduce {
    __device__ static __forceinline__ float sum(float v) {
        if constexpr (T < END) {
            v += xor_lane<step_mask(LB, T)>(v);
            return AllReduce<LB, T + 1, END>::sum(v);
        } else {
            return v;
        }
    }
    __device__ static __forceinline__ float max(float v) {
        if constexpr (T < END) {
            v = fmaxf(v, xor_lane<step_mask(LB, T)>(v));
            return AllReduce<LB, T + 1, END>::max(v);
        } else {
            return v;
        }
    }
};

// Halving steps T .. H-1 of the reduce-scatter over N values.
template <int LB, int N, int T, int H>
struct Halve {
    __device__ static __forceinline__ void run(float (&v)[N]) {
        if constexpr (T < H) {
            constexpr int half = N >> (T + 1);
#pragma unroll
            for (int k = 0; k < half; ++k)
                v[k] += xor_lane<step_mask(LB, T)>(v[k + half]);
            Halve<LB, N, T + 1, H>::run(v);
        }
    }
};

template <int DT, int D, int RB, bool CAUSAL>
__global__ __launch_bounds__(kWaves * 64) void split_kv_valu_kernel(SplitArgs a) {
    constexpr int LPT = D / 8;                  // lanes per token
    constexpr int LB = ilog2(LPT);              // 4 (D=128) or 3 (D=64)
    constexpr int TPW = 64 / LPT;               // token slots per wave
    constexpr int U = (LPT / RB) >= 4 ? 4 : (LPT / RB);  // tokens per slot per step
    constexpr int N = U * RB;                   // partial scores per lane per step
    constexpr int H = ilog2(N);                 // halving steps
    constexpr int LOGRB = ilog2(RB);
    constexpr int LOGU = ilog2(U);
    constexpr int TPS = TPW * U;                // tokens per wave step
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(N >= 2 && N <= LPT, "reduce-scatter shape");

    __shared__ __attribute__((aligned(16))) float lds_p[kWaves][TPW][N];
    __shared__ __attribute__((aligned(16))) float lds_a[kWaves][TPW][RB];
    __shared__ __attribute__((aligned(16))) float lds_ml[kWaves][TPW][2][RB];
    __shared__ __attribute__((aligned(16))) float lds_o[kWaves][RB][D];
    __shared__ __attribute__((aligned(16))) float lds_wml[kWaves][2][RB];

    const int split = blockIdx.x;
    const int kvh = blockIdx.y % a.Hkv;
    const int rb = blockIdx.y / a.Hkv;
    const int b = blockIdx.z;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sl = lane & (LPT - 1);
    const int sg = lane >> LB;

    const int n = clampi(a.seqlens ? a.seqlens[b] : a.kv_cap, 0, a.kv_cap);
    const int t_lo = split * a.chunk;
    if (split > 0 && t_lo >= n) return;       // partition past this sequence
    int t_hi = min(t_lo + a.chunk, n);
    const int row0 = rb * RB;
    if constexpr (CAUSAL) {
        // no row of this block sees a key past (last query position) + n - qLen
        const int i_max = (min(row0 + RB, a.R) - 1) / a.G;
        t_hi = min(t_hi, i_max + n - a.qLen + 1);
    }
    const int nsteps = t_hi > t_lo ? (t_hi - t_lo + TPS - 1) / TPS : 0;

    // lane permutation of the reduce-scatter
    const int gperm = sl ^ (((sl >> 2) & 1) * 3);
    const int phi = gperm >> (LB - H);
    const int phir = phi & (RB - 1);
    const int phiu = phi >> LOGRB;

    // the score this lane finishes with belongs to row (row0 + phir)
    const int my_row = row0 + phir;
    const bool row_ok = my_row < a.R;
    const int causal_last = my_row / a.G + n - a.qLen;

    // Q rows, resident for the whole partition (16-bit, unscaled)
    u32x4 qr[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int row = row0 + (r ^ phir);
        if (row < a.R) {
            const int i = row / a.G;
            const int h = kvh * a.G + row % a.G;
            const uint16_t *qp = (const uint16_t *)a.q +
                                 (((size_t)b * a.qLen + i) * a.Hq + h) * D + 8 * sl;
            qr[r] = *(const u32x4 *)qp;
        } else {
            qr[r] = u32x4{0, 0, 0, 0};
        }
    }

    const size_t tok_stride = (size_t)a.Hkv * D;
    const size_t head_off = ((size_t)b * a.kv_cap * a.Hkv + kvh) * D + 8 * sl;
    const uint16_t *kbase = (const uint16_t *)a.k + head_off;
    const uint16_t *vbase = (const uint16_t *)a.v + head_off;

    float m_run = kNegInf, l_run = 0.f;
    float o[RB][8];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] = 0.f;

    auto load_step = [&](int st, u32x4 (&kr)[U], u32x4 (&vr)[U]) {
        const int base = t_lo + st * TPS + sg;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // tokens past the partition are masked later; clamping keeps the
            // address inside the valid part of the cache (never the tail)
            const int tk = min(base + (u ^ phiu) * TPW, n - 1);
            const int tv = min(base + u * TPW, n - 1);
            kr[u] = *(const u32x4 *)(kbase + (size_t)tk * tok_stride);
            vr[u] = *(const u32x4 *)(vbase + (size_t)tv * tok_stride);
        }
    };

    auto compute_step = [&](int st, const u32x4 (&kr)[U], const u32x4 (&vr)[U]) {
        float v[N];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                float acc = 0.f;
                acc = dot2<DT>(qr[r][0], kr[u][0], acc);
                acc = dot2<DT>(qr[r][1], kr[u][1], acc);
                acc = dot2<DT>(qr[r][2], kr[u][2], acc);
                acc = dot2<DT>(qr[r][3], kr[u][3], acc);
                v[r + RB * u] = acc;
            }
        Halve<LB, N, 0, H>::run(v);
        const float s = AllReduce<LB, H, LB>::sum(v[0]);

        const int tok = t_lo + st * TPS + phiu * TPW + sg;
        bool vis = row_ok && tok < t_hi;
        if constexpr (CAUSAL) vis = vis && tok <= causal_last;
        const float x = vis ? s * a.qscale : kNegInf;

        const float mx = AllReduce<LB, 0, LOGU>::max(x);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float p = fast_exp2(x - m_use);
        // alpha = 1 exactly when the row maximum did not move (also for rows
        // that have seen nothing yet), so the rescale below can be skipped
        const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_use);
        const float psum = AllReduce<LB, 0, LOGU>::sum(p);
        l_run = l_run * alpha + psum;
        m_run = m_new;

        wave_lds_sync();
        lds_p[wave][sg][phi] = p;
        lds_a[wave][sg][phir] = alpha;
        wave_lds_sync();
        float pc[N], ac[RB];
#pragma unroll
        for (int k = 0; k < N; ++k) pc[k] = lds_p[wave][sg][k];
        bool moved = false;
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            ac[r] = lds_a[wave][sg][r];
            moved |= ac[r] != 1.f;
        }
        if (__any(moved)) {
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int e = 0; e < 8; ++e) o[r][e] *= ac[r];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vf[8];
#pragma unroll
            for (int c = 0; c < 4; ++c) unpack2<DT>(vr[u][c], vf[2 * c], vf[2 * c + 1]);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const float pr = pc[r + RB * u];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[r][e] = fmaf(pr, vf[e], o[r][e]);
            }
        }
    };

    // K-outer loop: wave w takes steps w, w + 4, ...; loads of the next step
    // are issued before the current one is computed (register double buffer).
    {
        u32x4 kA[U], vA[U], kB[U], vB[U];
        int st = wave;
        if (st < nsteps) load_step(st, kA, vA);
        while (st < nsteps) {
            if (st + kWaves < nsteps) load_step(st + kWaves, kB, vB);
            compute_step(st, kA, vA);
            st += kWaves;
            if (st >= nsteps) break;
            if (st + kWaves < nsteps) load_step(st + kWaves, kA, vA);
            compute_step(st, kB, vB);
            st += kWaves;
        }
    }

    // ---- epilogue: merge token slots, then waves, then write ----
    wave_lds_sync();
    if (phiu == 0) {
        lds_ml[wave][sg][0][phir] = m_run;
        lds_ml[wave][sg][1][phir] = l_run;
    }
    wave_lds_sync();
    float wm[RB], wl[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        float M = kNegInf;
#pragma unroll
        for (int s2 = 0; s2 < TPW; ++s2) M = fmaxf(M, lds_ml[wave][s2][0][r]);
        float L = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < TPW; ++s2) {
            const float ms = lds_ml[wave][s2][0][r];
            L += (ms == kNegInf ? 0.f : fast_exp2(ms - M)) * lds_ml[wave][s2][1][r];
        }
        const float mine = lds_ml[wave][sg][0][r];
        const float sc = mine == kNegInf ? 0.f : fast_exp2(mine - M);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[r][e] *= sc;
        wm[r] = M;
        wl[r] = L;
    }
#pragma unroll
    for (int x = LPT; x < 64; x <<= 1)
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[r][e] += __shfl_xor(o[r][e], x);
    if (sg == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) lds_o[wave][r][8 * sl + e] = o[r][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            lds_wml[wave][0][r] = wm[r];
            lds_wml[wave][1][r] = wl[r];
        }
    }
    __syncthreads();

    constexpr int Q4 = D / 4;
    for (int idx = threadIdx.x; idx < RB * Q4; idx += kWaves * 64) {
        const int r = idx / Q4;
        const int d0 = (idx % Q4) * 4;
        const int row = row0 + r;
        if (row >= a.R) continue;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_wml[w][0][r]);
        float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float mw = lds_wml[w][0][r];
                const float sc = mw == kNegInf ? 0.f : fast_exp2(mw - M);
                den += sc * lds_wml[w][1][r];
#pragma unroll
                for (int j = 0; j < 4; ++j) num[j] += sc * lds_o[w][r][d0 + j];
            }
        }
        const bool empty = !(den > 0.f);
        const float inv = empty ? 0.f : 1.f / den;
        const float lse2 = empty ? kNegInf : M + fast_log2(den);
        const int i = row / a.G;
        const int h = kvh * a.G + row % a.G;
        const size_t orow = ((size_t)b * a.Hq + h) * a.qLen + i;   // [B, Hq, qLen]
        if (a.S == 1) {
            uint16_t *op = (uint16_t *)a.out + (((size_t)b * a.qLen + i) * a.Hq + h) * D + d0;
            *(u32x2 *)op = u32x2{pack2<DT>(num[0] * inv, num[1] * inv),
                                 pack2<DT>(num[2] * inv, num[3] * inv)};
            if (d0 == 0 && a.lse) a.lse[orow] = empty ? kNegInf : lse2 * kLn2;
        } else {
            float *wp = a.ws_o + (orow * a.S + split) * D + d0;
            *(f32x4 *)wp = f32x4{num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv};
            if (d0 == 0) a.ws_lse[orow * a.S + split] = lse2;
        }
    }
}

template <int DT, int D, int RB, bool CAUSAL>
hipError_t launch_t(const SplitArgs &a, dim3 grid, hipStream_t stream) {
    SplitArgs args = a;
    void *kargs[] = {&args};
    return hipLaunchKernel((const void *)&split_kv_valu_kernel<DT, D, RB, CAUSAL>, grid,
                           dim3(kWaves * 64), kargs, 0, stream);
}

template <int DT, int D, int RB>
hipError_t launch_c(const SplitArgs &a, int causal, dim3 grid, hipStream_t stream) {
    return causal ? launch_t<DT, D, RB, true>(a, grid, stream)
                  : launch_t<DT, D, RB, false>(a, grid, stream);
}

template <int DT, int D>
hipError_t launch_rb(const SplitArgs &a, int rb, int causal, dim3 grid, hipStream_t stream) {
    switch (rb) {
    case 1: return launch_c<DT, D, 1>(a, causal, grid, stream);
    case 2: return launch_c<DT, D, 2>(a, causal, grid, stream);
    case 4: return launch_c<DT, D, 4>(a, causal, grid, stream);
    case 8: return launch_c<DT, D, 8>(a, causal, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_split_valu(const SplitArgs &a, int dtype, int D, int row_block,
                             int causal, dim3 grid, hipStream_t stream) {
    if (dtype == kFp16) {
        if (D == 128) return launch_rb<kFp16, 128>(a, row_block, causal, grid, stream);
        if (D == 64) return launch_rb<kFp16, 64>(a, row_block, causal, grid, stream);
    } else {
        if (D == 128) return launch_rb<kBf16, 128>(a, row_block, causal, grid, stream);
        if (D == 64) return launch_rb<kBf16, 64>(a, row_block, causal, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mxfa
