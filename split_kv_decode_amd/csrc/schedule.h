// Work schedules shared by the split kernels (device code).
//
// A "stream" is the KV token range [0, n_b) of one (sequence b, head block,
// row block); see launch.h.  drive_schedule hands a kernel's workgroup its
// segments, each as (b, n_b, head block, row block, t_lo, t_hi, slot, whole):
//   kFixed:    grid (S, head_blocks * row_blocks, B); one segment
//              [split * chunk, (split + 1) * chunk) per workgroup, slot
//              st * S + split (with several row blocks, see xcd_heads).
//   kBalanced: grid (P); the streams are laid end to end and workgroup w
//              (in XCD order, see xcd_order) takes [w * W, (w + 1) * W) of
//              the concatenation, W = max(
//              ceil(total / P), min_share), as one segment per stream it
//              touches, slot w + st.  Without per-sequence lengths the
//              host fixes W (uni_w) and may give every stream shares of its
//              own (uni_spw per stream; see uniform_shares in api.hip).
// `whole` marks a segment that is its stream's entire range; the kernel then
// writes the final output instead of a partial.  With ALIGN > 1 every bound
// inside a stream is rounded down to a multiple of ALIGN (the stream's end
// stays n): neighbouring segments round their shared bound alike, so they
// still cover [0, n) once, and a segment that rounds to nothing is still
// handed over (its workgroup writes an empty partial to its slot, which the
// merge kernel counts).  `whole` is decided on the bounds before rounding.  The valid lengths live on
// the device, so in the balanced schedule every workgroup first forms their
// prefix sums (workgroup 0 also stores them, and W, for the merge kernel).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace mxfa {

constexpr int kScheduleThreads = 256;

// Workgroup-uniform values read from LDS are otherwise held in vector
// registers; readfirstlane moves them to scalar registers.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ long long uni(long long x) {
    const int lo = __builtin_amdgcn_readfirstlane((int)(x & 0xffffffff));
    const int hi = __builtin_amdgcn_readfirstlane((int)(x >> 32));
    return ((long long)hi << 32) | (unsigned)lo;
}

__device__ __forceinline__ const void *uni_ptr(const void *p) {
    return (const void *)uni((long long)(uintptr_t)p);
}

// Workgroups of a launch are handed to the GPU's 8 XCDs in turn (workgroup
// i to XCD i % 8).  Share of workgroup i in a grid of n when shares
// 0 .. nb - 1 hold all the work: XCD x takes shares floor(x nb / 8) ..
// floor((x + 1) nb / 8) - 1, so the XCDs get equal work (within one share)
// and one XCD's shares are consecutive; the partial results of a stream are
// then written by
// workgroups of one XCD, and the merge kernel (which orders its rows the same
// way) reads each row's partials from the XCD that wrote them.  Workgroups
// past those shares get share nb, which holds no work.  On the
// Llama-70B-shaped MTP batch this takes the merge kernel from 6.3 to 5.0 us.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_share(int i, int n, int nb) {
    if (n % kXcds != 0) return i;
    const int x = i % kXcds, k = i / kXcds;
    const int lo = (int)((long long)x * nb / kXcds);
    const int hi = (int)((long long)(x + 1) * nb / kXcds);
    return k < hi - lo ? lo + k : nb;
}
__device__ __forceinline__ int xcd_order(int i, int n) { return xcd_share(i, n, n); }

// x / d and x % d for 0 <= x, 0 < d, in 32-bit arithmetic when both fit
// (the usual case; the 64-bit division costs several times as much)
__device__ __forceinline__ long long div_nn(long long x, long long d) {
    return (x <= 0x7fffffffLL && d <= 0x7fffffffLL) ? (long long)((uint32_t)x / (uint32_t)d)
                                                      : x / d;
}

// Exclusive prefix sums of the clamped sequence lengths into cum[0..B]
// (cum[B] = total), computed by the whole workgroup of 256 threads.
__device__ __forceinline__ void length_prefix_sums(const KernelArgs &a, long long *cum,
                                          long long *wave_tot) {
    constexpr int PER = (kMaxBalancedBatch + kScheduleThreads - 1) / kScheduleThreads;
    const int t = threadIdx.x;
    const int lane = t & 63, wave = t >> 6;
    // every load is issued before any is used (one memory round trip); the
    // descriptor ends with the array, so entries past it read 0
    const int *src = a.cu_k ? a.cu_k : a.seqlens;
    const uint32_t bytes = src ? (uint32_t)(a.cu_k ? a.B + 1 : a.B) * 4u : 0u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(uni_ptr(src), (uint32_t)uni((int)bytes));
    int x0[PER], x1[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const uint32_t bb = (uint32_t)(t * PER + j);
        x0[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(r, bb * 4u, 0, 0);
        x1[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(r, bb * 4u + 4u, 0, 0);
    }
    long long v[PER];
    long long mine = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int bb = t * PER + j;
        v[j] = bb < a.B ? seq_len_from(a, x0[j], x1[j]) : 0;
        mine += v[j];
    }
    // inclusive scan of `mine` across the wave
    long long inc = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const long long y = __shfl_up(inc, d);
        if (lane >= d) inc += y;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    long long before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    long long run = before + inc - mine;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int bb = t * PER + j;
        if (bb < a.B) cum[bb] = run;
        run += v[j];
    }
    if (t == kScheduleThreads - 1) cum[a.B] = run;     // the total (entries past B are 0)
    __syncthreads();
}

// Tokens per workgroup share of the balanced schedule when the streams hold
// T tokens in all (every workgroup and the merge kernel derive it alike).
__device__ __forceinline__ long long balanced_share(const KernelArgs &a, long long T) {
    const long long W = div_nn(T + a.S - 1, a.S);
    return W < a.min_share ? (long long)a.min_share : W;
}

template <int SCHED, int ALIGN = 1, class Segment>
__device__ __forceinline__ void drive_schedule(const KernelArgs &a, Segment &&segment) {
    const int HR = a.head_blocks * a.row_blocks;
    auto bound = [](int t, int n) { return t >= n ? n : (t & ~(ALIGN - 1)); };
    if constexpr (SCHED == kFixed) {
        int split = blockIdx.x;
        int y = blockIdx.y;
        int b = blockIdx.z;
        if (a.xcd_heads) {
            // Workgroup L (in launch order) runs on XCD L % 8.  Numbered head
            // block fastest, XCD x takes the head blocks congruent to x
            // modulo 8 (with 8 head blocks, one each), so the row blocks
            // that re-read a kv head's K/V share one XCD's L2 instead of
            // all eight fetching it: 5.4 times fewer bytes fetched past the
            // L2s on the Llama-70B-shaped chunked prefill (0.35 against 1.89
            // GiB per launch, at the same speed).  Every head carries the
            // same work, so the XCDs stay equally loaded.  The numbering is a
            // bijection of the grid, so results do not depend on where the
            // workgroups run; only the cache sharing does.
            const long long L = blockIdx.x + (long long)gridDim.x *
                                                  (blockIdx.y + (long long)gridDim.y * blockIdx.z);
            const int hb = (int)(L % a.head_blocks);
            const long long r = L / a.head_blocks;   // (split, row block, sequence), split fastest
            split = (int)(r % gridDim.x);
            const long long r2 = r / gridDim.x;
            b = (int)(r2 / a.row_blocks);
            y = hb * a.row_blocks + (int)(r2 % a.row_blocks);
        }
        const int n = seq_len(a, b);
        const int t_lo = split * a.chunk;
        if (split > 0 && t_lo >= n) return;   // partition past this sequence
        const int t_hi = min(t_lo + a.chunk, n);
        const int slot = (b * HR + y) * a.S + split;
        segment(b, n, y / a.row_blocks, y % a.row_blocks, bound(t_lo, n), bound(t_hi, n), slot,
                t_lo == 0 && t_hi == n);
    } else {
        __shared__ long long cum[kMaxBalancedBatch + 1];
        __shared__ long long wave_tot[kScheduleThreads / 64];
        // Without per-sequence lengths every sequence holds the same number
        // of keys, so the prefix sums are b * n and no workgroup waits for
        // the length loads and the scan before requesting its first tile.
        const bool uniform = a.seqlens == nullptr && a.cu_k == nullptr;
        const long long n_u = uniform ? seq_len_from(a, 0, 0) : 0;
        if (!uniform) length_prefix_sums(a, cum, wave_tot);
        // L: the stride of one stream in the concatenation.  With lengths of
        // one value the host has chosen the share width (uni_w) and, when
        // every stream gets shares of its own (uni_spw > 0), each stream is
        // padded to whole shares (L = uni_spw * W); segments end at the
        // stream's real length
        const long long L = uniform && a.uni_spw > 0 ? (long long)a.uni_spw * a.uni_w : n_u;
        auto cumv = [&](int bb) -> long long { return uniform ? bb * L : cum[bb]; };
        const long long T = uni(cumv(a.B) * HR);
        const long long W = uni(uniform ? (long long)a.uni_w : balanced_share(a, T));
        if (blockIdx.x == 0) {
            for (int bb = threadIdx.x; bb <= a.B; bb += kScheduleThreads)
                ((long long *)a.ws_cum)[bb] = cumv(bb);
            if (threadIdx.x == 0) ((long long *)a.ws_cum)[a.B + 1] = W;
        }
        // shares with work: fewer than the grid when W is held up by min_share
        const long long nbw = div_nn(T + W - 1, W);
        const int nb = (int)(nbw < a.S ? nbw : a.S);
        const int w = xcd_share(blockIdx.x, gridDim.x, nb);
        long long g = (long long)w * W;
        if (g >= T) return;
        const long long gend = g + W < T ? g + W : T;
        // sequence holding global token g: the last b with cum[b] * HR <= g
        // (g < T, so with uniform lengths L > 0)
        int lo = 0, hi = a.B - 1;
        if (uniform) {
            lo = (int)div_nn(g, L * HR);
        } else {
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (cum[mid] * HR <= g) lo = mid; else hi = mid - 1;
            }
        }
        int b = uni(lo);
        int n = uni((int)(cumv(b + 1) - cumv(b)));      // stride of b's streams
        const int nr = uniform ? (int)n_u : 0;           // real length (uniform)
        const long long off = uni(g - cumv(b) * HR);
        int j = uni((int)div_nn(off, n));
        int t = uni((int)(off - (long long)j * n));
        while (g < gend) {
            const int seg = (int)((long long)(n - t) < gend - g ? (long long)(n - t) : gend - g);
            const int len = uniform ? nr : n;
            const int e = t + seg < len ? t + seg : len;
            segment(b, len, j / a.row_blocks, j % a.row_blocks, bound(t, len), bound(e, len),
                    (int)(w + b * HR + j), t == 0 && e == len);
            g += seg;
            t = 0;
            if (++j == HR) {
                j = 0;
                do { ++b; } while (b < a.B && cumv(b + 1) == cumv(b));
                b = uni(b);
                if (b >= a.B) break;
                n = uni((int)(cumv(b + 1) - cumv(b)));
            }
        }
    }
}

}  // namespace mxfa
