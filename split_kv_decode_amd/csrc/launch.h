// Internal interface between the host planner (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfa {

// How the VALU split kernel maps the 16-lane slots of a wave to kv heads:
// every slot a different head, with 2 or 1 head groups per workgroup
// (2 * TPW or TPW heads per workgroup, TPW = 64 / (D / 8) slots per wave), or
// one head per workgroup with the slots on different tokens.
enum ValuLayout { kHeadsX2 = 0, kHeadsX1 = 1, kTokens = 2 };

// How KV tokens are handed to workgroups.
//   kFixed:    grid (S, head_blocks * row_blocks, B); workgroup (s, y, b) takes
//              tokens [s * chunk, (s + 1) * chunk) of its stream.
//   kBalanced: grid (P); the streams are laid end to end and workgroup w takes
//              an equal share [w * W, (w + 1) * W) of the concatenation, which
//              may span several streams (W from the device-side lengths).
enum Schedule { kFixed = 0, kBalanced = 1 };

// A "stream" is the KV token sequence of one (sequence b, head block hb, row
// block rb); stream index st = (b * head_blocks + hb) * row_blocks + rb.
//
// Partial results live in slots.  A slot holds, for the head_block heads x
// row_block rows of one stream, the normalised output [hpb][rb][D] (fp32) and
// the log2-sum-exp [hpb][rb].  Slots of stream st:
//   kFixed:    st * S + s for the partitions s < ceil(n_b / chunk);
//   kBalanced: w + st for the workgroups w that touch the stream (these never
//              collide: a later workgroup only reaches later streams).
// A workgroup that covers a whole stream writes the final output instead.
struct KernelArgs {
    const void *q;            // [B, qLen, Hq, D]
    const void *k;            // [B, kv_cap, Hkv, D], or pages [num_pages, page, Hkv, D]
    const void *v;            // same layout as k
    const int32_t *seqlens;   // [B] or nullptr
    // Paged cache: token j of sequence b is row j % page of page
    // block_table[b * max_pages + j / page]; nullptr for a contiguous cache.
    // kv_cap is then max_pages * page.
    const int32_t *block_table;
    int max_pages, num_pages;
    int log_page;             // log2(page), page a power of two >= kMinPage
    int new_len;              // tokens appended to every sequence by this call
    // Packed (varlen) batches: sequence b's queries are rows cu_q[b] ..
    // cu_q[b + 1] - 1 of q / out [total_q, Hq, D] (lse [Hq, total_q]) and its
    // keys rows cu_k[b] .. cu_k[b + 1] - 1 of k / v [total_k, Hkv, D]; qLen
    // and kv_cap are then the largest lengths.  nullptr: padded layouts.
    const int32_t *cu_q;
    const int32_t *cu_k;
    int total_q, total_k;
    void *out;                // [B, qLen, Hq, D]
    float *lse;               // [B, Hq, qLen] or nullptr
    float *ws_o;              // [slots][head_block][row_block][D]
    float *ws_lse;            // [slots][head_block][row_block]
    int *ws_cum;              // kBalanced: [B + 1] length prefix sums, then W
    int B, Hq, Hkv, qLen, kv_cap;
    int G;                    // Hq / Hkv
    int R;                    // G * qLen rows per kv head
    int D;                    // VALU kernel: head dim (= Dk = Dv)
    int Dk, Dv;               // head dims of q / k and of v / out (1 .. 256)
    int dv_tile;              // channels per row of ws_o (Dv rounded up to the kernel tile)
    int causal;
    int head_block, head_blocks;
    int row_block, row_blocks;
    int schedule;             // Schedule
    int chunk;                // kFixed: tokens per partition
    int S;                    // kFixed: partitions per stream; kBalanced: workgroups P
    int min_share;            // kBalanced: lower bound on tokens per workgroup
    // kBalanced with sequences of one length (no seqlens, no cu_k), set on
    // the host: tokens per workgroup share, and shares per stream when each
    // stream gets shares of its own (0: the streams are concatenated)
    int uni_w, uni_spw;
    // kFixed with several row blocks per kv head: 1 when the workgroups are
    // numbered head block fastest (see drive_schedule), else 0
    int xcd_heads;
    float qscale;             // log2(e) / sqrt(D)
};

// Smallest page of a paged cache: a load step of the VALU kernel (at most 16
// tokens) and a load of the matrix-core kernel (4 or 8 consecutive tokens)
// then never span two pages.
constexpr int kMinPage = 16;

// Largest batch the balanced schedule handles (its length prefix sums are
// kept in LDS by every workgroup).
constexpr int kMaxBalancedBatch = 1024;

__device__ __forceinline__ int clamp_to(int x, int lo, int hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

// Valid length of sequence b for this call: cache_seqlens[b] (kv_cap without
// them) clamped to [0, kv_cap], plus the tokens appended in the call, at most
// kv_cap; packed keys: cu_k[b + 1] - cu_k[b], offsets clamped into
// [0, total_k] and the length to kv_cap.
// seq_len_from applies that rule to values already loaded: x0 = cu_k[b] and
// x1 = cu_k[b + 1] for packed keys, x0 = cache_seqlens[b] otherwise (x1 unused).
__device__ __forceinline__ int seq_len_from(const KernelArgs &a, int x0, int x1) {
    if (a.cu_k) {
        const int lo = clamp_to(x0, 0, a.total_k);
        const int hi = clamp_to(x1, lo, a.total_k);
        return hi - lo < a.kv_cap ? hi - lo : a.kv_cap;
    }
    const int n = clamp_to(a.seqlens ? x0 : a.kv_cap, 0, a.kv_cap);
    return a.new_len > a.kv_cap - n ? a.kv_cap : n + a.new_len;
}
__device__ __forceinline__ int seq_len(const KernelArgs &a, int b) {
    if (a.cu_k) return seq_len_from(a, a.cu_k[b], a.cu_k[b + 1]);
    return seq_len_from(a, a.seqlens ? a.seqlens[b] : 0, 0);
}

// First key row of sequence b in k / v (token rows of Hkv * D values).
__device__ __forceinline__ size_t kv_token0(const KernelArgs &a, int b) {
    return a.cu_k ? (size_t)clamp_to(a.cu_k[b], 0, a.total_k) : (size_t)b * a.kv_cap;
}

// Query rows of sequence b (qLen, or its packed count, at most qLen).
__device__ __forceinline__ int q_count(const KernelArgs &a, int b) {
    if (!a.cu_q) return a.qLen;
    const int lo = clamp_to(a.cu_q[b], 0, a.total_q);
    const int hi = clamp_to(a.cu_q[b + 1], lo, a.total_q);
    return hi - lo < a.qLen ? hi - lo : a.qLen;
}

// Token row of query i of sequence b in q / out, and the lse entry of (b, h, i).
__device__ __forceinline__ size_t q_token(const KernelArgs &a, int b, int i) {
    return a.cu_q ? (size_t)clamp_to(a.cu_q[b], 0, a.total_q) + i : (size_t)b * a.qLen + i;
}
__device__ __forceinline__ size_t lse_index(const KernelArgs &a, int b, int h, int i) {
    return a.cu_q ? (size_t)h * a.total_q + q_token(a, b, i)
                  : ((size_t)b * a.Hq + h) * a.qLen + i;
}

hipError_t launch_split_valu(const KernelArgs &a, int dtype, int layout, dim3 grid,
                             hipStream_t stream);

// Matrix-core split kernel tile widths: the head dims (Dk, Dv), 1 to 256,
// are padded to (64, 64), (128, 128), (192, 128) or (256, 256).
// 16-row tiles per wave: four up to 128 x 128, two at 192 x 128, one at
// 256 x 256 (the accumulators, Q and the K / V staging must fit one wave's
// registers); two LDS stages per wave up to 128 x 128, else one.
inline __host__ __device__ void mfma_tile_dims(int dk, int dv, int *tk, int *tv) {
    if (dk <= 64 && dv <= 64) {
        *tk = 64, *tv = 64;
    } else if (dk <= 128 && dv <= 128) {
        *tk = 128, *tv = 128;
    } else if (dk <= 192 && dv <= 128) {
        *tk = 192, *tv = 128;
    } else {
        *tk = 256, *tv = 256;
    }
}
template <int DK, int DV>
struct MfmaShape {
    static constexpr int RT = (DK + DV <= 256) ? 4 : (DK + DV <= 320 ? 2 : 1);
    static constexpr int kStages = (DK + DV <= 256) ? 2 : 1;
};
inline __host__ __device__ int mfma_row_block(int dk, int dv) {
    int tk, tv;
    mfma_tile_dims(dk, dv, &tk, &tv);
    return (tk + tv <= 256 ? 4 : (tk + tv <= 320 ? 2 : 1)) * 16;
}

// Matrix-core split kernel: row_block = mfma_row_block(Dk, Dv), head_block 1
// or 2 (dividing Hkv).
hipError_t launch_split_mfma(const KernelArgs &a, int dtype, dim3 grid, hipStream_t stream);
hipError_t launch_split_mfma_wide(const KernelArgs &a, int dtype, dim3 grid,
                                  hipStream_t stream);
// Head dims that are not multiples of 8 (rows only 2-byte aligned): the
// matrix-core kernel's 16-row tiles with element loads and stores, one kv
// head per workgroup (row_block = kMfmaSmallRows, head_block = 1).
inline __host__ __device__ bool odd_head_dims(int dk, int dv) { return (dk % 8) || (dv % 8); }
hipError_t launch_split_mfma_odd(const KernelArgs &a, int dtype, dim3 grid, hipStream_t stream);

hipError_t launch_combine(const KernelArgs &a, int dtype, hipStream_t stream);

// Writes k_new / v_new [B, new_len, Hkv, D] into the cache (contiguous or
// paged, as described by a) at positions cache_seqlens[b] + t below kv_cap.
hipError_t launch_append(const KernelArgs &a, const void *k_new, const void *v_new,
                         hipStream_t stream);

// Query rows per kv head from which the matrix-core path is used (head dims
// 64 or 128, Dk = Dv; every other head shape always takes it): 4 at head dim
// 128, 8 at 64.  Measured with the 16-row variant below against the VALU
// kernel: at 4 rows and head dim 128 the Qwen3-8B batch 347-348 against
// 351 us per call, the Qwen3-4B long batch 160.3 against 163.2, the SmallQ
// q4 case 19.8 against 21.8; at head dim 64 (4 rows) the VALU kernel stays
// ahead (189 against 199 us), and at 1-2 rows the two trade places by case.
constexpr int kMfmaMinRows = 8;
constexpr int kMfmaMinRows128 = 4;
// ... except at exactly 4 rows (head dim 128) when contiguous caches hold at
// least this many bytes (B * kv_cap * Hkv * (Dk + Dv) * 2): after the VALU kernel
// moved to one workgroup per CU it streamed such batches faster than the
// 16-row variant, which ramps up faster on small ones.  Measured per call
// (GQA 4, head dim 128, 8192 keys): 67 MB 18.4 (matrix core) against 21.8 us
// (VALU), 134 MB 29.3 against 30.3, 268 MB 51.3 against 49.3, 537 MB 88.3
// against 86.7; Qwen3-8B 345.5 against 340.7, Qwen3-4B long 159.7 against
// 158.8.  The same holds through pages once the VALU kernel requests each
// step's block-table entry a step ahead: over 16-256 token pages the Qwen3-8B
// batch reached 84.5-84.7% of HBM peak against 80.5-80.9% on the matrix-core
// kernel, the Qwen3-4B long batch 79.7-80.0% against 76.2-77.3%.
// Below the same size the VALU kernel's workgroups take half a token row's
// heads (valu_layout in api.hip).
constexpr unsigned long long kValuStreamBytes = 256ull << 20;
// At most 16 rows per kv head (e.g. GQA 8 with one query token): the
// matrix-core kernel's small variant, one 16-row tile per wave and two
// workgroups per CU (tile widths up to 128 x 128).
#ifndef MXFA_MFMA_SMALL
#define MXFA_MFMA_SMALL 1
#endif
constexpr int kMfmaSmallRows = 16;
// 17 to 48 rows per kv head (GQA 8 with 3-6 token drafts, GQA 16 with 2-3):
// blocks of 32 or 48 rows, two or three 16-row tiles per wave, one
// workgroup per CU, where the 64-row tile would compute padded rows.
// Measured against the 64-row tile on batches that keep every CU busy
// (bf16, causal, whole calls): at 32 rows 4 x 32768 keys 92.7 -> 90.7 us,
// 1 x 32768 34.8 -> 32.8, 16 x 8192 95.3 -> 93.4, 8 x 16384 (16 query heads
// x 2 tokens) 92.4 -> 90.5; at 24 rows 91.7 -> 90.1; at 48 rows 4 x 32768
// 93.6 -> 92.7, 1 x 32768 36.0 -> 35.3, 8 x 16384 94.0 -> 93.0, head dim 64
// 55.5 -> 54.6; at 40 rows 16 x 8192 96.5 -> 95.5.  (Two 32-row workgroups
// per CU spilled at the 256-register limit and ran 9% slower.)
constexpr int kMfmaMaxMidRows = 48;
// kv heads per workgroup of the matrix-core kernel (1 or 2).  Measured on the
// Llama-70B-shaped MTP batch (537 MB of K/V): 2 heads take the split kernel
// from 97.6 to 93.5 us and the whole call from 101.6 to 100.0 us (the merge
// kernel reads twice the partials).
#ifndef MXFA_MFMA_HEADS
#define MXFA_MFMA_HEADS 2
#endif
constexpr int kMfmaHeads = MXFA_MFMA_HEADS;

}  // namespace mxfa
