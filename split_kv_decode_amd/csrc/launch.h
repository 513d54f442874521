// Internal interface between the host planner (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfa {

// Everything a split kernel needs; pointers are device addresses.
struct SplitArgs {
    const void *q;            // [B, qLen, Hq, D]
    const void *k;            // [B, kv_cap, Hkv, D]
    const void *v;            // [B, kv_cap, Hkv, D]
    const int32_t *seqlens;   // [B] or nullptr
    void *out;                // [B, qLen, Hq, D]   (written when S == 1)
    float *lse;               // [B, Hq, qLen] or nullptr (written when S == 1)
    float *ws_o;              // [B, Hq, qLen, S, D] normalised partial outputs
    float *ws_lse;            // [B, Hq, qLen, S]    partial lse, log2 units
    int B, Hq, Hkv, qLen, kv_cap;
    int G;                    // Hq / Hkv
    int R;                    // G * qLen rows per kv head
    int chunk;                // tokens per partition
    int S;                    // partitions per (b, kv head) at kv_cap
    float qscale;             // log2(e) / sqrt(D)
};

struct CombineArgs {
    const float *ws_o;
    const float *ws_lse;
    const int32_t *seqlens;
    void *out;
    float *lse;
    int B, Hq, qLen, kv_cap, chunk, S;
};

hipError_t launch_split_valu(const SplitArgs &a, int dtype, int D, int row_block,
                             int causal, dim3 grid, hipStream_t stream);

hipError_t launch_combine(const CombineArgs &a, int dtype, int D,
                          hipStream_t stream);

}  // namespace mxfa
