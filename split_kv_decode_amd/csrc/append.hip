// In-call KV append: the new keys and values of this step are written into
// the cache before attention reads it.
//
// The MXFlashAttn package page names a FlashAttention-compatible entry point
// for attention with a KV cache (Python API section), and its sdist README
// lists paged KV append among the verified capabilities (capability matrix);
// neither gives the rule, so the FlashAttention one is taken: token t of
// k_new / v_new [B, new_len, Hkv, D] goes to cache position
// cache_seqlens[b] + t of sequence b (contiguous row, or row pos % page of
// page block_table[b][pos / page]), and attention then sees
// cache_seqlens[b] + new_len keys.  Positions at or past kv_cap are dropped.
//
// A plain copy: one thread moves 16 bytes of K and 16 bytes of V, or, for
// head dims that are not multiples of 8 (rows only 2-byte aligned), one
// element of K and one of V.
#include "device_common.h"
#include "launch.h"

namespace mxfa {
namespace {

constexpr int kAppendThreads = 256;

template <bool PAGED, bool ELEM>
__global__ __launch_bounds__(kAppendThreads)
void kv_append_kernel(KernelArgs a, const uint16_t *__restrict__ k_new,
                      const uint16_t *__restrict__ v_new) {
    const int b = blockIdx.y;
    // pieces of a K / V head row a thread moves: 16-byte chunks, or elements
    const int nck = ELEM ? a.Dk : a.Dk / 8, ncv = ELEM ? a.Dv : a.Dv / 8;
    const int nch = nck > ncv ? nck : ncv;
    const long long idx = (long long)blockIdx.x * kAppendThreads + threadIdx.x;
    if (idx >= (long long)a.new_len * a.Hkv * nch) return;
    const int c = (int)(idx % nch);
    const int h = (int)((idx / nch) % a.Hkv);
    const int t = (int)(idx / ((long long)nch * a.Hkv));
    const int n0 = clampi(a.seqlens[b], 0, a.kv_cap);
    if (t >= a.kv_cap - n0) return;                 // past the capacity: dropped
    const int pos = n0 + t;
    size_t row;                                     // token row index in the cache
    if constexpr (PAGED) {
        const int pg = clampi(a.block_table[(size_t)b * a.max_pages + (pos >> a.log_page)], 0,
                              a.num_pages - 1);
        row = ((size_t)pg << a.log_page) + (pos & ((1 << a.log_page) - 1));
    } else {
        row = (size_t)b * a.kv_cap + pos;
    }
    const size_t tok = (size_t)b * a.new_len + t;
    if constexpr (ELEM) {
        if (c < nck)
            ((uint16_t *)a.k)[(row * a.Hkv + h) * a.Dk + c] = k_new[(tok * a.Hkv + h) * a.Dk + c];
        if (c < ncv)
            ((uint16_t *)a.v)[(row * a.Hkv + h) * a.Dv + c] = v_new[(tok * a.Hkv + h) * a.Dv + c];
        return;
    }
    if (c < nck)
        *(u32x4 *)((uint16_t *)a.k + (row * a.Hkv + h) * a.Dk + 8 * c) =
            *(const u32x4 *)(k_new + (tok * a.Hkv + h) * a.Dk + 8 * c);
    if (c < ncv)
        *(u32x4 *)((uint16_t *)a.v + (row * a.Hkv + h) * a.Dv + 8 * c) =
            *(const u32x4 *)(v_new + (tok * a.Hkv + h) * a.Dv + 8 * c);
}

}  // namespace

hipError_t launch_append(const KernelArgs &a, const void *k_new, const void *v_new,
                         hipStream_t stream) {
    const bool elem = odd_head_dims(a.Dk, a.Dv);
    const long long per_seq =
        (long long)a.new_len * a.Hkv * ((a.Dk > a.Dv ? a.Dk : a.Dv) / (elem ? 1 : 8));
    if (per_seq == 0 || a.B == 0 || a.kv_cap == 0) return hipSuccess;
    const long long blocks = (per_seq + kAppendThreads - 1) / kAppendThreads;
    if (blocks > INT32_MAX) return hipErrorInvalidValue;
    KernelArgs args = a;
    const uint16_t *kn = (const uint16_t *)k_new;
    const uint16_t *vn = (const uint16_t *)v_new;
    void *kargs[] = {&args, &kn, &vn};
    const void *fn = a.block_table ? (elem ? (const void *)&kv_append_kernel<true, true>
                                           : (const void *)&kv_append_kernel<true, false>)
                                   : (elem ? (const void *)&kv_append_kernel<false, true>
                                           : (const void *)&kv_append_kernel<false, false>);
    return hipLaunchKernel(fn, dim3((unsigned)blocks, a.B), dim3(kAppendThreads), kargs, 0,
                           stream);
}

}  // namespace mxfa
