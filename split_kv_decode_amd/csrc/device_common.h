// Device-side helpers shared by the gfx950 split-KV kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxfa {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kFp16 = 0;
constexpr int kBf16 = 1;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// fp32 dot product of two packed pairs of 16-bit values, added to c.
// Products of two 16-bit floats are exact in fp32; the sum is rounded once
// per instruction (v_dot2_f32_f16 / v_dot2_f32_bf16).
template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (DT == kFp16)
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a),
                                      __builtin_bit_cast(f16x2, b), c, false);
    else
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                               __builtin_bit_cast(bf16x2, b), c,
                                               false);
}

// Two 16-bit values packed in a dword -> two exact fp32 values.
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t x, float &lo, float &hi) {
    if constexpr (DT == kFp16) {
        const f16x2 h = __builtin_bit_cast(f16x2, x);
        lo = (float)h[0];
        hi = (float)h[1];
    } else {
        lo = __uint_as_float(x << 16);
        hi = __uint_as_float(x & 0xffff0000u);
    }
}

// fp32 -> storage dtype, round to nearest even; returns the bit pattern.
template <int DT>
__device__ __forceinline__ uint32_t to16(float x) {
    if constexpr (DT == kFp16)
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
    else
        return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return to16<DT>(lo) | (to16<DT>(hi) << 16);
}

// Value of `v` held by lane (lane ^ MASK) inside the same 16-lane row, via
// DPP: masks 1 and 2 are quad permutations, 7 is the half-row mirror (lane
// i <-> 7 - i inside each group of 8), 8 is a rotation by 8 in the row and
// 15 the full row mirror.
template <int MASK>
__device__ __forceinline__ float xor_lane(float v) {
    static_assert(MASK == 1 || MASK == 2 || MASK == 7 || MASK == 8 || MASK == 15,
                  "no single DPP control for this lane mask");
    constexpr int ctrl = MASK == 1 ? 0xB1 :      // quad_perm [1,0,3,2]
                         MASK == 2 ? 0x4E :      // quad_perm [2,3,0,1]
                         MASK == 7 ? 0x141 :     // row_half_mirror
                         MASK == 8 ? 0x128 :     // row_ror:8
                                     0x140;      // row_mirror
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xF, 0xF, false));
}

// exp2 / log2 on the hardware transcendental unit (v_exp_f32 / v_log_f32).
// exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
    return x < lo ? lo : (x > hi ? hi : x);
}

// Raw buffer descriptor over `bytes` bytes from `base` (stride 0, so the
// hardware range check applies to the per-lane byte offset: loads at or past
// `bytes` return zero and do not access memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// Cache policy of the streaming K/V loads: non-temporal (the nt bit, 2).
// Every K/V byte is read once per call, so the loads are marked as streaming
// rather than left to compete for L2 and the memory-attached last-level
// cache; on long caches this lifts the read rate by about a tenth.
#ifndef MXFA_KV_LOAD_POLICY
#define MXFA_KV_LOAD_POLICY 2
#endif

// 16-byte load through a buffer descriptor (buffer_load_dwordx4), with the
// streaming policy above or, for K/V that other workgroups read again soon
// (several row blocks of one kv head), the default one (POL = 0).
template <int POL = MXFA_KV_LOAD_POLICY>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, POL);
}

// Orders this wave's LDS accesses around a point where lanes exchange data
// through LDS without a workgroup barrier.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace mxfa
