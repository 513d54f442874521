// Split-KV decode attention, matrix-core path (gfx950 MFMA).
//
// Used when a kv head carries many query rows (R = (Hq/Hkv) * qLen >= 32, e.g.
// GQA groups times a multi-token draft): Q K^T and P V are then dense
// contractions with 16-row tiles, which is how the ops-transformer articles
// place FlashAttention on a matrix unit (Q K^T and P V on the cube unit,
// softmax and scaling on the vector unit).  fp32 accumulation throughout.
//
// Work decomposition.  A workgroup of 4 waves serves a segment of one stream
// (sequence b, kv head, block of 64 query rows; schedules in schedule.h).
// Wave w owns the 16 rows [16 w, 16 w + 16) of the block and sees every key
// of the segment, so no cross-wave merge is needed.  K and V tiles of 64 keys
// are loaded cooperatively (16-byte loads, 16 lanes per cache row of a head),
// double-buffered in LDS.
//
// Per tile, with v_mfma_f32_16x16x32 (lane l = 16 g + p; A: row p, k-slice
// 8g..8g+7; B: k-slice 8g..8g+7, column p; C: rows 4g..4g+3, column p):
//   S^T = K Q^T: A = 16 keys x 32 channels of K (one 16-byte LDS read per
//   lane), B = Q^T (the lane's query row p, resident in registers).  Lane
//   (g, p) receives the scores of keys 4g..4g+3 of each 16-key block for
//   query row p, so every lane owns exactly one query row: its running max m,
//   running sum l and the rescale alpha are per lane (online softmax of the
//   ops-transformer articles), the row max / sum across the 4 lane groups
//   take two permlane swaps.
//   O^T += V^T P^T over 32 keys: B = P^T is the lane's own probabilities
//   (rounded to the input type) for keys {4g..4g+3} and {16+4g..16+4g+3} --
//   the MFMA k-slice of lane group g is taken to mean exactly these keys --
//   and A = V^T holds the same keys for 16 channels, read from the V tile
//   with two transposed LDS reads (ds_read_b64_tr_b16: within a 16-lane group,
//   lane 4i + c reads 4 channels of key i and lane p receives channel p of
//   the 4 keys).
// K and V rows are stored in LDS with their 16-byte chunks XOR-swizzled by
// the key index, so the 16 keys read by one MFMA operand hit distinct banks.
#include "device_common.h"
#include "launch.h"
#include "schedule.h"

namespace mxfa {
namespace {

constexpr int kMWaves = 4;
constexpr int kTile = 64;                         // keys per LDS tile
constexpr int kRowTile = 16;                      // query rows per wave

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int DT>
struct MfmaType;
template <>
struct MfmaType<kFp16> {
    typedef f16x8 vec;
    __device__ static f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static _Float16 cvt(float x) { return (_Float16)x; }
};
template <>
struct MfmaType<kBf16> {
    typedef bf16x8 vec;
    __device__ static f32x4 mma(vec a, vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __bf16 cvt(float x) { return (__bf16)x; }
};

// max / sum of a per-lane value over the 4 lanes {p, p+16, p+32, p+48}
__device__ __forceinline__ float group_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
    r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float group_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(r[0]) + __int_as_float(r[1]);
    r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

template <int DT, int D>
struct Mfma {
    using T = MfmaType<DT>;
    typedef typename T::vec vec;
    static constexpr int NCH = D / 8;             // 16-byte chunks per row
    static constexpr int KK = D / 32;             // k-steps of Q K^T
    static constexpr int DB = D / 16;             // 16-channel blocks of O
    static constexpr int ROWB = D * 2;            // bytes per K/V row
    static constexpr int TILEB = kTile * ROWB;    // bytes per K (or V) tile
    static constexpr int KSTEP = 256 / NCH;       // keys per cooperative load pass
    static constexpr int LD = kTile / KSTEP;      // 16-byte loads per thread per tile
    static constexpr int RB = kMWaves * kRowTile; // query rows per workgroup

    struct Smem {
        uint8_t k[2][TILEB];
        uint8_t v[2][TILEB];
    };

    __device__ static uint32_t lds_off(int key, int chunk) {
        return (uint32_t)key * ROWB + (uint32_t)((chunk ^ (key % NCH)) * 16);
    }

    __device__ static __forceinline__ void segment(const KernelArgs &a, Smem &sm, int b, int n, int kvh, int rb,
                                   int t_lo, int t_hi, int slot, bool whole) {
        b = __builtin_amdgcn_readfirstlane(b);
        n = __builtin_amdgcn_readfirstlane(n);
        kvh = __builtin_amdgcn_readfirstlane(kvh);
        rb = __builtin_amdgcn_readfirstlane(rb);
        t_lo = __builtin_amdgcn_readfirstlane(t_lo);
        t_hi = __builtin_amdgcn_readfirstlane(t_hi);
        slot = __builtin_amdgcn_readfirstlane(slot);

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int g = lane >> 4;
        const int p = lane & 15;
        const int rloc = wave * kRowTile + p;          // row within the block
        const int row = rb * RB + rloc;                // row within the kv head
        const bool row_ok = row < a.R;
        const int qi = row_ok ? row / a.G : 0;
        const int qh = kvh * a.G + (row_ok ? row % a.G : 0);

        int t_end = t_hi;
        if (a.causal) {
            const int i_max = (min(rb * RB + RB, a.R) - 1) / a.G;
            t_end = min(t_end, i_max + n - a.qLen + 1);
        }
        const int causal_last = a.causal ? qi + n - a.qLen : INT32_MAX;
        const int ntiles = t_end > t_lo ? (t_end - t_lo + kTile - 1) / kTile : 0;

        // this lane's query row as the B operand of S^T = K Q^T
        vec qf[KK];
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            u32x4 x = {0, 0, 0, 0};
            if (row_ok)
                x = *(const u32x4 *)((const uint16_t *)a.q +
                                     (((size_t)b * a.qLen + qi) * a.Hq + qh) * D + 32 * kk + 8 * g);
            qf[kk] = __builtin_bit_cast(vec, x);
        }

        // K/V of sequence b; the descriptor range ends with token t_end - 1,
        // so loads past it return zeros without touching memory
        const uint32_t tok_bytes = (uint32_t)a.Hkv * D * 2;
        const size_t seq_off = (size_t)b * a.kv_cap * a.Hkv * D;
        const uint32_t range = (uint32_t)t_end * tok_bytes;
        const __amdgpu_buffer_rsrc_t krsrc = make_rsrc((const uint16_t *)a.k + seq_off, range);
        const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc((const uint16_t *)a.v + seq_off, range);
        const int cch = tid % NCH;                     // chunk this thread loads
        const int key0 = tid / NCH;                    // first key this thread loads
        const uint32_t goff = (uint32_t)key0 * tok_bytes + (uint32_t)kvh * ROWB + 16u * cch;

        u32x4 kst[LD], vst[LD];
        auto gload = [&](int tile) {
            const uint32_t base = (uint32_t)(t_lo + tile * kTile) * tok_bytes + goff;
#pragma unroll
            for (int u = 0; u < LD; ++u) {
                kst[u] = load16(krsrc, base + (uint32_t)(u * KSTEP) * tok_bytes);
                vst[u] = load16(vrsrc, base + (uint32_t)(u * KSTEP) * tok_bytes);
            }
        };
        auto lstore = [&](int stage) {
#pragma unroll
            for (int u = 0; u < LD; ++u) {
                const uint32_t off = lds_off(key0 + u * KSTEP, cch);
                *(u32x4 *)(sm.k[stage] + off) = kst[u];
                *(u32x4 *)(sm.v[stage] + off) = vst[u];
            }
        };

        float m_run = kNegInf, l_run = 0.f;
        f32x4 o[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto compute = [&](int stage, int tile) {
            const uint8_t *kt = sm.k[stage];
            const uint8_t *vt = sm.v[stage];
            // S^T for the 4 blocks of 16 keys
            f32x4 s[4];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const vec ka = __builtin_bit_cast(
                        vec, *(const u32x4 *)(kt + lds_off(kb * 16 + p, 4 * kk + g)));
                    s[kb] = T::mma(ka, qf[kk], s[kb]);
                }
            }
            // mask, scale to log2 units, online softmax for the lane's row
            const int key_base = t_lo + tile * kTile + 4 * g;
            float x[4][4];
            float mx = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = key_base + kb * 16 + i;
                    const bool vis = row_ok && key < t_end && key <= causal_last;
                    x[kb][i] = vis ? s[kb][i] * a.qscale : kNegInf;
                    mx = fmaxf(mx, x[kb][i]);
                }
            mx = group_max(mx);
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == kNegInf ? 0.f : m_new;
            const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_use);
            float ps = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[kb][i] = fast_exp2(x[kb][i] - m_use);
                    ps += x[kb][i];
                }
            ps = group_sum(ps);
            l_run = l_run * alpha + ps;
            m_run = m_new;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db] *= alpha;
            }
            // O^T += V^T P^T, 32 keys at a time
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                vec pb;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pb[i] = T::cvt(x[2 * h2][i]);
                    pb[4 + i] = T::cvt(x[2 * h2 + 1][i]);
                }
                const int kr = 32 * h2 + 4 * g + (p >> 2);     // key read by this lane
                const int c = p & 3;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int chunk = 2 * db + (c >> 1);
                    const uint32_t half = 8u * (c & 1);
                    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)(vt + lds_off(kr, chunk) + half));
                    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (lds_s16x4 *)(vt + lds_off(kr + 16, chunk) + half));
                    typedef short s16x8 __attribute__((ext_vector_type(8)));
                    const s16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    o[db] = T::mma(__builtin_bit_cast(vec, va), pb, o[db]);
                }
            }
        };

        // double-buffered K-outer loop over tiles of 64 keys; the loads of the
        // next tile are in flight while the current one is computed (loads
        // past the segment are free, so they are issued unconditionally)
        gload(0);
        lstore(0);
        __syncthreads();
        for (int tile = 0; tile < ntiles; ++tile) {
            gload(tile + 1);
            compute(tile & 1, tile);
            lstore((tile + 1) & 1);
            __syncthreads();
        }

        // epilogue: the lane's row, channels 16 db + 4 g .. + 3
        if (row_ok) {
            const bool empty = !(l_run > 0.f);
            const float inv = empty ? 0.f : 1.f / l_run;
            const float lse2 = empty ? kNegInf : m_run + fast_log2(l_run);
            if (whole) {
                uint16_t *op = (uint16_t *)a.out + (((size_t)b * a.qLen + qi) * a.Hq + qh) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *(u32x2 *)(op + 16 * db + 4 * g) =
                        u32x2{pack2<DT>(o[db][0] * inv, o[db][1] * inv),
                              pack2<DT>(o[db][2] * inv, o[db][3] * inv)};
                if (g == 0 && a.lse)
                    a.lse[((size_t)b * a.Hq + qh) * a.qLen + qi] = empty ? kNegInf : lse2 * kLn2;
            } else {
                const size_t e = (size_t)slot * RB + rloc;   // head_block = 1
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *(f32x4 *)(a.ws_o + e * D + 16 * db + 4 * g) = o[db] * inv;
                if (g == 0) a.ws_lse[e] = lse2;
            }
        }
    }
};

// Two workgroups per CU: LDS holds two double-buffered K/V tile sets, and
// the register allocator is held to two waves per SIMD.
#ifndef MXFA_MFMA_WAVES_PER_EU
#define MXFA_MFMA_WAVES_PER_EU 2
#endif

template <int DT, int D, int SCHED>
__global__ __launch_bounds__(kMWaves * 64)
__attribute__((amdgpu_waves_per_eu(MXFA_MFMA_WAVES_PER_EU)))
void split_kv_mfma_kernel(KernelArgs a) {
    using M = Mfma<DT, D>;
    __shared__ __attribute__((aligned(16))) typename M::Smem sm;
    drive_schedule<SCHED>(a, [&](int b, int n, int hb, int rb, int t_lo, int t_hi, int slot,
                                 bool whole) {
        M::segment(a, sm, b, n, hb, rb, t_lo, t_hi, slot, whole);
    });
}

template <int DT, int D>
hipError_t launch_t(const KernelArgs &a, dim3 grid, hipStream_t stream) {
    KernelArgs args = a;
    void *kargs[] = {&args};
    const void *fn = a.schedule == kBalanced
        ? (const void *)&split_kv_mfma_kernel<DT, D, kBalanced>
        : (const void *)&split_kv_mfma_kernel<DT, D, kFixed>;
    return hipLaunchKernel(fn, grid, dim3(kMWaves * 64), kargs, 0, stream);
}

}  // namespace

hipError_t launch_split_mfma(const KernelArgs &a, int dtype, dim3 grid, hipStream_t stream) {
    if (a.row_block != kMWaves * kRowTile || a.head_block != 1) return hipErrorInvalidValue;
    if (dtype == kFp16) {
        if (a.D == 128) return launch_t<kFp16, 128>(a, grid, stream);
        if (a.D == 64) return launch_t<kFp16, 64>(a, grid, stream);
    } else {
        if (a.D == 128) return launch_t<kBf16, 128>(a, grid, stream);
        if (a.D == 64) return launch_t<kBf16, 64>(a, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mxfa
