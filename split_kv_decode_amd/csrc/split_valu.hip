// Split-KV decode attention, vector-ALU path (gfx950).
//
// Used when a kv head carries few query rows (R = (Hq/Hkv) * qLen small), where
// Q K^T is too thin to be worth the matrix cores and the kernel is bound by
// streaming K and V from HBM.
//
// Work decomposition.  A workgroup (4 waves) owns one KV partition
// [split * chunk, (split + 1) * chunk) of one sequence b, for a block of HPW
// consecutive kv heads and a block of RB query rows per head -- the split-KV
// decomposition of the MXFlashAttn package page (M1 split-KV decode), with the
// K-outer loop and resident Q of the SmallQ FlashAttention README (algorithm
// notes).  Row r of a head's block is query position i = r / G and query head
// h = kvh * G + r % G.
//
// Lane layout.  A token's head slice (D 16-bit values) is read by LPT = D/8
// lanes, 16 contiguous bytes each; such a group of lanes is a "slot", and a
// wave has TPW = 64 / LPT slots.  Slot s of a wave serves kv head (s % HS) of
// the wave's head group and token sub-index (s / HS).  With HS = TPW every
// slot is a different head of the same token, so one load instruction reads
// one contiguous stretch of a token row (the heads sit side by side in the
// [B, kv_cap, Hkv, D] cache) and the workgroup streams whole token rows.  The
// workgroup's waves cover HG head groups x TI token interleaves (HG * TI = 4).
// Each lane loads U tokens of K and of V per step and computes partial dot
// products over its 8 channels for U tokens x RB rows (N = U * RB partials,
// v_dot2 with fp32 accumulation).
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
// the accumulated output rescaled by exp(m_old - m_new)).  Per slot and row,
// in log2 units (Q K^T is scaled by log2(e)/sqrt(D) so exp2 replaces exp):
// row max over the slot's U tokens by DPP, p = exp2(s - m_new),
// alpha = exp2(m_old - m_new), l = alpha * l + sum p.  p and alpha are shared
// within the slot through a small LDS array; the rescale of O is skipped when
// no row's maximum moved anywhere in the wave.  O += p V in fp32 with V
// converted from 16 bits (the SmallQ README's fp32 PV accumulation).
//
// Epilogue.  Slots and waves that served the same head hold independent
// (m, l, O) states for different tokens; they are merged with the same
// log-sum-exp rule, then written either as the final output (when the
// workgroup covered the whole KV range of its heads) or as a normalised
// partial O plus its log2-sum-exp for the combine kernel.
//
// Schedules (see launch.h).  With fixed partitions a workgroup processes one
// segment [split * chunk, ...) of one (sequence, head block, row block)
// stream.  With the balanced schedule the streams are laid end to end and
// every workgroup takes an equal share of the concatenation, processing the
// one or more stream segments that fall into it; this keeps all workgroups
// equally loaded however ragged the sequence lengths are.  The lengths are
// read on the device, so each workgroup first forms their prefix sums.
//
// Paged caches.  With a block table, token j of sequence b is row j % page of
// page block_table[b][j / page].  Steps are then aligned to multiples of
// TSTEP tokens (at most 16, and page >= 16), so the tokens of one step lie in
// one page: the page is looked up once per step (a vector load of its
// block-table entry, issued one step of the wave ahead) and the step reads
// through a buffer descriptor whose range ends at the page's last valid
// token.  Tokens of the first step that precede the segment are masked.
#include "device_common.h"
#include "launch.h"
#include "schedule.h"

namespace mxfa {
namespace {

constexpr int kWaves = 4;

// Occupancy target (waves per SIMD) handed to the register allocator.
#ifndef MXFA_VALU_WAVES_PER_EU
#define MXFA_VALU_WAVES_PER_EU 2
#endif

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

template <int DT, int D, int RB, int HS, int HG, bool PAGED>
struct Valu {
    static constexpr int LPT = D / 8;                  // lanes per slot
    static constexpr int LB = ilog2(LPT);              // 4 (D=128) or 3 (D=64)
    static constexpr int TPW = 64 / LPT;               // slots per wave
    static constexpr int TSUB = TPW / HS;              // token sub-slots per wave
    static constexpr int TI = kWaves / HG;             // token interleave across waves
    static constexpr int HPW = HG * HS;                // kv heads per workgroup
    static constexpr int U0 = (LPT / RB) >= 4 ? 4 : (LPT / RB);
    // tokens per slot per step; a paged step stays within kMinPage tokens
    static constexpr int U = (PAGED && U0 * TSUB > kMinPage) ? kMinPage / TSUB : U0;
    static constexpr int N = U * RB;                   // partial scores per lane per step
    static constexpr int H = ilog2(N);                 // halving steps
    static constexpr int LOGRB = ilog2(RB);
    static constexpr int LOGU = ilog2(U);
    static constexpr int TSTEP = U * TSUB;             // tokens per wave step
    static constexpr int NSTATE = TI * TSUB;           // partial states per (head, row)
    static_assert(D == 64 || D == 128, "head dim");
    static_assert(N >= 2 && N <= LPT, "reduce-scatter shape");
    static_assert(TPW % HS == 0 && kWaves % HG == 0, "slot mapping");

    struct Smem {
        float p[kWaves][TPW][N];
        float a[kWaves][TPW][RB];
        float m[NSTATE][HPW][RB];
        float l[NSTATE][HPW][RB];
        float o[NSTATE][HPW][RB][D];
    };

    // Tokens [t_lo, t_hi) of the stream (b, hb, rb); n is sequence b's valid
    // length.  whole: the segment is the stream's entire range [0, n), so the
    // final output is written; otherwise the partial goes to `slot`.
    __device__ static __forceinline__ void segment(const KernelArgs &a, Smem &sm, int b, int n, int hb, int rb,
                                   int t_lo, int t_hi, int slot, bool whole) {
        b = __builtin_amdgcn_readfirstlane(b);
        n = __builtin_amdgcn_readfirstlane(n);
        hb = __builtin_amdgcn_readfirstlane(hb);
        rb = __builtin_amdgcn_readfirstlane(rb);
        t_lo = __builtin_amdgcn_readfirstlane(t_lo);
        t_hi = __builtin_amdgcn_readfirstlane(t_hi);
        slot = __builtin_amdgcn_readfirstlane(slot);

        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int hg = wave % HG;
        const int ti = wave / HG;
        const int sl = lane & (LPT - 1);
        const int sg = lane >> LB;
        const int hs = sg % HS;
        const int ts = sg / HS;
        const int hh = hg * HS + hs;                // head index inside the block
        const int kvh = hb * HPW + hh;
        const bool head_ok = kvh < a.Hkv;

        const int row0 = rb * RB;
        // this sequence's query rows (fewer than R in a packed batch)
        const int qn = __builtin_amdgcn_readfirstlane(q_count(a, b));
        const int Rb = a.G * qn;
        if (row0 >= Rb) {
            t_hi = t_lo;                // a row block with no query: nothing to read
        } else if (a.causal) {
            // no row of this block sees a key past (last query position) + n - qn
            const int i_max = (min(row0 + RB, Rb) - 1) / a.G;
            t_hi = min(t_hi, i_max + n - qn + 1);
            t_hi = max(t_hi, t_lo);     // an empty segment, never a negative range
        }
        // first token of step 0: steps start on cache rows that are multiples
        // of TSTEP (a paged cache: within the page; a contiguous or packed
        // one: in the K/V arrays, so a step's rows are one aligned block of
        // TSTEP * Hkv * D * 2 bytes).  The rows before t_lo are masked; an
        // index below 0 reads nothing (its offset wraps past the descriptor
        // range).  Shares of the balanced schedule start anywhere, and with
        // misaligned steps (every step then straddles two such blocks) the
        // workgroups starting on odd rows ran 2.6% longer.
        const int t_base =
            PAGED ? (t_lo & ~(TSTEP - 1))
                  : t_lo - (int)((kv_token0(a, b) + (size_t)t_lo) & (size_t)(TSTEP - 1));
        const int nsteps = t_hi > t_lo ? (t_hi - t_base + TSTEP - 1) / TSTEP : 0;

        // lane permutation of the reduce-scatter
        const int gperm = sl ^ (((sl >> 2) & 1) * 3);
        const int phi = gperm >> (LB - H);
        const int phir = phi & (RB - 1);
        const int phiu = phi >> LOGRB;

        // the score this lane finishes with belongs to row (row0 + phir)
        const int my_row = row0 + phir;
        const bool row_ok = head_ok && my_row < Rb;
        const int causal_last = a.causal ? my_row / a.G + n - qn : INT32_MAX;

        // K/V of sequence b through buffer descriptors whose range ends with
        // token t_hi - 1: loads past the segment (the ragged end of the last
        // step, the prefetch after the final step) return zeros without
        // touching memory, so every load is issued unconditionally.  Lanes of
        // a head past Hkv get an offset beyond any valid range (< 2^30).
        const uint32_t tok_bytes = (uint32_t)a.Hkv * D * 2;
        const size_t seq_off = kv_token0(a, b) * a.Hkv * D;
        const uint32_t range = (uint32_t)t_hi * tok_bytes;
        const __amdgpu_buffer_rsrc_t krsrc =
            make_rsrc((const uint16_t *)a.k + (PAGED ? 0 : seq_off), range);
        const __amdgpu_buffer_rsrc_t vrsrc =
            make_rsrc((const uint16_t *)a.v + (PAGED ? 0 : seq_off), range);
        const uint32_t lane_base = head_ok ? (uint32_t)kvh * D * 2 + 16u * sl : 0x80000000u;
        uint32_t koff[U], voff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            koff[u] = lane_base + (uint32_t)((u ^ phiu) * TSUB + ts) * tok_bytes;
            voff[u] = lane_base + (uint32_t)(u * TSUB + ts) * tok_bytes;
        }

        // paged: the block-table entry of each step is read with a vector load
        // one load step of the wave ahead (tracked with the K/V loads, so the
        // wait for it never waits for LDS traffic or for loads issued after
        // it), through a descriptor that ends at the entry of the last page
        // holding a token below t_hi: entries past it read 0 and belong to
        // steps that load nothing
        const __amdgpu_buffer_rsrc_t bt_rsrc = make_rsrc(
            PAGED ? (const void *)(a.block_table + (size_t)b * a.max_pages) : nullptr,
            PAGED ? (uint32_t)((t_hi + (1 << a.log_page) - 1) >> a.log_page) * 4u : 0u);
        auto fetch_entry = [&](int st) -> uint32_t {
            return __builtin_amdgcn_raw_buffer_load_b32(
                bt_rsrc, (uint32_t)((t_base + st * TSTEP) >> a.log_page) * 4u, 0, 0);
        };
        uint32_t e_next = PAGED ? fetch_entry(ti) : 0u;    // the wave's first step

        auto load_step = [&](int st, u32x4 (&kr)[U], u32x4 (&vr)[U]) {
            if constexpr (PAGED) {
                // the step's page (its entry was requested one step ahead, and
                // the next step's is requested now); its descriptors end at the
                // last token below t_hi (no range when the step lies past it)
                const uint32_t e = e_next;
                e_next = fetch_entry(st + TI);
                const int tb = t_base + st * TSTEP;
                const int pi = tb >> a.log_page;
                const int valid = t_hi - (pi << a.log_page);
                const int page = 1 << a.log_page;
                const int pg = clampi(__builtin_amdgcn_readfirstlane((int)e), 0, a.num_pages - 1);
                const uint32_t rng = valid <= 0 ? 0u : (uint32_t)min(valid, page) * tok_bytes;
                const size_t poff = ((size_t)pg << a.log_page) * a.Hkv * D;
                const __amdgpu_buffer_rsrc_t kp = make_rsrc((const uint16_t *)a.k + poff, rng);
                const __amdgpu_buffer_rsrc_t vp = make_rsrc((const uint16_t *)a.v + poff, rng);
                const uint32_t base = (uint32_t)(tb & (page - 1)) * tok_bytes;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    kr[u] = load16(kp, base + koff[u]);
                    vr[u] = load16(vp, base + voff[u]);
                }
            } else {
                const uint32_t base = (uint32_t)(t_base + st * TSTEP) * tok_bytes;
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    kr[u] = load16(krsrc, base + koff[u]);
                    vr[u] = load16(vrsrc, base + voff[u]);
                }
            }
        };

        // the wave's first step is requested before Q is loaded
        const int nmine = nsteps > ti ? (nsteps - ti + TI - 1) / TI : 0;
        u32x4 kA[U], vA[U], kB[U], vB[U];
        int st = ti;
        load_step(st, kA, vA);

        // Q rows of this lane's head, resident for the whole segment (16-bit)
        u32x4 qr[RB];
        const size_t qtok0 = q_token(a, b, 0);
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int row = row0 + (r ^ phir);
            if (head_ok && row < Rb) {
                const int i = row / a.G;
                const int h = kvh * a.G + row % a.G;
                const uint16_t *qp = (const uint16_t *)a.q +
                                     ((qtok0 + i) * a.Hq + h) * D + 8 * sl;
                qr[r] = *(const u32x4 *)qp;
            } else {
                qr[r] = u32x4{0, 0, 0, 0};
            }
        }

        float m_run = kNegInf, l_run = 0.f;
        float o[RB][8];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[r][e] = 0.f;

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

            const int tok = t_base + st * TSTEP + phiu * TSUB + ts;
            const bool vis = row_ok && tok < t_hi && tok <= causal_last && tok >= t_lo;
            const float x = vis ? s * a.qscale : kNegInf;

            const float mx = AllReduce<LB, 0, LOGU>::max(x);
            const float m_new = fmaxf(m_run, mx);
            const float m_use = m_new == kNegInf ? 0.f : m_new;
            const float p = fast_exp2(x - m_use);
            // alpha = 1 exactly when the row maximum did not move (also for
            // rows that have seen nothing yet), so the rescale can be skipped
            const float alpha = m_new == m_run ? 1.f : fast_exp2(m_run - m_use);
            const float psum = AllReduce<LB, 0, LOGU>::sum(p);
            l_run = l_run * alpha + psum;
            m_run = m_new;

            wave_lds_sync();
            sm.p[wave][sg][phi] = p;
            sm.a[wave][sg][phir] = alpha;
            wave_lds_sync();
            float pc[N], ac[RB];
#pragma unroll
            for (int k = 0; k < N; ++k) pc[k] = sm.p[wave][sg][k];
            bool moved = false;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                ac[r] = sm.a[wave][sg][r];
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

        // K-outer loop: the wave with token interleave ti takes steps ti,
        // ti + TI, ...; the loads of its next step are issued before the
        // current one is computed (register double buffer).  Loads are
        // unconditional, so the wait counts stay exact.
        {
            for (int pair = 0; pair < nmine / 2; ++pair) {
                load_step(st + TI, kB, vB);
                compute_step(st, kA, vA);
                load_step(st + 2 * TI, kA, vA);
                compute_step(st + TI, kB, vB);
                st += 2 * TI;
            }
            if (nmine & 1) compute_step(st, kA, vA);
        }

        // ---- merge the states of each (head, row), then write ----
        const int state = ti * TSUB + ts;
        if (phiu == 0) {
            sm.m[state][hh][phir] = m_run;
            sm.l[state][hh][phir] = l_run;
        }
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int e = 0; e < 8; e += 4)
                *(f32x4 *)&sm.o[state][hh][r][8 * sl + e] =
                    f32x4{o[r][e], o[r][e + 1], o[r][e + 2], o[r][e + 3]};
        __syncthreads();

        constexpr int Q4 = D / 4;
        for (int idx = threadIdx.x; idx < HPW * RB * Q4; idx += kWaves * 64) {
            const int d0 = (idx % Q4) * 4;
            const int r = (idx / Q4) % RB;
            const int hx = idx / (Q4 * RB);
            const int row = row0 + r;
            const int head = hb * HPW + hx;
            if (row >= Rb || head >= a.Hkv) continue;
            float M = kNegInf;
#pragma unroll
            for (int s2 = 0; s2 < NSTATE; ++s2) M = fmaxf(M, sm.m[s2][hx][r]);
            float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
            if (M != kNegInf) {
#pragma unroll
                for (int s2 = 0; s2 < NSTATE; ++s2) {
                    const float ms = sm.m[s2][hx][r];
                    const float sc = ms == kNegInf ? 0.f : fast_exp2(ms - M);
                    den += sc * sm.l[s2][hx][r];
                    const f32x4 os = *(const f32x4 *)&sm.o[s2][hx][r][d0];
#pragma unroll
                    for (int j = 0; j < 4; ++j) num[j] += sc * os[j];
                }
            }
            const bool empty = !(den > 0.f);
            const float inv = empty ? 0.f : 1.f / den;
            const float lse2 = empty ? kNegInf : M + fast_log2(den);
            if (whole) {
                const int i = row / a.G;
                const int h = head * a.G + row % a.G;
                uint16_t *op = (uint16_t *)a.out + (q_token(a, b, i) * a.Hq + h) * D + d0;
                *(u32x2 *)op = u32x2{pack2<DT>(num[0] * inv, num[1] * inv),
                                     pack2<DT>(num[2] * inv, num[3] * inv)};
                if (d0 == 0 && a.lse)
                    a.lse[lse_index(a, b, h, i)] = empty ? kNegInf : lse2 * kLn2;
            } else {
                const size_t e = ((size_t)slot * HPW + hx) * RB + r;
                *(f32x4 *)(a.ws_o + e * D + d0) =
                    f32x4{num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv};
                if (d0 == 0) a.ws_lse[e] = lse2;
            }
        }
        __syncthreads();    // the LDS state is reused by the next segment
    }
};

template <int DT, int D, int RB, int HS, int HG, int SCHED, bool PAGED>
__global__ __launch_bounds__(kWaves * 64)
__attribute__((amdgpu_waves_per_eu(MXFA_VALU_WAVES_PER_EU)))
void split_kv_valu_kernel(KernelArgs a) {
    using V = Valu<DT, D, RB, HS, HG, PAGED>;
    __shared__ __attribute__((aligned(16))) typename V::Smem sm;
    drive_schedule<SCHED>(a, [&](int b, int n, int hb, int rb, int t_lo, int t_hi, int slot,
                                 bool whole) {
        V::segment(a, sm, b, n, hb, rb, t_lo, t_hi, slot, whole);
    });
}

template <int DT, int D, int RB, int HS, int HG>
hipError_t launch_t(const KernelArgs &a, dim3 grid, hipStream_t stream) {
    KernelArgs args = a;
    void *kargs[] = {&args};
    const bool paged = a.block_table != nullptr;
    const void *fn =
        a.schedule == kBalanced
            ? (paged ? (const void *)&split_kv_valu_kernel<DT, D, RB, HS, HG, kBalanced, true>
                     : (const void *)&split_kv_valu_kernel<DT, D, RB, HS, HG, kBalanced, false>)
            : (paged ? (const void *)&split_kv_valu_kernel<DT, D, RB, HS, HG, kFixed, true>
                     : (const void *)&split_kv_valu_kernel<DT, D, RB, HS, HG, kFixed, false>);
    return hipLaunchKernel(fn, grid, dim3(kWaves * 64), kargs, 0, stream);
}

// Head layouts: all slots are heads with 2 or 1 head groups per workgroup,
// or one head per workgroup with the slots on different tokens.
template <int DT, int D, int RB>
hipError_t launch_h(const KernelArgs &a, int layout, dim3 grid, hipStream_t stream) {
    constexpr int TPW = 64 / (D / 8);
    switch (layout) {
    case kHeadsX2: return launch_t<DT, D, RB, TPW, 2>(a, grid, stream);
    case kHeadsX1: return launch_t<DT, D, RB, TPW, 1>(a, grid, stream);
    case kTokens: return launch_t<DT, D, RB, 1, 1>(a, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, int D>
hipError_t launch_rb(const KernelArgs &a, int layout, dim3 grid, hipStream_t stream) {
    switch (a.row_block) {
    case 1: return launch_h<DT, D, 1>(a, layout, grid, stream);
    case 2: return launch_h<DT, D, 2>(a, layout, grid, stream);
    case 4: return launch_h<DT, D, 4>(a, layout, grid, stream);
    case 8: return launch_h<DT, D, 8>(a, layout, grid, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_split_valu(const KernelArgs &a, int dtype, int layout, dim3 grid,
                             hipStream_t stream) {
    if (dtype == kFp16) {
        if (a.D == 128) return launch_rb<kFp16, 128>(a, layout, grid, stream);
        if (a.D == 64) return launch_rb<kFp16, 64>(a, layout, grid, stream);
    } else {
        if (a.D == 128) return launch_rb<kBf16, 128>(a, layout, grid, stream);
        if (a.D == 64) return launch_rb<kBf16, 64>(a, layout, grid, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mxfa
