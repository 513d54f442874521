// Matrix-core split kernel (templates; instantiated per tile width in
// split_mfma.hip and split_mfma_wide.hip).
//
// Split-KV decode attention, matrix-core path (gfx950 MFMA).
//
// Used when a kv head carries several query rows (R = (Hq/Hkv) * qLen of at
// least 4 at head dim 128, 8 at 64; GQA groups times a multi-token draft):
// Q K^T and P V are then dense
// contractions with 16-row tiles, which is how the ops-transformer articles
// place FlashAttention on a matrix unit (Q K^T and P V on the cube unit,
// softmax and scaling on the vector unit).  fp32 accumulation throughout.
//
// Work decomposition.  A workgroup of 4 waves (one per SIMD, one workgroup
// per CU) serves a segment of one stream (sequence b, block of HPW kv heads,
// block of 64 query rows; schedules in schedule.h).  Each kv head of the
// block gets WPH = 4 / HPW waves; the segment is cut into tiles of 32 keys
// and the head's wave j takes tiles j, j + WPH, j + 2 WPH, ...: every wave
// holds all 64 rows of its head (4 row tiles of 16) and its own online-
// softmax state, and streams its tiles with no workgroup barrier, one tile in
// flight in registers.  At the end of the segment the states of each head's
// waves are merged through LDS with the same log-sum-exp rule as the split
// merge.  With two heads per workgroup (the planner's choice when Hkv is
// even) the workgroup reads 512 contiguous bytes of each token row of the
// cache instead of 256, which streams measurably faster from HBM; the price
// is twice as many partial results per row for the merge kernel.
//
// Per tile, with v_mfma_f32_16x16x32 (lane l = 16 g + p; A: row p, k-slice
// 8g..8g+7; B: k-slice 8g..8g+7, column p; C: rows 4g..4g+3, column p):
//   S^T = K Q^T: A = 16 keys x 32 channels of K, loaded from memory straight
//   into the operand layout (lane (g, p) loads 16 bytes of key p) in the
//   64-row launches (KD), or read back from the wave's LDS tile (16-row
//   variant), B = Q^T (the lane's query row p of each row tile, resident in
//   registers).  Lane
//   (g, p) receives the scores of keys 4g..4g+3 of each 16-key block for
//   query row p, so every lane owns one query row per row tile: its running
//   max m, running sum l and the rescale alpha are per lane (online softmax
//   of the ops-transformer articles), the row max / sum across the 4 lane
//   groups take two permlane swaps.
//   O^T += V^T P^T over the 32 keys: B = P^T is the lane's own probabilities
//   (rounded to the input type) for keys {4g..4g+3} and {16+4g..16+4g+3} --
//   the MFMA k-slice of lane group g is taken to mean exactly these keys --
//   and A = V^T holds the same keys for 16 channels, read from the wave's V
//   tile in LDS with two transposed reads (ds_read_b64_tr_b16: within a
//   16-lane group, lane 4i + c reads 4 channels of key i and lane p receives
//   channel p of the 4 keys).  One V^T operand serves all 4 row tiles.
// V (and, without KD, K) rows are stored in LDS with their 16-byte chunks
// XOR-swizzled by the key index (twice the key index for V), so the keys read
// by one transposed read hit distinct banks.
//
// Paged caches.  With a block table, token j of sequence b is row j % page of
// page block_table[b][j / page].  Tiles are then aligned to multiples of 32
// tokens and each 16-byte load instruction covers at most 8 consecutive
// tokens, all in one page since page >= 16: the tile's pages are looked up
// one tile ahead and read through descriptors whose range ends at the page's
// last valid token.  Keys of the first tile that precede the segment are
// masked.
//
// Few rows.  With at most 16 query rows per kv head (SMALL) a wave holds one
// row tile and one LDS stage, about 215 registers and 73 KB of LDS per
// workgroup, so two workgroups share a CU.  With 17 to 48 rows a wave holds
// two or three row tiles (RTO = 2, 3) and the launch keeps one workgroup per
// CU, so no matrix product or exponential is spent on the padded rows of a
// 64-row tile.
//
// Head dims.  The tile widths DK x DV (64 x 64, 128 x 128, 192 x 128 or
// 256 x 256) hold any head dims Dk <= DK, Dv <= DV that are multiples of 8:
// the Q channels past Dk are zero, the K and V chunks past the head read a
// valid chunk again (they meet zero Q or feed O channels that are never
// written), and only the first Dv output channels are stored.  Wide tiles
// keep fewer row tiles per wave (32 rows at 192 x 128, 16 at 256 x 256) and
// one LDS stage, so registers and LDS stay within one workgroup per CU.
// Any other head dim (ODD: Dk or Dv not a multiple of 8, so head rows are
// only 2-byte aligned) pads to the same tiles on chip, as the SmallQ
// README's algorithm notes pad the head dim to 16: every 16-byte chunk is
// assembled from 16-bit loads, its elements past the head are set to zero
// (a neighbouring head's or token's values, or the NaN of an unused cache
// slot, must not reach a product), and outputs are stored element by
// element so that nothing past the head is written.  These launches use one
// 16-row tile per wave with K staged in LDS (the loads' 16-bit pieces need
// twice the registers of a 16-byte load while in flight) and one workgroup
// per CU.
#pragma once

#include "device_common.h"
#include "launch.h"
#include "schedule.h"

namespace mxfa {
namespace mfma {

constexpr int kMWaves = 4;
constexpr int kKT = 32;                           // keys per wave tile
// how far (log2 units) a score may exceed the softmax reference before the
// reference is moved: probabilities stay <= 2^8, exact after normalisation
constexpr float kSlack = 8.f;

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

// The 8 16-bit elements of a head-row chunk whose first element is element
// e0 of the head, at byte offset `off` (2-byte aligned) of descriptor r, as
// a 16-byte operand; elements at or past `lim` (the head width) are zero.
// Every load stays inside the descriptor's range or reads 0 (the range
// ends at the segment's last token), so the loads are unconditional and
// the mask is a select, never a product.
template <int POL>
__device__ __forceinline__ u32x4 load_chunk_elems(__amdgpu_buffer_rsrc_t r, uint32_t off, int e0,
                                                  int lim) {
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        h[j] = __builtin_amdgcn_raw_buffer_load_b16(r, off + 2u * j, 0, POL);
    u32x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        x[j] = (e0 + 2 * j < lim ? h[2 * j] : 0u) | ((e0 + 2 * j + 1 < lim ? h[2 * j + 1] : 0u) << 16);
    return x;
}

// DK / DV: the tile widths (padded head dims) of K and V; the real widths
// a.Dk <= DK and a.Dv <= DV are multiples of 8, or any dims with ODD.
// POL: cache policy of the K/V loads (the streaming one when each K/V byte
// is read once; 0 when several row blocks of a head read it again).
// SMALL: one row tile (16 rows) per wave and one LDS stage, for at most 16
// query rows per kv head; two workgroups share a CU.
// KD: K is loaded from memory straight into the matrix operand layout (16
// keys x 64 bytes per load instruction) instead of through LDS (the 64-row
// launches; it matters most when several row blocks of a head re-read its
// K/V from the caches, where the LDS round trip limits the kernel).
// ODD: head dims that are not multiples of 8 (with SMALL, without KD).
// RTO: 16-row tiles per wave when not the tile widths' default (2 for 17-32
// rows per kv head, 3 for 33-48; 0 keeps the default).
template <int DT, int DK, int DV, int HPW, bool PAGED, int POL = MXFA_KV_LOAD_POLICY,
          bool SMALL = false, bool KD = false, bool ODD = false, int RTO = 0>
struct Mfma {
    using T = MfmaType<DT>;
    typedef typename T::vec vec;
    static constexpr int NCHK = DK / 8;           // 16-byte chunks per K row
    static constexpr int NCHV = DV / 8;           // 16-byte chunks per V row
    static constexpr int KK = DK / 32;            // k-steps of Q K^T
    static constexpr int DB = DV / 16;            // 16-channel blocks of O
    static constexpr int ROWK = DK * 2;           // LDS bytes per K row of one head
    static constexpr int ROWV = DV * 2;
    static constexpr int KTB = kKT * ROWK;        // bytes of one wave's K tile
    static constexpr int VTB = kKT * ROWV;
    static constexpr int LDK = kKT * NCHK / 64;   // K loads per lane per tile
    static constexpr int LDV = kKT * NCHV / 64;   // V loads per lane per tile
    static constexpr int RT = SMALL ? 1 : RTO ? RTO : MfmaShape<DK, DV>::RT;   // 16-row tiles per wave
    static constexpr int STG = SMALL ? 1 : MfmaShape<DK, DV>::kStages;    // LDS tile stages per wave
    static constexpr int RB = RT * 16;            // query rows per workgroup and head
    static constexpr int WPH = kMWaves / HPW;     // waves per kv head
    // XOR swizzle of the 16-byte chunks of a row by the key index, within
    // aligned groups of SW chunks (a power of two).  V rows use twice the key
    // index: a transposed read takes 2 chunks of 4 consecutive keys, which
    // then land in 8 distinct chunk slots (with the plain key index keys 2i
    // and 2i + 1 swap the same two slots, a 2-way bank conflict when rows
    // are a multiple of 256 bytes)
    static constexpr int SWK = (NCHK & (NCHK - 1)) == 0 ? NCHK : 8;
    static constexpr int SWV = (NCHV & (NCHV - 1)) == 0 ? NCHV : 8;
    static_assert(DK % 32 == 0 && DV % 32 == 0 && DK <= 256 && DV <= 256, "tile widths");
    static_assert(NCHK % 8 == 0 && NCHV % 8 == 0, "loads of 4+ chunks stay in one key row group");
    static_assert(!ODD || (SMALL && !KD), "odd head dims: 16-row tiles, K through LDS");

    // LDS: during the tile loop, STG K and V tile pairs per wave; during the
    // merge, each wave's RB x DV block of O as fp32 rows of ORS bytes (16
    // bytes of padding, so the fragment stores of 16 rows hit distinct banks).
    static constexpr int ORS = DV * 4 + 16;
    static constexpr int STAGE_BYTES = kMWaves * STG * (KTB + VTB);
    static constexpr int MERGE_BYTES = kMWaves * RB * ORS;
    static constexpr int BUF_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
    struct Smem {
        uint8_t buf[BUF_BYTES];
        float m[kMWaves][RB];
        float l[kMWaves][RB];
        float wt[kMWaves][RB];   // merge weight of each source wave's row
    };

    // the K and V tiles of stage `stage` of a wave, 16-byte chunks of a row
    // XOR-swizzled by the key index
    __device__ static uint32_t k_off(int wave, int stage, int key, int chunk) {
        return (uint32_t)((wave * STG + stage) * (KTB + VTB) + key * ROWK +
                          ((chunk ^ (key % SWK)) * 16));
    }
    __device__ static uint32_t v_off(int wave, int stage, int key, int chunk) {
        return (uint32_t)((wave * STG + stage) * (KTB + VTB) + KTB + key * ROWV +
                          ((chunk ^ ((2 * key) % SWV)) * 16));
    }
    __device__ static uint32_t o_off(int src, int row, int ch) {
        return (uint32_t)((src * RB + row) * ORS + ch * 4);
    }

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
        const int g = lane >> 4;
        const int p = lane & 15;
        // the wave's kv head (hx-th of the block) and its share of the tiles
        const int hx = wave / WPH;
        const int sub = wave % WPH;
        const int kvh = hb * HPW + hx;

        // this sequence's query rows (fewer than R in a packed batch); keys
        // past t_end are invisible to every row of the block
        const int qn = __builtin_amdgcn_readfirstlane(q_count(a, b));
        const int Rb = a.G * qn;
        int t_end = t_hi;
        if (rb * RB >= Rb) {
            t_end = t_lo;               // a row block with no query: nothing to read
        } else if (a.causal) {
            const int i_max = (min(rb * RB + RB, Rb) - 1) / a.G;
            t_end = min(t_end, i_max + n - qn + 1);
            t_end = max(t_end, t_lo);   // an empty segment, never a negative range
        }
        t_end = __builtin_amdgcn_readfirstlane(t_end);
        // first key of tile 0.  A paged cache is read in page-aligned tiles:
        // its segments start on multiples of kKT (the schedule rounds their
        // bounds), so no tile holds keys from before the segment.
        const int t_base = t_lo;
        const int ntiles = t_end > t_lo ? (t_end - t_base + kKT - 1) / kKT : 0;
        const int my_tiles = ntiles > sub ? (ntiles - sub + WPH - 1) / WPH : 0;

        // K/V of sequence b; the descriptor range ends with token t_end - 1,
        // so loads past it return zeros without touching memory
        const uint32_t ktok = (uint32_t)a.Hkv * a.Dk * 2;   // bytes per token row
        const uint32_t vtok = (uint32_t)a.Hkv * a.Dv * 2;
        const size_t kv0 = kv_token0(a, b);
        const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(
            (const uint16_t *)a.k + (PAGED ? 0 : kv0 * a.Hkv * a.Dk), (uint32_t)t_end * ktok);
        const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(
            (const uint16_t *)a.v + (PAGED ? 0 : kv0 * a.Hkv * a.Dv), (uint32_t)t_end * vtok);
        // K and V row-major: load instruction u of a tile covers the flat
        // chunks 64 u .. 64 u + 63 of the tile's rows, lane l chunk
        // (64 u + l) % NCH of key (64 u + l) / NCH.  The lane's byte offset
        // from the first key of its instruction (kfirst(u) = 64 u / NCH);
        // chunks past the head's width read chunk 0 again (their Q channels
        // are zero and their O channels are never written).
        // With KD, load (kb, kk) of a tile gives lane (g, p) the 16 bytes of
        // key 16 kb + p, chunk 4 kk + g: exactly its slice of the A operand
        // of S^T = K Q^T; koff[kk] is the lane's offset from key 16 kb.
        uint32_t koff[LDK], voff[LDV];
#pragma unroll
        for (int u = 0; u < LDK; ++u) {
            if constexpr (KD) {
                const int ch = 4 * (u % KK) + g;
                koff[u] = (uint32_t)p * ktok + (uint32_t)kvh * a.Dk * 2 + 16u * (8 * ch < a.Dk ? ch : 0);
            } else {
                const int f = 64 * u + lane, key = f / NCHK, ch = f % NCHK;
                koff[u] = (uint32_t)(key - 64 * u / NCHK) * ktok + (uint32_t)kvh * a.Dk * 2 +
                          16u * (8 * ch < a.Dk ? ch : 0);
            }
        }
#pragma unroll
        for (int u = 0; u < LDV; ++u) {
            const int f = 64 * u + lane, key = f / NCHV, ch = f % NCHV;
            voff[u] = (uint32_t)(key - 64 * u / NCHV) * vtok + (uint32_t)kvh * a.Dv * 2 +
                      16u * (8 * ch < a.Dv ? ch : 0);
        }

        u32x4 ks[LDK], vs[LDV];
        // the chunk (of the head row) a lane's load u of K / V covers without
        // KD: (64 u + lane) % NCH (NCH = 24 at the 192-wide K tile does not
        // divide 64, so it depends on u)
        int kch[LDK], vch[LDV];
#pragma unroll
        for (int u = 0; u < LDK; ++u) kch[u] = (64 * u + lane) % NCHK;
#pragma unroll
        for (int u = 0; u < LDV; ++u) vch[u] = (64 * u + lane) % NCHV;
        // tile index of the wave's i-th tile; indices past the segment are
        // clamped to ntiles, whose keys all lie past t_end (loads read nothing)
        auto tile_of = [&](int i) { return min(sub + WPH * i, ntiles); };
        // paged: a tile (32 keys, aligned) lies in one page, or in two when the
        // page is 16 tokens; its block-table entries are read with vector
        // loads one tile ahead (tracked with the K/V loads, no scalar-cache
        // wait in the loop) through a descriptor that ends at the last page
        // holding a token below t_end (entries past it read as 0 and are not
        // used).  pg_cur: the pages of the tile loaded next.  The keys of one
        // load instruction (at most 8 consecutive, NCH a multiple of 8) never
        // straddle a page boundary.
        const int page = 1 << a.log_page;
        const __amdgpu_buffer_rsrc_t bt_rsrc = make_rsrc(
            PAGED ? (const void *)(a.block_table + (size_t)b * a.max_pages) : nullptr,
            PAGED ? (uint32_t)((t_end + page - 1) >> a.log_page) * 4u : 0u);
        uint32_t pg_cur[2] = {0u, 0u};
        auto fetch_pages = [&](int j, uint32_t (&pg)[2]) {
            const int t0 = t_base + j * kKT;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                pg[h] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(
                    bt_rsrc, (uint32_t)((t0 + 16 * h) >> a.log_page) * 4u, 0, 0);
        };
        // a tile's two 16-key halves each lie in one page (the same page when
        // pages hold 32 keys or more), and so does every load (its keys stay
        // inside one half): per half one descriptor from the half's
        // block-table entry, whose range ends at the last token below t_end,
        // and the half's byte offset in that page.  Built once per tile and pool, so
        // a load adds only its key's constant offset (a descriptor and a
        // multiply per load, with the SGPR spills they caused, took the
        // Llama-70B-shaped MTP batch in cache-ordered 64-token pages from
        // 101.3 to 103.0 us).
        auto page_halves = [&](const void *pool, uint32_t tokb, size_t row_elems, int t0,
                               __amdgpu_buffer_rsrc_t (&r)[2], uint32_t (&soff)[2]) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int th = t0 + 16 * h;
                const int valid = t_end - (th & ~(page - 1));
                const int pg = clampi(__builtin_amdgcn_readfirstlane((int)pg_cur[h]), 0,
                                      a.num_pages - 1);
                const uint32_t rng = valid <= 0 ? 0u : (uint32_t)min(valid, page) * tokb;
                r[h] = make_rsrc((const uint16_t *)pool + ((size_t)pg << a.log_page) * row_elems,
                                 rng);
                soff[h] = (uint32_t)(th & (page - 1)) * tokb;
            }
        };
        auto gload_v = [&](int j) {
            const int t0 = t_base + j * kKT;
            __amdgpu_buffer_rsrc_t pr[2];
            uint32_t ps[2];
            if constexpr (PAGED) page_halves(a.v, vtok, (size_t)a.Hkv * a.Dv, t0, pr, ps);
#pragma unroll
            for (int u = 0; u < LDV; ++u) {
                const int tok = t0 + 64 * u / NCHV;
                if constexpr (PAGED) {
                    const int dt = 64 * u / NCHV, h = dt >= 16 ? 1 : 0;
                    const uint32_t off = ps[h] + (uint32_t)(dt - 16 * h) * vtok + voff[u];
                    if constexpr (ODD) vs[u] = load_chunk_elems<POL>(pr[h], off, 8 * vch[u], a.Dv);
                    else vs[u] = load16<POL>(pr[h], off);
                } else if constexpr (ODD)
                    vs[u] = load_chunk_elems<POL>(vrsrc, (uint32_t)tok * vtok + voff[u], 8 * vch[u], a.Dv);
                else
                    vs[u] = load16<POL>(vrsrc, (uint32_t)tok * vtok + voff[u]);
            }
        };
        auto gload_k = [&](int j) {
            const int t0 = t_base + j * kKT;
            __amdgpu_buffer_rsrc_t pr[2];
            uint32_t ps[2];
            if constexpr (PAGED) page_halves(a.k, ktok, (size_t)a.Hkv * a.Dk, t0, pr, ps);
#pragma unroll
            for (int u = 0; u < LDK; ++u) {
                const int tok = KD ? t0 + 16 * (u / KK) : t0 + 64 * u / NCHK;
                if constexpr (PAGED) {
                    const int dt = KD ? 16 * (u / KK) : 64 * u / NCHK, h = dt >= 16 ? 1 : 0;
                    const uint32_t off = ps[h] + (uint32_t)(dt - 16 * h) * ktok + koff[u];
                    if constexpr (ODD) ks[u] = load_chunk_elems<POL>(pr[h], off, 8 * kch[u], a.Dk);
                    else ks[u] = load16<POL>(pr[h], off);
                } else if constexpr (ODD)
                    ks[u] = load_chunk_elems<POL>(krsrc, (uint32_t)tok * ktok + koff[u], 8 * kch[u], a.Dk);
                else
                    ks[u] = load16<POL>(krsrc, (uint32_t)tok * ktok + koff[u]);
            }
        };

        // one tile in flight per wave: the first tile is requested before
        // anything else, then Q is loaded while it streams; each later tile's
        // loads are issued as soon as the tile before it is in LDS
        if constexpr (PAGED) fetch_pages(tile_of(0), pg_cur);
        gload_v(tile_of(0));
        gload_k(tile_of(0));
        if constexpr (PAGED) fetch_pages(tile_of(1), pg_cur);

        // the lane's query row p of each row tile, as the B operand of S^T =
        // K Q^T; rows past R are zero and never written
        vec qf[RT][KK];
        int klim[RT];      // last key visible to the lane's row
        const size_t qtok0 = q_token(a, b, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int row = rb * RB + rt * 16 + p;
            const bool ok = row < Rb;
            const int qi = ok ? row / a.G : 0;
            const int qh = kvh * a.G + (ok ? row % a.G : 0);
            klim[rt] = (a.causal && ok) ? min(t_end - 1, qi + n - qn) : t_end - 1;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                u32x4 x = {0, 0, 0, 0};
                const uint16_t *qrow = (const uint16_t *)a.q + ((qtok0 + qi) * a.Hq + qh) * a.Dk;
                if constexpr (ODD) {
                    // 2-byte aligned rows: element loads, channels past the head zero
                    const int e0 = 32 * kk + 8 * g;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = ok && e0 + 2 * j < a.Dk ? qrow[e0 + 2 * j] : 0u;
                        const uint32_t hi = ok && e0 + 2 * j + 1 < a.Dk ? qrow[e0 + 2 * j + 1] : 0u;
                        x[j] = lo | (hi << 16);
                    }
                } else if (ok && 32 * kk + 8 * g < a.Dk) {   // channels past the head: zero
                    x = *(const u32x4 *)(qrow + 32 * kk + 8 * g);
                }
                qf[rt][kk] = __builtin_bit_cast(vec, x);
            }
        }

        // online softmax with a lazily moved reference: every lane keeps the
        // reference m of its row (the same in the row's 4 lanes) and a partial
        // sum l over its own keys; probabilities are exp2(x - m) <= 2^kSlack,
        // and m (with O and l) moves only when a score passes m + kSlack
        float m_run[RT], l_run[RT];
        f32x4 o[RT][DB];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            m_run[rt] = kNegInf;
            l_run[rt] = 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[rt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        auto compute = [&](int set, int j, int jn, int jnn) {
            const int key0 = t_base + j * kKT;
            // stage this tile's K (without KD) and V rows in the wave's LDS
            // buffer `set`; the next tile streams while this one is computed
            if constexpr (!KD) {
#pragma unroll
                for (int u = 0; u < LDK; ++u)
                    *(u32x4 *)(sm.buf + k_off(wave, set, (64 * u + lane) / NCHK, (64 * u + lane) % NCHK)) =
                        ks[u];
                gload_k(jn);
            }
            uint32_t pg_nxt[2];
            if constexpr (PAGED) fetch_pages(jnn, pg_nxt);
#pragma unroll
            for (int u = 0; u < LDV; ++u)
                *(u32x4 *)(sm.buf + v_off(wave, set, (64 * u + lane) / NCHV, (64 * u + lane) % NCHV)) =
                    vs[u];
            gload_v(jn);
            if constexpr (PAGED && !KD) {
                pg_cur[0] = pg_nxt[0];
                pg_cur[1] = pg_nxt[1];
            }
            wave_lds_sync();   // the tiles written above are visible to the whole wave
            // S^T for 4 row tiles x 2 blocks of 16 keys, in log2 units; the A
            // operand (16 keys x 32 channels of K) serves all row tiles
            vec ka[2][KK];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int kk = 0; kk < KK; ++kk)
                    ka[kb][kk] = KD ? __builtin_bit_cast(vec, ks[kb * KK + kk])
                                    : __builtin_bit_cast(vec, *(const u32x4 *)(sm.buf + k_off(
                                                                  wave, set, 16 * kb + p, 4 * kk + g)));
            float x[RT][2][4];
            float mloc[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                // key 16 kb + 4 g + i of the tile is visible iff 16 kb + i <= vis
                const int vis = klim[rt] - key0 - 4 * g;
                mloc[rt] = kNegInf;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < KK; ++kk)
                        acc = T::mma(ka[kb][kk], qf[rt][kk], acc);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float v = 16 * kb + i <= vis ? acc[i] * a.qscale : kNegInf;
                        x[rt][kb][i] = v;
                        mloc[rt] = fmaxf(mloc[rt], v);
                    }
                }
            }
            if constexpr (KD) {
                // K of this tile is consumed: the next tile's K streams now
                gload_k(jn);
                if constexpr (PAGED) {
                    pg_cur[0] = pg_nxt[0];
                    pg_cur[1] = pg_nxt[1];
                }
            }
            // move the reference where a score passed it by more than kSlack
            bool move = false;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) move |= mloc[rt] > m_run[rt] + kSlack;
            if (__builtin_amdgcn_readfirstlane(__any(move) ? 1 : 0)) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const float m_new = fmaxf(m_run[rt], group_max(mloc[rt]));
                    const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run[rt] - m_new);
                    m_run[rt] = m_new;
                    l_run[rt] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) o[rt][db] *= alpha;
                }
            }
            vec pb[RT];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const float m_use = m_run[rt] == kNegInf ? 0.f : m_run[rt];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = fast_exp2(x[rt][kb][i] - m_use);
                        l_run[rt] += e;
                        pb[rt][4 * kb + i] = T::cvt(e);
                    }
            }
            // O^T += V^T P^T; the V^T operand of a channel block serves all row tiles
            const int kr = 4 * g + (p >> 2);            // key read by this lane
            const int c = p & 3;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int chunk = 2 * db + (c >> 1);
                const uint32_t half = 8u * (c & 1);
                const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(sm.buf + v_off(wave, set, kr, chunk) + half));
                const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(sm.buf + v_off(wave, set, kr + 16, chunk) + half));
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
                    o[rt][db] = T::mma(__builtin_bit_cast(vec, va), pb[rt], o[rt][db]);
            }
        };
        for (int i = 0; i < my_tiles; ++i) {
            const int j = tile_of(i);
            compute(STG == 2 ? (i & 1) : 0, j, tile_of(i + 1), tile_of(i + 2));
        }

        // the row sums over the 4 lanes of each row
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) l_run[rt] = group_sum(l_run[rt]);

        // merge the states of each head's WPH waves: every wave leaves its
        // rows of O and its (m, l) in LDS, then the head's waves split its RB
        // rows (wave sub takes rows sub * RPW ..)
        __syncthreads();                       // every wave is done with its V tiles
        if (g == 0) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                sm.m[wave][rt * 16 + p] = m_run[rt];
                sm.l[wave][rt * 16 + p] = l_run[rt];
            }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                *(f32x4 *)(sm.buf + o_off(wave, rt * 16 + p, 16 * db + 4 * g)) = o[rt][db];
        __syncthreads();
        constexpr int LPR = DV / 4;            // lanes per row
        constexpr int RPI = 64 / LPR;          // rows per instruction
        constexpr int RPW = RB / WPH;          // rows per wave
        static_assert(RPW % RPI == 0 && RPW <= 64, "merge split");
        const int src0 = hx * WPH;             // the head's first wave
        // per row (lane j takes the wave's row j): the log-sum-exp rule gives
        // each source wave the weight 2^(m_w - M) / L and the row its lse
        if (lane < RPW) {
            const int rloc = sub * RPW + lane;
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < WPH; ++w) M = fmaxf(M, sm.m[src0 + w][rloc]);
            float sc[WPH];
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < WPH; ++w) {
                const float mw = sm.m[src0 + w][rloc];
                sc[w] = mw == kNegInf ? 0.f : fast_exp2(mw - M);
                L += sc[w] * sm.l[src0 + w][rloc];
            }
            const bool empty = !(L > 0.f);
            const float inv = empty ? 0.f : 1.f / L;
#pragma unroll
            for (int w = 0; w < WPH; ++w) sm.wt[src0 + w][rloc] = sc[w] * inv;
            const int row = rb * RB + rloc;
            if (row < Rb) {
                const float lse2 = empty ? kNegInf : M + fast_log2(L);
                if (whole) {
                    if (a.lse)
                        a.lse[lse_index(a, b, kvh * a.G + row % a.G, row / a.G)] =
                            empty ? kNegInf : lse2 * kLn2;
                } else {
                    a.ws_lse[((size_t)slot * HPW + hx) * RB + rloc] = lse2;
                }
            }
        }
        wave_lds_sync();                       // the wave reads back its own weights
        // then a lane takes 4 channels of a row, and the lanes of one store
        // instruction cover RPI whole rows: results go out as contiguous runs
        const int c0 = 4 * (lane % LPR);       // the lane's first channel
#pragma unroll
        for (int i = 0; i < RPW / RPI; ++i) {
            const int rloc = sub * RPW + i * RPI + lane / LPR;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < WPH; ++w)
                acc += sm.wt[src0 + w][rloc] * *(const f32x4 *)(sm.buf + o_off(src0 + w, rloc, c0));
            const int row = rb * RB + rloc;
            if (row < Rb) {
                if (whole) {
                    const int qi = row / a.G;
                    const int qh = kvh * a.G + row % a.G;
                    uint16_t *op = (uint16_t *)a.out + ((qtok0 + qi) * a.Hq + qh) * a.Dv;
                    if constexpr (ODD) {
                        // 2-byte aligned rows: element stores, none past the head
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (c0 + e < a.Dv) op[c0 + e] = (uint16_t)to16<DT>(acc[e]);
                    } else if (c0 < a.Dv) {            // channels past the head: not written
                        *(u32x2 *)(op + c0) = u32x2{pack2<DT>(acc[0], acc[1]), pack2<DT>(acc[2], acc[3])};
                    }
                } else {
                    const size_t e = ((size_t)slot * HPW + hx) * RB + rloc;
                    *(f32x4 *)(a.ws_o + e * DV + c0) = acc;
                }
            }
        }
        __syncthreads();                       // the next segment reuses the LDS
    }
};

// One workgroup per CU, one wave per SIMD: each wave keeps its head's rows
// of accumulators and one K/V tile in registers.

template <int DT, int DK, int DV, int HPW, int SCHED, bool PAGED, int POL, bool SMALL, bool KD,
          bool ODD = false, int RTO = 0>
__global__ __launch_bounds__(kMWaves * 64)
__attribute__((amdgpu_waves_per_eu(SMALL && !ODD ? 2 : 1, SMALL && !ODD ? 2 : 1)))
void split_kv_mfma_kernel(KernelArgs a) {
    using M = Mfma<DT, DK, DV, HPW, PAGED, POL, SMALL, KD, ODD, RTO>;
    __shared__ __attribute__((aligned(16))) typename M::Smem sm;
    // a paged cache is read in page-aligned tiles, so its segments start on
    // tile boundaries (no key of a segment's first tile precedes it)
    drive_schedule<SCHED, PAGED ? kKT : 1>(a, [&](int b, int n, int hb, int rb, int t_lo, int t_hi,
                                                 int slot, bool whole) {
        M::segment(a, sm, b, n, hb, rb, t_lo, t_hi, slot, whole);
    });
}

template <int DT, int DK, int DV, int HPW, int POL, bool SMALL = false, bool KD = false,
          bool ODD = false, int RTO = 0>
const void *kernel_for(const KernelArgs &a) {
    const bool paged = a.block_table != nullptr;
    return a.schedule == kBalanced
               ? (paged ? (const void *)&split_kv_mfma_kernel<DT, DK, DV, HPW, kBalanced, true, POL, SMALL, KD, ODD, RTO>
                        : (const void *)&split_kv_mfma_kernel<DT, DK, DV, HPW, kBalanced, false, POL, SMALL, KD, ODD, RTO>)
               : (paged ? (const void *)&split_kv_mfma_kernel<DT, DK, DV, HPW, kFixed, true, POL, SMALL, KD, ODD, RTO>
                        : (const void *)&split_kv_mfma_kernel<DT, DK, DV, HPW, kFixed, false, POL, SMALL, KD, ODD, RTO>);
}

// Head dims that are not multiples of 8: 16-row tiles, one kv head per
// workgroup, K through LDS, element loads and stores.
template <int DT, int DK, int DV>
hipError_t launch_odd_t(const KernelArgs &a, dim3 grid, hipStream_t stream) {
    if (a.row_block != kMfmaSmallRows || a.Dk > DK || a.Dv > DV || a.head_block != 1)
        return hipErrorInvalidValue;
    KernelArgs args = a;
    void *kargs[] = {&args};
    const void *fn = kernel_for<DT, DK, DV, 1, MXFA_KV_LOAD_POLICY, true, false, true>(a);
    return hipLaunchKernel(fn, grid, dim3(kMWaves * 64), kargs, 0, stream);
}

template <int DK, int DV>
hipError_t launch_odd_dims(const KernelArgs &a, int dtype, dim3 grid, hipStream_t stream) {
    return dtype == kFp16 ? launch_odd_t<kFp16, DK, DV>(a, grid, stream)
                          : launch_odd_t<kBf16, DK, DV>(a, grid, stream);
}

template <int DT, int DK, int DV>
hipError_t launch_t(const KernelArgs &a, dim3 grid, hipStream_t stream) {
    constexpr bool kHasSmall = DK + DV <= 256;
    const bool small = kHasSmall && a.row_block == kMfmaSmallRows;
    // 32- and 48-row blocks: two or three 16-row tiles per wave
    const bool mid = kHasSmall && (a.row_block == 2 * kMfmaSmallRows || a.row_block == 3 * kMfmaSmallRows);
    if ((!small && !mid && a.row_block != Mfma<DT, DK, DV, 1, false>::RB) || a.Dk > DK || a.Dv > DV ||
        (a.head_block != 1 && a.head_block != 2) || a.Hkv % a.head_block != 0)
        return hipErrorInvalidValue;
    KernelArgs args = a;
    void *kargs[] = {&args};
    if constexpr (kHasSmall) {
        if (small) {
            const void *f = a.head_block == 2 ? kernel_for<DT, DK, DV, 2, MXFA_KV_LOAD_POLICY, true>(a)
                                              : kernel_for<DT, DK, DV, 1, MXFA_KV_LOAD_POLICY, true>(a);
            return hipLaunchKernel(f, grid, dim3(kMWaves * 64), kargs, 0, stream);
        }
        if (mid) {
            const bool three = a.row_block == 3 * kMfmaSmallRows;
            const void *f =
                a.head_block == 2
                    ? (three ? kernel_for<DT, DK, DV, 2, MXFA_KV_LOAD_POLICY, false, true, false, 3>(a)
                             : kernel_for<DT, DK, DV, 2, MXFA_KV_LOAD_POLICY, false, true, false, 2>(a))
                    : (three ? kernel_for<DT, DK, DV, 1, MXFA_KV_LOAD_POLICY, false, true, false, 3>(a)
                             : kernel_for<DT, DK, DV, 1, MXFA_KV_LOAD_POLICY, false, true, false, 2>(a));
            return hipLaunchKernel(f, grid, dim3(kMWaves * 64), kargs, 0, stream);
        }
    }
    // two kv heads per workgroup only with a single row block; several row
    // blocks re-read each head's K/V, which then keep the default cache
    // policy.  These launches load K straight into the operand layout (the
    // 16-row variant above keeps the LDS path, which measured faster there).
    const void *fn = a.head_block == 2    ? kernel_for<DT, DK, DV, 2, MXFA_KV_LOAD_POLICY, false, true>(a)
                     : a.row_blocks > 1 ? kernel_for<DT, DK, DV, 1, 0, false, true>(a)
                                        : kernel_for<DT, DK, DV, 1, MXFA_KV_LOAD_POLICY, false, true>(a);
    return hipLaunchKernel(fn, grid, dim3(kMWaves * 64), kargs, 0, stream);
}

template <int DK, int DV>
hipError_t launch_dims(const KernelArgs &a, int dtype, dim3 grid, hipStream_t stream) {
    return dtype == kFp16 ? launch_t<kFp16, DK, DV>(a, grid, stream)
                          : launch_t<kBf16, DK, DV>(a, grid, stream);
}

}  // namespace mfma
}  // namespace mxfa
