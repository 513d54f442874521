// Split-KV decode attention, matrix-core path (gfx950 MFMA).
//
// Used when a kv head carries many query rows (R = (Hq/Hkv) * qLen >= 32, e.g.
// GQA groups times a multi-token draft): Q K^T and P V are then dense
// contractions with 16-row tiles, which is how the ops-transformer articles
// place FlashAttention on a matrix unit (Q K^T and P V on the cube unit,
// softmax and scaling on the vector unit).  fp32 accumulation throughout.
//
// Work decomposition.  A workgroup of 4 waves (one per SIMD, one workgroup
// per CU) serves a segment of one stream (sequence b, kv head, block of 64
// query rows; schedules in schedule.h).  The segment is cut into tiles of 32
// keys and wave w takes tiles w, w + 4, w + 8, ...: every wave holds all 64
// rows (4 row tiles of 16) and its own online-softmax state, and streams its
// tiles with no workgroup barrier.  Two tiles per wave are in flight in
// registers.  At the end of the segment the 4 per-wave states are merged
// through LDS with the same log-sum-exp rule as the split merge.
//
// Per tile, with v_mfma_f32_16x16x32 (lane l = 16 g + p; A: row p, k-slice
// 8g..8g+7; B: k-slice 8g..8g+7, column p; C: rows 4g..4g+3, column p):
//   S^T = K Q^T: A = 16 keys x 32 channels of K, loaded from memory straight
//   into the operand layout (lane (g, p) loads 16 bytes of key p), B = Q^T
//   (the lane's query row p of each row tile, resident in registers).  Lane
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
// V rows are stored in LDS with their 16-byte chunks XOR-swizzled by the key
// index, so the keys read by one transposed read hit distinct banks.
//
// Paged caches.  With a block table, token j of sequence b is row j % page of
// page block_table[b][j / page].  Tiles are then aligned to multiples of 32
// tokens and each 16-byte load instruction covers 4 (D = 128) or 8 (D = 64)
// consecutive tokens, all in one page since page >= 16: the page is looked up
// per load (a scalar load) and read through a descriptor whose range ends at
// the page's last valid token.  Keys of the first tile that precede the
// segment are masked.
#include "device_common.h"
#include "launch.h"
#include "schedule.h"

namespace mxfa {
namespace {

constexpr int kMWaves = 4;
constexpr int kKT = 32;                           // keys per wave tile
constexpr int kRowTiles = 4;                      // 16-row tiles per wave
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

template <int DT, int D, bool PAGED>
struct Mfma {
    using T = MfmaType<DT>;
    typedef typename T::vec vec;
    static constexpr int NCH = D / 8;             // 16-byte chunks per row
    static constexpr int KK = D / 32;             // k-steps of Q K^T
    static constexpr int DB = D / 16;             // 16-channel blocks of O
    static constexpr int ROWB = D * 2;            // bytes per K/V row of one head
    static constexpr int VTB = kKT * ROWB;        // bytes of one wave's K (or V) tile
    static constexpr int VKEYS = 64 / NCH;        // keys per V load instruction
    static constexpr int LDV = kKT / VKEYS;       // V loads per lane per tile
    static constexpr int LDK = LDV;               // K loads per lane per tile
    static constexpr int RB = kRowTiles * 16;     // query rows per workgroup

    // LDS: during the tile loop, two K and V tile pairs per wave; during the
    // merge, the 4 waves' O fragments (4 sources x 4 row tiles x DB x 64 lanes
    // x f32x4).
    static constexpr int STAGE_BYTES = kMWaves * 2 * 2 * VTB;
    static constexpr int MERGE_BYTES = kMWaves * kRowTiles * DB * 64 * 16;
    static constexpr int BUF_BYTES = STAGE_BYTES > MERGE_BYTES ? STAGE_BYTES : MERGE_BYTES;
    struct Smem {
        uint8_t buf[BUF_BYTES];
        float m[kMWaves][RB];
        float l[kMWaves][RB];
    };

    // tile t (0 = K, 1 = V) of stage `stage` of a wave; 16-byte chunks of a
    // row XOR-swizzled by the key index
    __device__ static uint32_t t_off(int wave, int stage, int t, int key, int chunk) {
        return (uint32_t)(((wave * 2 + stage) * 2 + t) * VTB + key * ROWB +
                          ((chunk ^ (key % NCH)) * 16));
    }
    __device__ static uint32_t o_off(int src, int rt, int db, int lane) {
        return (uint32_t)((((src * kRowTiles + rt) * DB + db) * 64 + lane) * 16);
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

        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int g = lane >> 4;
        const int p = lane & 15;

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
        // first key of tile 0: a paged cache is read in page-aligned tiles
        const int t_base = PAGED ? (t_lo & ~(kKT - 1)) : t_lo;
        const int ntiles = t_end > t_lo ? (t_end - t_base + kKT - 1) / kKT : 0;
        const int my_tiles = ntiles > wave ? (ntiles - wave + kMWaves - 1) / kMWaves : 0;

        // the lane's query row p of each row tile, as the B operand of S^T =
        // K Q^T; rows past R are zero and never written
        vec qf[kRowTiles][KK];
        int klim[kRowTiles];      // last key visible to the lane's row
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
            const int row = rb * RB + rt * 16 + p;
            const bool ok = row < Rb;
            const int qi = ok ? row / a.G : 0;
            const int qh = kvh * a.G + (ok ? row % a.G : 0);
            klim[rt] = (a.causal && ok) ? min(t_end - 1, qi + n - qn) : t_end - 1;
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                u32x4 x = {0, 0, 0, 0};
                if (ok)
                    x = *(const u32x4 *)((const uint16_t *)a.q +
                                         (q_token(a, b, qi) * a.Hq + qh) * D + 32 * kk + 8 * g);
                qf[rt][kk] = __builtin_bit_cast(vec, x);
            }
        }

        // K/V of sequence b; the descriptor range ends with token t_end - 1,
        // so loads past it return zeros without touching memory
        const uint32_t tok_bytes = (uint32_t)a.Hkv * D * 2;
        const size_t seq_off = kv_token0(a, b) * a.Hkv * D;
        const uint32_t range = (uint32_t)t_end * tok_bytes;
        const __amdgpu_buffer_rsrc_t krsrc =
            make_rsrc((const uint16_t *)a.k + (PAGED ? 0 : seq_off), range);
        const __amdgpu_buffer_rsrc_t vrsrc =
            make_rsrc((const uint16_t *)a.v + (PAGED ? 0 : seq_off), range);
        // K and V row-major: lane l loads chunk l % NCH of key l / NCH (+ VKEYS u)
        const int vch = lane % NCH;
        const int vkey = lane / NCH;
        const uint32_t vofs = (uint32_t)vkey * tok_bytes + (uint32_t)kvh * ROWB + 16u * vch;

        u32x4 ks[LDK], vs[LDV];
        // tile index of the wave's i-th tile; indices past the segment are
        // clamped to ntiles, whose keys all lie past t_end (loads read nothing)
        auto tile_of = [&](int i) { return min(wave + kMWaves * i, ntiles); };
        // paged: a tile (32 keys, aligned) lies in one page, or in two when the
        // page is 16 tokens; its block-table entries are read with vector
        // loads one tile ahead (tracked with the K/V loads, no scalar-cache
        // wait in the loop) through a descriptor that ends at the last page
        // holding a token below t_end (entries past it read as 0 and are not
        // used).  pg_cur: the pages of the tile loaded next.
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
        // the load of tokens tok .. tok + VKEYS - 1 (tok a multiple of VKEYS,
        // in half h of its tile) from page entry e, through a descriptor whose
        // range ends at the last token below t_end
        auto page_load = [&](const void *pool, int tok, uint32_t e) {
            const int pi = tok >> a.log_page;
            const int valid = t_end - (pi << a.log_page);
            const int pg = clampi(__builtin_amdgcn_readfirstlane((int)e), 0, a.num_pages - 1);
            const uint32_t rng = valid <= 0 ? 0u : (uint32_t)min(valid, page) * tok_bytes;
            const __amdgpu_buffer_rsrc_t r = make_rsrc(
                (const uint16_t *)pool + ((size_t)pg << a.log_page) * a.Hkv * D, rng);
            return load16(r, (uint32_t)(tok & (page - 1)) * tok_bytes + vofs);
        };
        auto gload_v = [&](int j) {
            if constexpr (PAGED) {
#pragma unroll
                for (int u = 0; u < LDV; ++u)
                    vs[u] = page_load(a.v, t_base + j * kKT + u * VKEYS, pg_cur[u * VKEYS >= 16]);
            } else {
                const uint32_t base = (uint32_t)(t_lo + j * kKT) * tok_bytes;
#pragma unroll
                for (int u = 0; u < LDV; ++u)
                    vs[u] = load16(vrsrc, base + vofs + (uint32_t)(u * VKEYS) * tok_bytes);
            }
        };
        auto gload_k = [&](int j) {
            if constexpr (PAGED) {
#pragma unroll
                for (int u = 0; u < LDK; ++u)
                    ks[u] = page_load(a.k, t_base + j * kKT + u * VKEYS, pg_cur[u * VKEYS >= 16]);
            } else {
                const uint32_t base = (uint32_t)(t_lo + j * kKT) * tok_bytes;
#pragma unroll
                for (int u = 0; u < LDK; ++u)
                    ks[u] = load16(krsrc, base + vofs + (uint32_t)(u * VKEYS) * tok_bytes);
            }
        };

        // online softmax with a lazily moved reference: every lane keeps the
        // reference m of its row (the same in the row's 4 lanes) and a partial
        // sum l over its own keys; probabilities are exp2(x - m) <= 2^kSlack,
        // and m (with O and l) moves only when a score passes m + kSlack
        float m_run[kRowTiles], l_run[kRowTiles];
        f32x4 o[kRowTiles][DB];
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) {
            m_run[rt] = kNegInf;
            l_run[rt] = 0.f;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[rt][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        auto compute = [&](int set, int j, int jn, int jnn) {
            const int key0 = t_base + j * kKT;
            // paged: keys of the first tile before t_lo are not part of the segment
            const int vis_lo = (PAGED && key0 < t_lo) ? t_lo - key0 - 4 * g : INT32_MIN;
            // stage this tile's K and V rows in the wave's LDS buffer `set`
#pragma unroll
            for (int u = 0; u < LDK; ++u)
                *(u32x4 *)(sm.buf + t_off(wave, set, 0, vkey + u * VKEYS, vch)) = ks[u];
            gload_k(jn);       // the next tile streams while this one is computed
            uint32_t pg_nxt[2];
            if constexpr (PAGED) fetch_pages(jnn, pg_nxt);
#pragma unroll
            for (int u = 0; u < LDV; ++u)
                *(u32x4 *)(sm.buf + t_off(wave, set, 1, vkey + u * VKEYS, vch)) = vs[u];
            gload_v(jn);
            if constexpr (PAGED) {
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
                    ka[kb][kk] = __builtin_bit_cast(
                        vec, *(const u32x4 *)(sm.buf + t_off(wave, set, 0, 16 * kb + p, 4 * kk + g)));
            float x[kRowTiles][2][4];
            float mloc[kRowTiles];
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
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
                        const float v = (16 * kb + i <= vis && 16 * kb + i >= vis_lo)
                                            ? acc[i] * a.qscale : kNegInf;
                        x[rt][kb][i] = v;
                        mloc[rt] = fmaxf(mloc[rt], v);
                    }
                }
            }
            // move the reference where a score passed it by more than kSlack
            bool move = false;
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) move |= mloc[rt] > m_run[rt] + kSlack;
            if (__builtin_amdgcn_readfirstlane(__any(move) ? 1 : 0)) {
#pragma unroll
                for (int rt = 0; rt < kRowTiles; ++rt) {
                    const float m_new = fmaxf(m_run[rt], group_max(mloc[rt]));
                    const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run[rt] - m_new);
                    m_run[rt] = m_new;
                    l_run[rt] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) o[rt][db] *= alpha;
                }
            }
            vec pb[kRowTiles];
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
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
                    (lds_s16x4 *)(sm.buf + t_off(wave, set, 1, kr, chunk) + half));
                const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4 *)(sm.buf + t_off(wave, set, 1, kr + 16, chunk) + half));
                typedef short s16x8 __attribute__((ext_vector_type(8)));
                const s16x8 va = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
                for (int rt = 0; rt < kRowTiles; ++rt)
                    o[rt][db] = T::mma(__builtin_bit_cast(vec, va), pb[rt], o[rt][db]);
            }
        };
        // one tile in flight per wave: the next tile's loads are issued as
        // soon as this tile is in LDS
        if constexpr (PAGED) fetch_pages(tile_of(0), pg_cur);
        gload_v(tile_of(0));
        gload_k(tile_of(0));
        if constexpr (PAGED) fetch_pages(tile_of(1), pg_cur);
        for (int i = 0; i < my_tiles; ++i) {
            const int j = tile_of(i);
            compute(i & 1, j, tile_of(i + 1), tile_of(i + 2));
        }

        // the row sums over the 4 lanes of each row
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) l_run[rt] = group_sum(l_run[rt]);

        // merge the 4 waves' states; wave w finishes row tile w
        __syncthreads();                       // every wave is done with its V tiles
        if (g == 0) {
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
                sm.m[wave][rt * 16 + p] = m_run[rt];
                sm.l[wave][rt * 16 + p] = l_run[rt];
            }
        }
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
            for (int db = 0; db < DB; ++db) *(f32x4 *)(sm.buf + o_off(wave, rt, db, lane)) = o[rt][db];
        __syncthreads();
        const int rloc = wave * 16 + p;
        float msrc[kMWaves];
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kMWaves; ++w) {
            msrc[w] = sm.m[w][rloc];
            M = fmaxf(M, msrc[w]);
        }
        float L = 0.f;
        f32x4 acc[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kMWaves; ++w) {
            const float sc = msrc[w] == kNegInf ? 0.f : fast_exp2(msrc[w] - M);
            L += sc * sm.l[w][rloc];
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] += sc * *(const f32x4 *)(sm.buf + o_off(w, wave, db, lane));
        }

        // epilogue: the lane's row, channels 16 db + 4 g .. + 3
        const int row = rb * RB + rloc;
        if (row < Rb) {
            const int qi = row / a.G;
            const int qh = kvh * a.G + row % a.G;
            const bool empty = !(L > 0.f);
            const float inv = empty ? 0.f : 1.f / L;
            const float lse2 = empty ? kNegInf : M + fast_log2(L);
            if (whole) {
                uint16_t *op = (uint16_t *)a.out + (q_token(a, b, qi) * a.Hq + qh) * D;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *(u32x2 *)(op + 16 * db + 4 * g) =
                        u32x2{pack2<DT>(acc[db][0] * inv, acc[db][1] * inv),
                              pack2<DT>(acc[db][2] * inv, acc[db][3] * inv)};
                if (g == 0 && a.lse)
                    a.lse[lse_index(a, b, qh, qi)] = empty ? kNegInf : lse2 * kLn2;
            } else {
                const size_t e = (size_t)slot * RB + rloc;   // head_block = 1
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    *(f32x4 *)(a.ws_o + e * D + 16 * db + 4 * g) = acc[db] * inv;
                if (g == 0) a.ws_lse[e] = lse2;
            }
        }
        __syncthreads();                       // the next segment reuses the LDS
    }
};

// One workgroup per CU, one wave per SIMD: each wave keeps 64 rows of
// accumulators and two K/V tiles in registers.

template <int DT, int D, int SCHED, bool PAGED>
__global__ __launch_bounds__(kMWaves * 64)
__attribute__((amdgpu_waves_per_eu(1, 1)))
void split_kv_mfma_kernel(KernelArgs a) {
    using M = Mfma<DT, D, PAGED>;
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
    const bool paged = a.block_table != nullptr;
    const void *fn =
        a.schedule == kBalanced
            ? (paged ? (const void *)&split_kv_mfma_kernel<DT, D, kBalanced, true>
                     : (const void *)&split_kv_mfma_kernel<DT, D, kBalanced, false>)
            : (paged ? (const void *)&split_kv_mfma_kernel<DT, D, kFixed, true>
                     : (const void *)&split_kv_mfma_kernel<DT, D, kFixed, false>);
    return hipLaunchKernel(fn, grid, dim3(kMWaves * 64), kargs, 0, stream);
}

}  // namespace

hipError_t launch_split_mfma(const KernelArgs &a, int dtype, dim3 grid, hipStream_t stream) {
    if (a.row_block != kRowTiles * 16 || a.head_block != 1) return hipErrorInvalidValue;
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
