// Host side of the C ABI declared in include/mxfa.h: argument checks (pure
// host code, run before any HIP call), the partitioning planner, scratch
// management and kernel launches.
#include "mxfa.h"
#include "launch.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

namespace {

using namespace mxfa;

constexpr int kVersion = 100;           // 0.1.0
constexpr int kDefaultCUs = 256;        // MI355X
constexpr int kMaxDevices = 64;
constexpr int kMaxGridYZ = 65535;
constexpr size_t kWsAlign = 256;

// Problem-size checks only; pointers are checked separately.  A paged
// cache has page_size > 0 and kv_cap = max_pages * page_size.
struct Problem {
    int B, Hq, Hkv, D, qLen, kv_cap, causal, dtype;
    int page_size = 0, max_pages = 0, num_pages = 0;
    int new_len = 0;          // tokens appended to every sequence before attention
    // packed batch: cu_q / cu_k offsets on the device, qLen / kv_cap the
    // largest lengths
    const int32_t *cu_q = nullptr, *cu_k = nullptr;
    int total_q = 0, total_k = 0;
    // head dims of q / k and of v / out when they differ (0: both are D)
    int Dk = 0, Dv = 0;
    int dk() const { return Dk ? Dk : D; }
    int dv() const { return Dv ? Dv : D; }
    int dmax() const { return dk() > dv() ? dk() : dv(); }
};

// Scratch of the allocation-free entry point (mxfa_fwd_kvcache_noalloc): a
// fixed array in device memory, one copy per GPU the library is loaded on,
// held until the process ends.  Host code never uses its name as an address
// (on the host it is only a stand-in); the device address of each GPU's copy
// comes from hipGetSymbolAddress, taken once per device with that device
// current, and is what kernels and copies are given.
static __device__ __align__(256) unsigned char scratch[MXFA_NOALLOC_SCRATCH_BYTES];
std::atomic<void *> g_scratch_ptr[kMaxDevices];

thread_local mxfa_plan_t t_last_plan;
thread_local bool t_has_last = false;
thread_local hipEvent_t t_ev_before = nullptr;
thread_local hipEvent_t t_ev_after = nullptr;

std::atomic<int> g_cus[kMaxDevices];   // 0 = not yet queried

bool mul_ok(uint64_t a, uint64_t b, uint64_t *out) {
    return !__builtin_mul_overflow(a, b, out);
}

mxfa_status check_problem(const Problem &p) {
    if (p.B < 0 || p.qLen < 0 || p.kv_cap < 0 || p.Hq <= 0 || p.Hkv <= 0 || p.dk() <= 0 ||
        p.dv() <= 0)
        return MXFA_ERR_INVALID_ARG;
    if (p.Hq % p.Hkv != 0) return MXFA_ERR_INVALID_ARG;
    if (p.causal != 0 && p.causal != 1) return MXFA_ERR_INVALID_ARG;
    if (p.dtype != MXFA_FP16 && p.dtype != MXFA_BF16) return MXFA_ERR_INVALID_ARG;
    // byte sizes of every tensor must be representable
    uint64_t x;
    if (!mul_ok((uint64_t)p.B, (uint64_t)p.kv_cap, &x) || !mul_ok(x, (uint64_t)p.Hkv, &x) ||
        !mul_ok(x, (uint64_t)p.dmax(), &x) || !mul_ok(x, 2, &x) || x > (UINT64_C(1) << 62))
        return MXFA_ERR_INVALID_ARG;
    if (!mul_ok((uint64_t)p.B, (uint64_t)p.qLen, &x) || !mul_ok(x, (uint64_t)p.Hq, &x) ||
        !mul_ok(x, (uint64_t)p.dmax(), &x) || !mul_ok(x, 8, &x) || x > (UINT64_C(1) << 62))
        return MXFA_ERR_INVALID_ARG;
    // head dims: any from 1 to 256 (the matrix-core tiles pad them on chip)
    if (p.dk() > 256 || p.dv() > 256) return MXFA_ERR_UNSUPPORTED;
    if (p.B > kMaxGridYZ) return MXFA_ERR_UNSUPPORTED;
    if (p.page_size > 0) {
        // paged: the pool's byte size must be representable; one page is
        // addressed with 32-bit offsets, so it must stay below 2^30 bytes
        if (!mul_ok((uint64_t)p.num_pages, (uint64_t)p.page_size, &x) ||
            !mul_ok(x, (uint64_t)p.Hkv, &x) || !mul_ok(x, (uint64_t)p.dmax(), &x) ||
            !mul_ok(x, 2, &x) || x > (UINT64_C(1) << 62))
            return MXFA_ERR_INVALID_ARG;
        if ((uint64_t)p.page_size * p.Hkv * p.dmax() * 2 > (UINT64_C(1) << 30))
            return MXFA_ERR_UNSUPPORTED;
        return MXFA_OK;
    }
    // K/V are addressed with 32-bit byte offsets inside one sequence; loads
    // issued ahead may run up to 1024 tokens past the cache, so both the
    // cache and that slack must stay below 2^30 bytes
    if ((uint64_t)p.kv_cap * p.Hkv * p.dmax() * 2 > (UINT64_C(1) << 30))
        return MXFA_ERR_UNSUPPORTED;
    if ((uint64_t)1024 * p.Hkv * p.dmax() * 2 > (UINT64_C(1) << 30)) return MXFA_ERR_UNSUPPORTED;
    return MXFA_OK;
}

// A paged problem: page_size a power of two >= kMinPage (a smaller or
// irregular page is a valid layout the kernels do not implement), the
// logical capacity max_pages * page_size an int, and at least one page when
// sequences may hold tokens.
mxfa_status paged_problem(int B, int Hq, int Hkv, int D, int qLen, int num_pages,
                          int page_size, int max_pages, int causal, int dtype, Problem *out) {
    if (num_pages < 0 || page_size <= 0 || max_pages < 0) return MXFA_ERR_INVALID_ARG;
    if (max_pages > 0 && num_pages == 0) return MXFA_ERR_INVALID_ARG;
    if ((page_size & (page_size - 1)) != 0 || page_size < kMinPage) return MXFA_ERR_UNSUPPORTED;
    if ((int64_t)max_pages * page_size > INT32_MAX) return MXFA_ERR_UNSUPPORTED;
    Problem p{B, Hq, Hkv, D, qLen, max_pages * page_size, causal, dtype};
    p.page_size = page_size;
    p.max_pages = max_pages;
    p.num_pages = num_pages;
    const mxfa_status st = check_problem(p);
    if (st == MXFA_OK) *out = p;
    return st;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// k and v are never read when the cache has no capacity, so they may be NULL.
mxfa_status check_pointers(const void *q, const void *k, const void *v,
                           const int32_t *seqlens, const void *out, const float *lse,
                           int kv_cap) {
    if (!q || !out) return MXFA_ERR_INVALID_ARG;
    if (kv_cap > 0 && (!k || !v)) return MXFA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16))
        return MXFA_ERR_INVALID_ARG;
    if (seqlens && !aligned(seqlens, 4)) return MXFA_ERR_INVALID_ARG;
    if (lse && !aligned(lse, 4)) return MXFA_ERR_INVALID_ARG;
    return MXFA_OK;
}

int next_pow2_le8(int r) { return r <= 1 ? 1 : r <= 2 ? 2 : r <= 4 ? 4 : 8; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// Slot layout of the VALU kernel: whole head groups when Hkv allows it, so
// that a workgroup streams whole token rows of the cache (all heads side by
// side), else one head per workgroup.
// Slot layout of the VALU kernel.  Whole token rows (2 * tpw heads, the
// slots of both wave pairs) stream best on large caches; below 256 MiB of
// K/V (small: true) half that block doubles the streams, so that the share
// floor leaves no workgroup idle on short caches and each output row has
// half the partials to merge: SmallQ MHA q1/q2 calls (32 heads, 1K-4K keys)
// took 12.2-18.7 against 13.7-19.8 us per call (one head per workgroup was
// slower from 3K keys on).
int valu_layout(int Hkv, int D, bool small, int *heads_per_block) {
    const int tpw = 64 / (D / 8);
    if (!small && Hkv % (2 * tpw) == 0) {
        *heads_per_block = 2 * tpw;
        return kHeadsX2;
    }
    if (Hkv % tpw == 0) {
        *heads_per_block = tpw;
        return kHeadsX1;
    }
    *heads_per_block = 1;
    return kTokens;
}

// Partitioning (see launch.h for the two schedules).
//   Fixed partitions: a workgroup serves one (sequence, head block, row block)
//   stream and one partition of `chunk` tokens of it.  The partition length
//   is chosen so that the grid holds about kTargetPerCU workgroups per CU at
//   full length, but no shorter than a floor that keeps the partial results
//   (row_block x (D + 1) floats per head, written once, read once by the
//   merge) a small fraction of the partition's K/V bytes.
//   Balanced: a fixed grid of one or two workgroups per CU (see make_plan),
//   each taking
//   an equal share (at least the same floor) of all streams laid end to end,
//   so ragged batches keep every workgroup equally busy.
// The balanced schedule is used when the planner is free to choose
// (num_splits = 0), the problem needs more than one partition and the batch
// fits the kernel's on-chip length table; a forced num_splits selects fixed
// partitions.  The SmallQ README derives its KV block from the on-chip buffer
// size; here the on-chip tile is fixed per kernel and only the work split is
// planned.
// Channels per row of the partial outputs: the head dim on the VALU path,
// the padded V tile width on the matrix-core path.
int out_tile(const Problem &p, int path) {
    if (path != MXFA_PATH_MFMA) return p.dv();
    int tk, tv;
    mfma_tile_dims(p.dk(), p.dv(), &tk, &tv);
    return tv;
}

struct FullPlan {
    mxfa_plan_t pub;
    int head_blocks, row_blocks, min_share;
    size_t o_bytes, lse_bytes, cum_bytes;
};

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// The partitioning of a problem whose kernel, tile (row block) and head
// block are chosen (pl.path, pl.row_block, pl.layout, pl.rows set): fixed
// partitions or the balanced schedule, the grid and the scratch layout.
// *busy: how many workgroups get work when every sequence holds kv_cap keys.
mxfa_status finish_plan(const Problem &p, long long R, bool odd, int num_splits, int num_cus,
                        mxfa_plan_t pl, int hpb, FullPlan *fp, long long *busy) {
    constexpr int kChunkAlign = 64;
    constexpr int kTargetPerCU = 8;
    // workgroups per CU in the balanced grid: for the VALU kernel one (1-7%
    // faster than two on MHA and GQA-2 decode batches of 0.5-2 GB, 0.5-0.7 us
    // faster on the SmallQ calls, whose merge then reads half as many
    // partials; through pages too, since each step's page is requested a step
    // ahead: paged SmallQ q1/q2 calls 0.6-1.3 us faster, the paged Qwen3-8B
    // batch 336 against 349 us); two for the matrix-core kernel's 16-row
    // variant, one for its 64-row tiles (their LDS and registers fill the CU)
    const int kValuPerCU = 1;
    constexpr int kMfmaPerCU = 1;
    const int row_blocks = R > 0 ? ceil_div(R, pl.row_block) : 1;
    pl.head_block = hpb;
    const int head_blocks = ceil_div(p.Hkv, hpb);
    if ((long long)head_blocks * row_blocks > kMaxGridYZ) return MXFA_ERR_UNSUPPORTED;
    pl.num_cus = num_cus;
    const long long streams = (long long)p.B * head_blocks * row_blocks;
    // the partial-result floor counts the rows a block actually holds
    const int rows_held = (int)(R < pl.row_block ? R : pl.row_block);
    const int min_chunk =
        ceil_div(16 * rows_held > 64 ? 16 * rows_held : 64, kChunkAlign) * kChunkAlign;
    // the balanced share floor: 8 tokens per row held, at least 32.  Measured
    // on the 1023-token SmallQ cases, where the floor decides how many
    // workgroups get work: 14.3 against 17.4 us per call at q1 and 15.8
    // against 18.7 at q2 for 32 tokens against 64 (16 gained nothing more),
    // and 16.3 against 16.7 us at q8 for 64 tokens against 128; on the
    // final kernels 12.1 against 12.7 us at q8 for 64 tokens against 32
    // (4 or 2 tokens per row changed no other SmallQ or small GQA call).
    constexpr int kShareAlign = 32;
    const int min_share = ceil_div(8 * rows_held > 32 ? 8 * rows_held : 32, kShareAlign) *
                          kShareAlign;

    int S, chunk;
    if (p.kv_cap == 0) {
        S = 1;
        chunk = 1;
    } else if (num_splits > 0) {
        S = num_splits > p.kv_cap ? p.kv_cap : num_splits;
        chunk = ceil_div(p.kv_cap, S);
        S = ceil_div(p.kv_cap, chunk);
    } else {
        const long long target = (long long)num_cus * kTargetPerCU;
        long long want = streams > 0 ? (target + streams - 1) / streams : 1;
        const long long smax = (p.kv_cap + min_chunk - 1) / min_chunk;
        if (want > smax) want = smax;
        if (want < 1) want = 1;
        chunk = ceil_div(p.kv_cap, want);
        chunk = ceil_div(chunk, kChunkAlign) * kChunkAlign;
        S = ceil_div(p.kv_cap, chunk);
    }
    long long slots;
    if (num_splits == 0 && S > 1 && p.B <= kMaxBalancedBatch) {
        pl.schedule = kBalanced;
        const int P = num_cus * (pl.path == MXFA_PATH_VALU ? kValuPerCU
                                 : pl.row_block == kMfmaSmallRows && !odd ? 2 : kMfmaPerCU);
        pl.num_splits = P;
        pl.chunk = 0;
        pl.grid_x = P;
        pl.grid_y = 1;
        pl.grid_z = 1;
        pl.combine = 1;
        slots = P + streams;
    } else {
        pl.schedule = kFixed;
        pl.num_splits = S;
        pl.chunk = chunk;
        pl.grid_x = S;
        pl.grid_y = head_blocks * row_blocks;
        pl.grid_z = p.B;
        pl.combine = S > 1 ? 1 : 0;
        slots = streams * S;
    }
    FullPlan f;
    std::memset(&f, 0, sizeof(f));
    if (pl.combine) {
        const size_t entries = (size_t)slots * hpb * pl.row_block;
        f.o_bytes = align_up(entries * out_tile(p, pl.path) * sizeof(float));
        f.lse_bytes = align_up(entries * sizeof(float));
        f.cum_bytes = pl.schedule == kBalanced ? align_up((size_t)(p.B + 2) * sizeof(long long)) : 0;
        pl.workspace_bytes = f.o_bytes + f.lse_bytes + f.cum_bytes;
    }
    f.pub = pl;
    f.head_blocks = head_blocks;
    f.row_blocks = row_blocks;
    f.min_share = min_share;
    // workgroups with work, at most (every sequence at full length)
    if (pl.schedule == kBalanced) {
        const long long T = streams * p.kv_cap;
        long long W = (T + pl.grid_x - 1) / pl.grid_x;
        if (W < min_share) W = min_share;
        const long long nb = (T + W - 1) / W;
        *busy = nb < pl.grid_x ? nb : pl.grid_x;
    } else {
        *busy = streams * S;
    }
    *fp = f;
    return MXFA_OK;
}

mxfa_status make_plan(const Problem &p, int num_splits, int num_cus, FullPlan *fp) {
    mxfa_plan_t pl;
    std::memset(&pl, 0, sizeof(pl));
    if (num_cus <= 0) num_cus = kDefaultCUs;
    const int G = p.Hq / p.Hkv;
    const long long R = (long long)G * p.qLen;
    if (R > INT32_MAX) return MXFA_ERR_UNSUPPORTED;
    pl.rows = (int)R;
    int hpb = 1;
    const bool valu_dims = p.dk() == p.dv() && (p.dk() == 64 || p.dk() == 128);
    const int mfma_min = p.dk() == 128 ? kMfmaMinRows128 : kMfmaMinRows;
    // at exactly the 128-dim threshold, large caches (contiguous or paged)
    // stream faster through the VALU kernel (launch.h records the crossover)
    const uint64_t cache_bytes =
        (uint64_t)p.B * (uint64_t)p.kv_cap * p.Hkv * (uint64_t)(p.dk() + p.dv()) * 2;
    const bool valu_stream = p.dk() == 128 && R == kMfmaMinRows128 &&
                             cache_bytes >= kValuStreamBytes;
    // head dims that are not multiples of 8: 2-byte aligned rows, element
    // loads on the matrix-core kernel's 16-row tiles, one kv head per workgroup
    const bool odd = odd_head_dims(p.dk(), p.dv());
    if ((R >= mfma_min && !valu_stream) || !valu_dims) {
        // many rows per kv head (Q K^T and P V are dense 16-row tiles), or a
        // head shape only the matrix-core kernel's padded tiles hold
        pl.path = MXFA_PATH_MFMA;
        pl.row_block = mfma_row_block(p.dk(), p.dv());
        if (odd || (MXFA_MFMA_SMALL && R <= kMfmaSmallRows && p.dk() <= 128 && p.dv() <= 128))
            pl.row_block = kMfmaSmallRows;
        else if (R <= kMfmaMaxMidRows && p.dk() <= 128 && p.dv() <= 128)
            pl.row_block = (int)((R + kMfmaSmallRows - 1) / kMfmaSmallRows) * kMfmaSmallRows;
        pl.layout = kTokens;
        // two kv heads per workgroup (two waves each) when Hkv is even and
        // one row block holds all rows (decode): the workgroup then reads 512
        // contiguous bytes of every token row instead of 256.  With several
        // row blocks (prefill chunks) every block reads its head's K/V again
        // from the caches, and pairing heads doubles what those re-reads
        // cycle through: a packed chunked-prefill batch fell from 536 to 313
        // TFLOP/s with pairs, so such problems keep one head per workgroup.
        if (!odd && p.Hkv % kMfmaHeads == 0 && R <= pl.row_block) hpb = kMfmaHeads;
    } else {
        pl.path = MXFA_PATH_VALU;
        pl.row_block = next_pow2_le8((int)R);
        pl.layout = valu_layout(p.Hkv, p.D, cache_bytes < kValuStreamBytes, &hpb);
    }
    FullPlan f;
    long long busy = 0;
    const mxfa_status st = finish_plan(p, R, odd, num_splits, num_cus, pl, hpb, &f, &busy);
    if (st != MXFA_OK) return st;
    // Many rows per kv head but few workgroups with work on 64-row tiles
    // (short caches, few sequences or kv heads): 16-row tiles, one kv head
    // per workgroup and two workgroups per CU give four times the row
    // blocks, each re-reading its head's K/V, which on such caches come back
    // from the caches rather than HBM.  Measured against the 64-row plan
    // (bf16, causal drafts of 8 tokens, whole calls): GQA 8 with 2-4
    // sequences at 256-2048 keys 8.1-20.9 against 16.5-39.3 us, one sequence
    // at 8192 keys 23.6 against 30.2 us, the 128-key tiny causal batch 4.4
    // against 6.9 us; equal where the 64-row plan keeps half the CUs busy
    // (4 sequences at 4096 keys, 31.6 us each), and slower past it (4
    // sequences at 8192 keys: 55.7 against 37.1 us; the 32K-key Llama-70B
    // MTP batch keeps every CU busy on 64-row tiles).  A forced partition
    // count keeps the tile the head shape selects.
    if (pl.path == MXFA_PATH_MFMA && num_splits == 0 && !odd && MXFA_MFMA_SMALL &&
        pl.row_block != kMfmaSmallRows && R > kMfmaSmallRows && p.dk() <= 128 &&
        p.dv() <= 128 && 2 * busy <= num_cus) {
        mxfa_plan_t p16 = pl;
        p16.row_block = kMfmaSmallRows;
        FullPlan f16;
        long long busy16 = 0;
        if (finish_plan(p, R, odd, num_splits, num_cus, p16, 1, &f16, &busy16) == MXFA_OK) f = f16;
    }
    *fp = f;
    return MXFA_OK;
}

mxfa_status device_cus(int *cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MXFA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = g_cus[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *cus = c;
            return MXFA_OK;
        }
    }
    int c = 0;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        c <= 0)
        return MXFA_ERR_HIP;
    if (dev >= 0 && dev < kMaxDevices) g_cus[dev].store(c, std::memory_order_relaxed);
    *cus = c;
    return MXFA_OK;
}

// The balanced schedule over N streams that all hold n keys (no
// per-sequence lengths), decided on the host so that neither kernel spends
// its start on it: *w = the share width of the concatenated layout,
// max(ceil(N n / S), min_share); when shares of that width also fit
// floor(S / N) to a stream, *spw = ceil(n / w), and stream st gets shares
// st * spw .. st * spw + spw - 1 of its own, so that no share straddles two
// streams (else *spw = 0 and the streams stay concatenated).  A straddling
// workgroup runs two segments, each with its own start-up and partial
// stores, and on short launches it is the last to finish: the SmallQ MHA
// calls at 1023 and 3000 keys took 1.4-4.0 us less each (q4 kv1023 16.2 ->
// 12.3 us, q8 kv3000 20.7 -> 17.1 us).
void uniform_shares(long long n, long long N, int S, int min_share, int *w, int *spw) {
    const long long wc = (N * n + S - 1) / S;
    *w = (int)(wc < min_share ? min_share : wc);
    *spw = 0;
    if (n <= 0 || N <= 0 || N > S) return;
    const long long k = S / N;
    long long wa = (n + k - 1) / k;
    if (wa < min_share) wa = min_share;
    if (wa == *w) *spw = (int)((n + wa - 1) / wa);
}

// Kernel arguments that describe the cache and the sequences.
KernelArgs cache_args(const void *k, const void *v, const int32_t *seqlens,
                      const int32_t *block_table, const Problem &p) {
    KernelArgs a;
    std::memset(&a, 0, sizeof(a));
    a.k = k;
    a.v = v;
    a.seqlens = seqlens;
    if (p.page_size > 0) {
        a.block_table = block_table;
        a.max_pages = p.max_pages;
        a.num_pages = p.num_pages;
        a.log_page = __builtin_ctz((unsigned)p.page_size);
    }
    a.B = p.B;
    a.Hq = p.Hq;
    a.Hkv = p.Hkv;
    a.D = p.dk();
    a.Dk = p.dk();
    a.Dv = p.dv();
    a.kv_cap = p.kv_cap;
    a.new_len = p.new_len;
    a.cu_q = p.cu_q;
    a.cu_k = p.cu_k;
    a.total_q = p.total_q;
    a.total_k = p.total_k;
    return a;
}

mxfa_status run(const void *q, const void *k, const void *v, const int32_t *seqlens,
                const int32_t *block_table, const void *k_new, const void *v_new, void *out,
                float *lse, const Problem &p, const FullPlan &f, void *ws, hipStream_t stream) {
    const mxfa_plan_t &pl = f.pub;
    KernelArgs a = cache_args(k, v, seqlens, block_table, p);
    a.q = q;
    a.out = out;
    a.lse = lse;
    if (pl.combine) {
        a.ws_o = (float *)ws;
        a.ws_lse = (float *)((char *)ws + f.o_bytes);
        a.ws_cum = f.cum_bytes ? (int *)((char *)ws + f.o_bytes + f.lse_bytes) : nullptr;
    }
    a.qLen = p.qLen;
    a.G = p.Hq / p.Hkv;
    a.R = pl.rows;
    a.causal = p.causal;
    a.head_block = pl.head_block;
    a.head_blocks = f.head_blocks;
    a.row_block = pl.row_block;
    a.row_blocks = f.row_blocks;
    a.schedule = pl.schedule;
    a.chunk = pl.chunk;
    a.S = pl.num_splits;
    a.min_share = f.min_share;
    // fixed partitions of several row blocks per kv head: head block
    // fastest in launch order, so each XCD serves whole kv heads (when the
    // head blocks and the 8 XCDs divide one another)
    a.xcd_heads = pl.schedule == kFixed && f.row_blocks > 1 &&
                  (f.head_blocks % 8 == 0 || 8 % f.head_blocks == 0);
    if (pl.schedule == kBalanced && !a.seqlens && !a.cu_k)
        uniform_shares(p.kv_cap, (long long)p.B * f.head_blocks * f.row_blocks, a.S,
                       a.min_share, &a.uni_w, &a.uni_spw);
    a.qscale = (float)(1.4426950408889634 / std::sqrt((double)p.dk()));
    a.dv_tile = out_tile(p, pl.path);
    const dim3 grid(pl.grid_x, pl.grid_y, pl.grid_z);
    if (p.new_len > 0 && launch_append(a, k_new, v_new, stream) != hipSuccess)
        return MXFA_ERR_HIP;
    if (t_ev_before && hipEventRecord(t_ev_before, stream) != hipSuccess) return MXFA_ERR_HIP;
    const hipError_t e = pl.path == MXFA_PATH_MFMA
                             ? launch_split_mfma(a, p.dtype, grid, stream)
                             : launch_split_valu(a, p.dtype, pl.layout, grid, stream);
    if (e != hipSuccess) return MXFA_ERR_HIP;
    if (t_ev_after && hipEventRecord(t_ev_after, stream) != hipSuccess) return MXFA_ERR_HIP;
    if (pl.combine && launch_combine(a, p.dtype, stream) != hipSuccess) return MXFA_ERR_HIP;
    return MXFA_OK;
}

void record(const mxfa_plan_t &pl) {
    t_last_plan = pl;
    t_has_last = true;
}

// Plan and launch a checked problem.  own_ws: allocate the scratch on the
// stream (stream-ordered) instead of using the caller's.
mxfa_status execute(const void *q, const void *k, const void *v, const int32_t *seqlens,
                    const int32_t *block_table, const void *k_new, const void *v_new,
                    void *out, float *lse, const Problem &p, int num_splits, void *workspace,
                    size_t workspace_bytes, bool own_ws, hipStream_t s) {
    if (!own_ws && workspace && !aligned(workspace, kWsAlign)) return MXFA_ERR_INVALID_ARG;
    int cus = 0;
    mxfa_status st = device_cus(&cus);
    if (st != MXFA_OK) return st;
    FullPlan f;
    st = make_plan(p, num_splits, cus, &f);
    if (st != MXFA_OK) return st;
    void *ws = workspace;
    if (own_ws) {
        ws = nullptr;
        if (f.pub.workspace_bytes > 0 && hipMallocAsync(&ws, f.pub.workspace_bytes, s) != hipSuccess)
            return MXFA_ERR_HIP;
    } else if (f.pub.workspace_bytes > 0 && (!workspace || workspace_bytes < f.pub.workspace_bytes)) {
        return MXFA_ERR_WORKSPACE;
    }
    st = run(q, k, v, seqlens, block_table, k_new, v_new, out, lse, p, f, ws, s);
    if (own_ws && ws && hipFreeAsync(ws, s) != hipSuccess && st == MXFA_OK) st = MXFA_ERR_HIP;
    if (st == MXFA_OK) record(f.pub);
    return st;
}

}  // namespace

extern "C" {

MXFA_API mxfa_status mxfa_plan(int B, int Hq, int Hkv, int D, int qLen, int kv_cap,
                               int causal, int dtype, int num_splits, int num_cus,
                               mxfa_plan_t *plan) {
    if (!plan || num_splits < 0) return MXFA_ERR_INVALID_ARG;
    const Problem p{B, Hq, Hkv, D, qLen, kv_cap, causal, dtype};
    mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    FullPlan f;
    st = make_plan(p, num_splits, num_cus, &f);
    if (st == MXFA_OK) *plan = f.pub;
    return st;
}

MXFA_API mxfa_status mxfa_workspace_size(int B, int Hq, int Hkv, int D, int qLen, int kv_cap,
                                         int causal, int dtype, int num_splits,
                                         size_t *bytes) {
    if (!bytes || num_splits < 0) return MXFA_ERR_INVALID_ARG;
    const Problem p{B, Hq, Hkv, D, qLen, kv_cap, causal, dtype};
    mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != MXFA_OK) return st;
    FullPlan f;
    st = make_plan(p, num_splits, cus, &f);
    if (st != MXFA_OK) return st;
    *bytes = (B == 0 || qLen == 0) ? 0 : f.pub.workspace_bytes;
    return MXFA_OK;
}

MXFA_API mxfa_status mxfa_fwd_kvcache_ws(const void *q, const void *k_cache, const void *v_cache,
                                         const int32_t *cache_seqlens, void *out, float *lse,
                                         int B, int Hq, int Hkv, int D, int qLen, int kv_cap,
                                         int causal, int dtype, int num_splits, void *workspace,
                                         size_t workspace_bytes, void *stream) {
    const Problem p{B, Hq, Hkv, D, qLen, kv_cap, causal, dtype};
    mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    if (num_splits < 0) return MXFA_ERR_INVALID_ARG;
    if (B == 0 || qLen == 0) return MXFA_OK;       // nothing to compute
    st = check_pointers(q, k_cache, v_cache, cache_seqlens, out, lse, kv_cap);
    if (st != MXFA_OK) return st;
    return execute(q, k_cache, v_cache, cache_seqlens, nullptr, nullptr, nullptr, out, lse, p,
                   num_splits, workspace, workspace_bytes, false, (hipStream_t)stream);
}

MXFA_API mxfa_status mxfa_fwd_kvcache(const void *q, const void *k_cache, const void *v_cache,
                                      const int32_t *cache_seqlens, void *out, float *lse,
                                      int B, int Hq, int Hkv, int D, int qLen, int kv_cap,
                                      int causal, int dtype, void *stream) {
    const Problem p{B, Hq, Hkv, D, qLen, kv_cap, causal, dtype};
    mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    if (B == 0 || qLen == 0) return MXFA_OK;
    st = check_pointers(q, k_cache, v_cache, cache_seqlens, out, lse, kv_cap);
    if (st != MXFA_OK) return st;
    return execute(q, k_cache, v_cache, cache_seqlens, nullptr, nullptr, nullptr, out, lse, p,
                   0, nullptr, 0, true, (hipStream_t)stream);
}

MXFA_API mxfa_status mxfa_workspace_size_paged(int B, int Hq, int Hkv, int D, int qLen,
                                               int page_size, int max_pages, int causal,
                                               int dtype, int num_splits, size_t *bytes) {
    if (!bytes || num_splits < 0) return MXFA_ERR_INVALID_ARG;
    Problem p;
    // the plan does not depend on the pool size: any positive page count
    mxfa_status st = paged_problem(B, Hq, Hkv, D, qLen, 1, page_size, max_pages, causal,
                                   dtype, &p);
    if (st != MXFA_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != MXFA_OK) return st;
    FullPlan f;
    st = make_plan(p, num_splits, cus, &f);
    if (st != MXFA_OK) return st;
    *bytes = (B == 0 || qLen == 0) ? 0 : f.pub.workspace_bytes;
    return MXFA_OK;
}

MXFA_API mxfa_status mxfa_fwd_kvcache_paged_ws(
    const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
    const int32_t *cache_seqlens, void *out, float *lse, int B, int Hq, int Hkv, int D,
    int qLen, int num_pages, int page_size, int max_pages, int causal, int dtype,
    int num_splits, void *workspace, size_t workspace_bytes, void *stream) {
    Problem p;
    mxfa_status st = paged_problem(B, Hq, Hkv, D, qLen, num_pages, page_size, max_pages,
                                   causal, dtype, &p);
    if (st != MXFA_OK) return st;
    if (num_splits < 0) return MXFA_ERR_INVALID_ARG;
    if (B == 0 || qLen == 0) return MXFA_OK;
    st = check_pointers(q, k_pages, v_pages, cache_seqlens, out, lse, p.kv_cap);
    if (st != MXFA_OK) return st;
    if (p.kv_cap > 0 && (!block_table || !aligned(block_table, 4))) return MXFA_ERR_INVALID_ARG;
    return execute(q, k_pages, v_pages, cache_seqlens, block_table, nullptr, nullptr, out, lse,
                   p, num_splits, workspace, workspace_bytes, false, (hipStream_t)stream);
}

MXFA_API mxfa_status mxfa_fwd_kvcache_paged(
    const void *q, const void *k_pages, const void *v_pages, const int32_t *block_table,
    const int32_t *cache_seqlens, void *out, float *lse, int B, int Hq, int Hkv, int D,
    int qLen, int num_pages, int page_size, int max_pages, int causal, int dtype,
    void *stream) {
    Problem p;
    mxfa_status st = paged_problem(B, Hq, Hkv, D, qLen, num_pages, page_size, max_pages,
                                   causal, dtype, &p);
    if (st != MXFA_OK) return st;
    if (B == 0 || qLen == 0) return MXFA_OK;
    st = check_pointers(q, k_pages, v_pages, cache_seqlens, out, lse, p.kv_cap);
    if (st != MXFA_OK) return st;
    if (p.kv_cap > 0 && (!block_table || !aligned(block_table, 4))) return MXFA_ERR_INVALID_ARG;
    return execute(q, k_pages, v_pages, cache_seqlens, block_table, nullptr, nullptr, out, lse,
                   p, 0, nullptr, 0, true, (hipStream_t)stream);
}

namespace {

// Shared body of the two appending entry points (p already checked).
mxfa_status fwd_append(const void *q, void *k, void *v, const int32_t *block_table,
                       const void *k_new, const void *v_new, const int32_t *cache_seqlens,
                       void *out, float *lse, Problem p, int new_len, int num_splits,
                       void *workspace, size_t workspace_bytes, hipStream_t s) {
    if (new_len < 0 || num_splits < 0) return MXFA_ERR_INVALID_ARG;
    uint64_t x;
    if (!mul_ok((uint64_t)p.B, (uint64_t)new_len, &x) || !mul_ok(x, (uint64_t)p.Hkv, &x) ||
        !mul_ok(x, (uint64_t)p.dmax(), &x) || !mul_ok(x, 2, &x) || x > (UINT64_C(1) << 62))
        return MXFA_ERR_INVALID_ARG;
    p.new_len = new_len;
    if (p.B == 0) return MXFA_OK;
    const bool appends = new_len > 0 && p.kv_cap > 0;
    if (new_len > 0) {
        // the positions come from cache_seqlens
        if (!cache_seqlens || !aligned(cache_seqlens, 4)) return MXFA_ERR_INVALID_ARG;
        if (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16))
            return MXFA_ERR_INVALID_ARG;
    }
    if (appends && (!k || !v || !aligned(k, 16) || !aligned(v, 16))) return MXFA_ERR_INVALID_ARG;
    if (appends && p.page_size > 0 && (!block_table || !aligned(block_table, 4)))
        return MXFA_ERR_INVALID_ARG;
    if (p.qLen == 0) {
        // no query: only the cache update
        if (!appends) return MXFA_OK;
        const KernelArgs a = cache_args(k, v, cache_seqlens, block_table, p);
        return launch_append(a, k_new, v_new, s) == hipSuccess ? MXFA_OK : MXFA_ERR_HIP;
    }
    mxfa_status st = check_pointers(q, k, v, cache_seqlens, out, lse, p.kv_cap);
    if (st != MXFA_OK) return st;
    if (p.page_size > 0 && p.kv_cap > 0 && (!block_table || !aligned(block_table, 4)))
        return MXFA_ERR_INVALID_ARG;
    return execute(q, k, v, cache_seqlens, block_table, k_new, v_new, out, lse, p, num_splits,
                   workspace, workspace_bytes, workspace == nullptr, s);
}

}  // namespace

MXFA_API mxfa_status mxfa_fwd_kvcache_append(
    const void *q, void *k_cache, void *v_cache, const void *k_new, const void *v_new,
    const int32_t *cache_seqlens, void *out, float *lse, int B, int Hq, int Hkv, int D,
    int qLen, int new_len, int kv_cap, int causal, int dtype, int num_splits, void *workspace,
    size_t workspace_bytes, void *stream) {
    const Problem p{B, Hq, Hkv, D, qLen, kv_cap, causal, dtype};
    const mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    return fwd_append(q, k_cache, v_cache, nullptr, k_new, v_new, cache_seqlens, out, lse, p,
                      new_len, num_splits, workspace, workspace_bytes, (hipStream_t)stream);
}

MXFA_API mxfa_status mxfa_fwd_kvcache_paged_append(
    const void *q, void *k_pages, void *v_pages, const int32_t *block_table,
    const void *k_new, const void *v_new, const int32_t *cache_seqlens, void *out,
    float *lse, int B, int Hq, int Hkv, int D, int qLen, int new_len, int num_pages,
    int page_size, int max_pages, int causal, int dtype, int num_splits, void *workspace,
    size_t workspace_bytes, void *stream) {
    Problem p;
    const mxfa_status st = paged_problem(B, Hq, Hkv, D, qLen, num_pages, page_size, max_pages,
                                         causal, dtype, &p);
    if (st != MXFA_OK) return st;
    return fwd_append(q, k_pages, v_pages, block_table, k_new, v_new, cache_seqlens, out, lse,
                      p, new_len, num_splits, workspace, workspace_bytes, (hipStream_t)stream);
}

MXFA_API mxfa_status mxfa_fwd_varlen(const void *q, const void *k, const void *v,
                                     const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k,
                                     void *out, float *lse, int B, int Hq, int Hkv, int D,
                                     int total_q, int total_k, int max_seqlen_q,
                                     int max_seqlen_k, int causal, int dtype, int num_splits,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    if (total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_splits < 0)
        return MXFA_ERR_INVALID_ARG;
    Problem p{B, Hq, Hkv, D, max_seqlen_q, max_seqlen_k, causal, dtype};
    mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    uint64_t x;
    if (!mul_ok((uint64_t)total_q, (uint64_t)Hq, &x) || !mul_ok(x, (uint64_t)D * 8, &x) ||
        x > (UINT64_C(1) << 62) || !mul_ok((uint64_t)total_k, (uint64_t)Hkv, &x) ||
        !mul_ok(x, (uint64_t)D * 2, &x) || x > (UINT64_C(1) << 62))
        return MXFA_ERR_INVALID_ARG;
    if (B == 0 || max_seqlen_q == 0 || total_q == 0) return MXFA_OK;
    if (!cu_seqlens_q || !cu_seqlens_k || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
        return MXFA_ERR_INVALID_ARG;
    // keys exist only when both the pool and the longest sequence are non-empty
    st = check_pointers(q, k, v, nullptr, out, lse,
                        total_k > 0 && max_seqlen_k > 0 ? max_seqlen_k : 0);
    if (st != MXFA_OK) return st;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.total_q = total_q;
    p.total_k = total_k;
    return execute(q, k, v, nullptr, nullptr, nullptr, nullptr, out, lse, p, num_splits,
                   workspace, workspace_bytes, workspace == nullptr, (hipStream_t)stream);
}

MXFA_API mxfa_status mxfa_workspace_size_dkdv(int B, int Hq, int Hkv, int Dk, int Dv, int qLen,
                                              int kv_cap, int causal, int dtype, int num_splits,
                                              size_t *bytes) {
    if (!bytes || num_splits < 0) return MXFA_ERR_INVALID_ARG;
    Problem p{B, Hq, Hkv, Dk, qLen, kv_cap, causal, dtype};
    p.Dk = Dk;
    p.Dv = Dv;
    mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    int cus = 0;
    st = device_cus(&cus);
    if (st != MXFA_OK) return st;
    FullPlan f;
    st = make_plan(p, num_splits, cus, &f);
    if (st != MXFA_OK) return st;
    *bytes = (B == 0 || qLen == 0) ? 0 : f.pub.workspace_bytes;
    return MXFA_OK;
}

MXFA_API mxfa_status mxfa_fwd_kvcache_dkdv(const void *q, const void *k_cache,
                                           const void *v_cache, const int32_t *cache_seqlens,
                                           void *out, float *lse, int B, int Hq, int Hkv,
                                           int Dk, int Dv, int qLen, int kv_cap, int causal,
                                           int dtype, int num_splits, void *workspace,
                                           size_t workspace_bytes, void *stream) {
    Problem p{B, Hq, Hkv, Dk, qLen, kv_cap, causal, dtype};
    p.Dk = Dk;
    p.Dv = Dv;
    mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    if (num_splits < 0) return MXFA_ERR_INVALID_ARG;
    if (B == 0 || qLen == 0) return MXFA_OK;
    st = check_pointers(q, k_cache, v_cache, cache_seqlens, out, lse, kv_cap);
    if (st != MXFA_OK) return st;
    return execute(q, k_cache, v_cache, cache_seqlens, nullptr, nullptr, nullptr, out, lse, p,
                   num_splits, workspace, workspace_bytes, workspace == nullptr,
                   (hipStream_t)stream);
}

MXFA_API mxfa_status mxfa_fwd_kvcache_noalloc(const void *q, const void *k_cache,
                                              const void *v_cache, const int32_t *cache_seqlens,
                                              void *out, float *lse, int B, int Hq, int Hkv,
                                              int D, int qLen, int kv_cap, int causal, int dtype,
                                              int num_splits, void *stream) {
    const Problem p{B, Hq, Hkv, D, qLen, kv_cap, causal, dtype};
    mxfa_status st = check_problem(p);
    if (st != MXFA_OK) return st;
    if (num_splits < 0) return MXFA_ERR_INVALID_ARG;
    if (B == 0 || qLen == 0) return MXFA_OK;
    st = check_pointers(q, k_cache, v_cache, cache_seqlens, out, lse, kv_cap);
    if (st != MXFA_OK) return st;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MXFA_ERR_HIP;
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!ptr) {
        // first call on this device (it is current): the device address of
        // its copy of the array; a concurrent first call stores the same value
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return MXFA_ERR_HIP;
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
    // execute() plans first and returns MXFA_ERR_WORKSPACE, before any launch,
    // when the plan needs more scratch than the array holds
    return execute(q, k_cache, v_cache, cache_seqlens, nullptr, nullptr, nullptr, out, lse, p,
                   num_splits, ptr, MXFA_NOALLOC_SCRATCH_BYTES, false, (hipStream_t)stream);
}

MXFA_API mxfa_status mxfa_last_plan(mxfa_plan_t *plan) {
    if (!plan || !t_has_last) return MXFA_ERR_INVALID_ARG;
    *plan = t_last_plan;
    return MXFA_OK;
}

MXFA_API mxfa_status mxfa_set_timing_events(void *before, void *after) {
    if ((before == nullptr) != (after == nullptr)) return MXFA_ERR_INVALID_ARG;
    t_ev_before = (hipEvent_t)before;
    t_ev_after = (hipEvent_t)after;
    return MXFA_OK;
}

MXFA_API const char *mxfa_status_string(int status) {
    switch (status) {
    case MXFA_OK: return "MXFA_OK: success";
    case MXFA_ERR_INVALID_ARG: return "MXFA_ERR_INVALID_ARG: invalid argument";
    case MXFA_ERR_UNSUPPORTED:
        return "MXFA_ERR_UNSUPPORTED: unsupported shape (head dims up to 256; see mxfa.h for "
               "the other limits)";
    case MXFA_ERR_WORKSPACE: return "MXFA_ERR_WORKSPACE: workspace missing or too small";
    case MXFA_ERR_HIP: return "MXFA_ERR_HIP: HIP runtime error";
    default: return "unknown mxfa status";
    }
}

MXFA_API int mxfa_version(void) { return kVersion; }

}  // extern "C"
