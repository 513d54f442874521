/*
 * mxfa.h -- C ABI of the MI355X (gfx950) split-KV decode-attention library.
 *
 * One call computes FlashAttention-style forward attention for a few query
 * tokens against a KV cache:
 *
 *     O = softmax(Q K^T / sqrt(D) [+ causal mask]) V          per query head,
 *
 * the formula of the interface section of "SmallQ FlashAttention for Ascend
 * 910B" (scale 1/sqrt(headDim)), evaluated the FlashAttention way described
 * in the ops-transformer articles (CSDN "FlashAttention in CANN
 * ops-transformer", section on the FlashAttention idea and online softmax;
 * mhpn.cn "ops-transformer source walk-through", section on tiling and
 * online softmax): K/V are streamed tile by tile while a running maximum m,
 * a running sum l and a rescaled output accumulator are kept on chip.  The
 * KV sequence of every (batch, kv head) is cut into partitions that run in
 * parallel ("M1 Split-KV decode" on the MXFlashAttn package page, use-case
 * and verified-capability sections); a second kernel merges the partial
 * (O, log-sum-exp) results.  Grouped-query attention: query head h reads kv
 * head h / (Hq / Hkv) (GQA ratios as on the MXFlashAttn package page).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are contiguous, row-major, in device memory, all 16-bit tensors in
 * the same dtype (mxfa_dtype):
 *     q, out        [B, qLen, Hq, D]
 *     k_cache,
 *     v_cache       [B, kv_cap, Hkv, D]      kv_cap = cache capacity per sequence
 *     cache_seqlens int32 [B]                valid length n_b of each sequence;
 *                                            NULL means n_b = kv_cap for all b
 *     lse           float32 [B, Hq, qLen]    natural log of sum_j exp(s_j), s_j
 *                                            the scaled scores; may be NULL
 * Values of cache_seqlens are read on the device and clamped to [0, kv_cap].
 * Cache slots at or beyond n_b are never read.  With causal = 1 the mask is
 * aligned to the bottom right: query row i (0 <= i < qLen) sees key j iff
 * j <= i + n_b - qLen.  A row that sees no key gets O = 0 and lse = -inf.
 * Arithmetic: 16-bit inputs, fp32 accumulation (as the SmallQ README's
 * algorithm notes prescribe), output rounded to nearest-even.
 *
 * Supported: any head dim D from 1 to 256 (the SmallQ README's support
 * range allows any head dim of at least 1 and was verified at 64, 128, 256
 * and the 192 / 128 split of MLA heads; its algorithm notes pad the head dim
 * on chip).  64 and 128 are the fast paths; other dims are padded to a tile
 * of 64, 128, 192 or 256 channels inside the matrix-core kernel, and dims
 * that are not multiples of 8 (rows only 2-byte aligned) are read and
 * written element by element.  Any Hq that is a multiple of Hkv; fp16 and
 * bf16.  Other shapes return MXFA_ERR_UNSUPPORTED; nothing falls back
 * silently.
 *
 * Ownership and threading: the caller owns every buffer.  The library keeps
 * no pointer after a call returns.  Its only mutable state is the
 * thread-local record of the last plan, the thread-local timing hook (see
 * mxfa_set_timing_events) and a per-device cache of the CU count, so calls
 * from several host threads are safe.
 *
 * Asynchrony: kernels are enqueued on `stream` (a hipStream_t passed as
 * void *, so that this header needs no HIP header and plain C and ctypes
 * callers can use it; NULL = the null stream) and the call returns without
 * synchronising, as in the SmallQ FlashAttention README's "aclnn API call"
 * section, where the caller synchronises the stream.  The status
 * covers argument checks and launch errors only; faults during execution
 * surface at the caller's next synchronisation.
 *
 * Errors: all argument checks run before any HIP runtime call.  On any
 * status other than MXFA_OK nothing has been enqueued and out / lse are
 * untouched.
 */
#ifndef MXFA_H_
#define MXFA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MXFA_API __attribute__((visibility("default")))
#else
#define MXFA_API
#endif

typedef enum {
    MXFA_OK = 0,
    MXFA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, bad enum */
    MXFA_ERR_UNSUPPORTED = 2,   /* valid request outside the supported shapes  */
    MXFA_ERR_WORKSPACE = 3,     /* caller workspace missing or too small       */
    MXFA_ERR_HIP = 4            /* HIP runtime error (allocation or launch)    */
} mxfa_status;

typedef enum { MXFA_FP16 = 0, MXFA_BF16 = 1 } mxfa_dtype;

typedef enum {
    MXFA_PATH_VALU = 0,         /* vector-ALU split kernel (few rows per kv head) */
    MXFA_PATH_MFMA = 1          /* matrix-core split kernel (>= 4 rows per kv head at head dim 128, or >= 5
                                   when the caches, contiguous or paged, hold 256 MiB or more; >= 8 at
                                   64; head dims other than 64 / 128) */
} mxfa_path;

/* How a call is carried out.  The analogue of the dispatch record the
 * MXFlashAttn package exposes through get_last_dispatch_info (package page,
 * "Python API" section): which kernel path ran and with what partitioning. */
typedef struct {
    int path;            /* mxfa_path */
    int layout;          /* VALU path: 0 = each wave slot a different kv head,
                            2 head groups per workgroup; 1 = same with one
                            head group; 2 = one kv head per workgroup */
    int schedule;        /* 0 = fixed partitions of `chunk` tokens per stream;
                            1 = balanced: grid_x workgroups share the
                            concatenated KV streams of all sequences equally */
    int rows;            /* R = (Hq / Hkv) * qLen query rows per kv head */
    int row_block;       /* query rows handled by one workgroup and kv head:
                            VALU 1, 2, 4 or 8; matrix-core 16, 32, 48 or 64 */
    int head_block;      /* kv heads handled by one workgroup */
    int num_splits;      /* fixed: KV partitions per stream at kv_cap;
                            balanced: number of workgroups */
    int chunk;           /* fixed: tokens per partition (the last one may be
                            shorter); balanced: 0 (set on the device) */
    int grid_x, grid_y, grid_z;  /* split-kernel grid: partitions, head blocks x row blocks, batch */
    int combine;         /* 1 if the merge kernel runs, else 0 */
    int num_cus;         /* compute units the plan was made for */
    size_t workspace_bytes;      /* device scratch the call needs (0 without merge) */
} mxfa_plan_t;

/* Split-KV decode attention, library-managed scratch: the FlashAttention-
 * compatible attention-with-KV-cache entry point of the MXFlashAttn package
 * page (Python API section), computed by the split-KV decode method its
 * use-case section describes.  The arguments carry what the Python API keeps
 * in tensor shapes, so the cache capacity kv_cap (the cache's second
 * dimension) is passed explicitly: without it the batch stride of a
 * contiguous [B, kv_cap, Hkv, D] cache is unknown.
 * Partial results of the KV partitions go to a scratch buffer taken from
 * the stream-ordered allocator (hipMallocAsync / hipFreeAsync on `stream`).
 * Arguments as in the conventions above.  causal is 0 or 1; dtype is an
 * mxfa_dtype.  Pointers q, k_cache, v_cache, out must be 16-byte aligned;
 * lse and cache_seqlens 4-byte aligned.  B == 0 or qLen == 0 is a no-op.
 * Returns MXFA_OK, or an error status as listed in mxfa_status. */
MXFA_API mxfa_status mxfa_fwd_kvcache(const void *q, const void *k_cache,
                                      const void *v_cache,
                                      const int32_t *cache_seqlens, void *out,
                                      float *lse, int B, int Hq, int Hkv,
                                      int D, int qLen, int kv_cap, int causal,
                                      int dtype, void *stream);

/* Same computation with caller-provided scratch and an optional forced
 * partition count: the execute half of the two-phase call of the SmallQ
 * FlashAttention README's "aclnn API call" section (query the workspace size,
 * allocate it, then enqueue the operator on a stream and let the caller
 * synchronise).  num_splits = 0 lets the planner choose; a positive value
 * asks for that many KV partitions per (batch, kv head) at kv_cap (clamped to
 * [1, kv_cap]).  workspace must be 256-byte aligned and hold at least the
 * number of bytes mxfa_workspace_size reports for the same arguments; it may
 * be NULL when that number is 0.  The caller must not use the workspace for
 * anything else until the work enqueued on `stream` has finished.
 * Returns MXFA_ERR_WORKSPACE if the workspace is missing or too small. */
MXFA_API mxfa_status mxfa_fwd_kvcache_ws(const void *q, const void *k_cache,
                                         const void *v_cache,
                                         const int32_t *cache_seqlens,
                                         void *out, float *lse, int B, int Hq,
                                         int Hkv, int D, int qLen, int kv_cap,
                                         int causal, int dtype, int num_splits,
                                         void *workspace,
                                         size_t workspace_bytes, void *stream);

/* Scratch bytes that mxfa_fwd_kvcache_ws needs for these arguments, written
 * to *bytes: the size-query half of the two-phase call of the SmallQ
 * FlashAttention README's "aclnn API call" section, which likewise writes the
 * size through a pointer and returns a status.  It takes the execute call's
 * problem arguments (causal and dtype included) and checks them the same
 * way, so a bad problem is reported before any allocation.  The
 * partitioning depends on the CU count of the current HIP
 * device, so call it with the device current that will run the attention
 * (the count is queried once per device and cached).  Returns the same
 * validation statuses as the attention calls (checked before any HIP call),
 * or MXFA_ERR_HIP if the device query fails. */
MXFA_API mxfa_status mxfa_workspace_size(int B, int Hq, int Hkv, int D,
                                         int qLen, int kv_cap, int causal,
                                         int dtype, int num_splits,
                                         size_t *bytes);

/* Largest scratch, in bytes, that mxfa_fwd_kvcache_noalloc can use. */
#define MXFA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Allocation-free variant of mxfa_fwd_kvcache_ws, for callers that cannot
 * allocate device memory during the call: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments and
 * results as mxfa_fwd_kvcache_ws without the workspace arguments: the
 * partial results go to a fixed scratch array of MXFA_NOALLOC_SCRATCH_BYTES
 * in device memory that the library holds on every GPU it runs on until the
 * process ends.  The call makes no allocation (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device looks up that
 * device's array once.  A problem whose plan needs more scratch than the
 * array holds (mxfa_workspace_size reports the need) returns
 * MXFA_ERR_WORKSPACE before anything is enqueued.  Nothing in the array has
 * to start at zero: every value a call reads was written earlier in the same
 * call.  All calls on one GPU share the array, so calls that may overlap on
 * one GPU (other streams, other host threads) race on it and must be
 * ordered by the caller. */
MXFA_API mxfa_status mxfa_fwd_kvcache_noalloc(const void *q, const void *k_cache,
                                              const void *v_cache,
                                              const int32_t *cache_seqlens, void *out,
                                              float *lse, int B, int Hq, int Hkv, int D,
                                              int qLen, int kv_cap, int causal, int dtype,
                                              int num_splits, void *stream);

/* Paged KV cache.  The MXFlashAttn sdist README lists a paged KV cache among
 * its implemented layouts (capability matrix) and describes its kernel as a
 * split-KV paged decode kernel (introduction); the pages give no layout, so
 * the FlashAttention-style block table is taken:
 *     k_pages,
 *     v_pages      [num_pages, page_size, Hkv, D]   a pool of fixed-size pages
 *     block_table  int32 [B, max_pages]             page of each block of
 *                                                   page_size tokens
 * Token j of sequence b is row j % page_size of page
 * block_table[b * max_pages + j / page_size]; every other convention is the
 * contiguous cache's with kv_cap = max_pages * page_size (cache_seqlens are
 * clamped to it; NULL means every sequence holds max_pages * page_size
 * tokens).  Only the entries for blocks below n_b are read; they should lie
 * in [0, num_pages), and a value outside is clamped into it (never an
 * out-of-pool access).  Pages may be shared between sequences and appear in
 * any order.  page_size must be a power of two >= 16 (else
 * MXFA_ERR_UNSUPPORTED; page_size <= 0 is MXFA_ERR_INVALID_ARG) and one
 * page must stay below 2^30 bytes; max_pages * page_size must fit an int.
 * block_table must be non-NULL and 4-byte aligned when max_pages > 0, and
 * num_pages >= 1 then.  The plan, scratch and merge are those of the
 * contiguous cache with the same kv_cap. */
MXFA_API mxfa_status mxfa_fwd_kvcache_paged(const void *q, const void *k_pages,
                                            const void *v_pages,
                                            const int32_t *block_table,
                                            const int32_t *cache_seqlens,
                                            void *out, float *lse, int B, int Hq,
                                            int Hkv, int D, int qLen,
                                            int num_pages, int page_size,
                                            int max_pages, int causal, int dtype,
                                            void *stream);

/* Paged cache with caller-provided scratch and an optional forced partition
 * count; num_splits and workspace as for mxfa_fwd_kvcache_ws, the size from
 * mxfa_workspace_size_paged. */
MXFA_API mxfa_status mxfa_fwd_kvcache_paged_ws(
    const void *q, const void *k_pages, const void *v_pages,
    const int32_t *block_table, const int32_t *cache_seqlens, void *out,
    float *lse, int B, int Hq, int Hkv, int D, int qLen, int num_pages,
    int page_size, int max_pages, int causal, int dtype, int num_splits,
    void *workspace, size_t workspace_bytes, void *stream);

/* Scratch bytes that mxfa_fwd_kvcache_paged_ws needs (the pool size does not
 * enter); the size query of the two-phase call (SmallQ FlashAttention README,
 * "aclnn API call"), with the validation and device rules of
 * mxfa_workspace_size. */
MXFA_API mxfa_status mxfa_workspace_size_paged(int B, int Hq, int Hkv, int D,
                                               int qLen, int page_size,
                                               int max_pages, int causal,
                                               int dtype, int num_splits,
                                               size_t *bytes);

/* In-call KV append, then attention.  The MXFlashAttn package page names a
 * FlashAttention-compatible attention-with-KV-cache entry point (Python API
 * section) and its sdist README lists paged KV append as verified
 * (capability matrix); the FlashAttention rule is taken:
 *     k_new, v_new  [B, new_len, Hkv, D]   this step's keys and values
 * token t of sequence b is written to cache position cache_seqlens[b] + t
 * (cache_seqlens clamped to [0, kv_cap]); positions at or past kv_cap are
 * dropped.  Attention then runs as in mxfa_fwd_kvcache over
 * min(cache_seqlens[b] + new_len, kv_cap) keys, so the causal mask aligns the
 * last query row with the last new token when new_len == qLen.
 * cache_seqlens is required (non-NULL) when new_len > 0 and is not modified;
 * the caller advances it.  k_cache / v_cache are written in place (the
 * append kernel runs on `stream` before the attention kernels).  With
 * qLen == 0 only the cache is updated.  new_len < 0 is MXFA_ERR_INVALID_ARG;
 * k_new / v_new must be 16-byte aligned.  workspace == NULL: scratch from the
 * stream-ordered allocator; otherwise as for mxfa_fwd_kvcache_ws (size from
 * mxfa_workspace_size).  num_splits as for mxfa_fwd_kvcache_ws. */
MXFA_API mxfa_status mxfa_fwd_kvcache_append(
    const void *q, void *k_cache, void *v_cache, const void *k_new,
    const void *v_new, const int32_t *cache_seqlens, void *out, float *lse,
    int B, int Hq, int Hkv, int D, int qLen, int new_len, int kv_cap,
    int causal, int dtype, int num_splits, void *workspace,
    size_t workspace_bytes, void *stream);

/* The same over a paged cache: position pos of sequence b is row
 * pos % page_size of page block_table[b * max_pages + pos / page_size]
 * (the block table must already name the pages the new tokens land in);
 * workspace size from mxfa_workspace_size_paged. */
MXFA_API mxfa_status mxfa_fwd_kvcache_paged_append(
    const void *q, void *k_pages, void *v_pages, const int32_t *block_table,
    const void *k_new, const void *v_new, const int32_t *cache_seqlens,
    void *out, float *lse, int B, int Hq, int Hkv, int D, int qLen,
    int new_len, int num_pages, int page_size, int max_pages, int causal,
    int dtype, int num_splits, void *workspace, size_t workspace_bytes,
    void *stream);

/* Packed (variable-length) batch.  The MXFlashAttn package page lists a
 * flash_attn_varlen_func entry point (Python API section) and its sdist README
 * a varlen layout (capability matrix), without a layout; the FlashAttention
 * one is taken:
 *     q, out        [total_q, Hq, D]      queries of all sequences, packed
 *     k, v          [total_k, Hkv, D]     keys / values, packed
 *     cu_seqlens_q,
 *     cu_seqlens_k  int32 [B + 1]         device offsets: sequence b owns rows
 *                                         cu[b] .. cu[b + 1] - 1
 *     lse           float32 [Hq, total_q] (may be NULL)
 * Sequence b has q_b = cu_seqlens_q[b + 1] - cu_seqlens_q[b] queries and
 * n_b = cu_seqlens_k[b + 1] - cu_seqlens_k[b] keys; offsets are clamped into
 * [0, total] and the lengths to max_seqlen_q / max_seqlen_k, which the caller
 * passes as upper bounds (they size the plan; max_seqlen_k * Hkv * D * 2
 * must stay below 2^30 bytes).  With causal = 1, query i of sequence b sees
 * key j iff j <= i + n_b - q_b.  Rows of out past every sequence's queries
 * are not written.  workspace == NULL: scratch from the stream-ordered
 * allocator; otherwise at least mxfa_workspace_size(B, Hq, Hkv, D,
 * max_seqlen_q, max_seqlen_k, causal, dtype, num_splits) bytes. */
MXFA_API mxfa_status mxfa_fwd_varlen(const void *q, const void *k,
                                     const void *v,
                                     const int32_t *cu_seqlens_q,
                                     const int32_t *cu_seqlens_k, void *out,
                                     float *lse, int B, int Hq, int Hkv, int D,
                                     int total_q, int total_k, int max_seqlen_q,
                                     int max_seqlen_k, int causal, int dtype,
                                     int num_splits, void *workspace,
                                     size_t workspace_bytes, void *stream);

/* Different head dims for keys and values (the DeepSeek V3 MLA heads the
 * SmallQ README verifies: K side 192, V side 128): q [B, qLen, Hq, Dk],
 * k_cache [B, kv_cap, Hkv, Dk], v_cache [B, kv_cap, Hkv, Dv], out
 * [B, qLen, Hq, Dv]; the scale is 1/sqrt(Dk).  Dk and Dv are any dims from
 * 1 to 256.  workspace == NULL: scratch from the stream-ordered allocator;
 * otherwise at least mxfa_workspace_size_dkdv bytes.  Otherwise as
 * mxfa_fwd_kvcache_ws. */
MXFA_API mxfa_status mxfa_fwd_kvcache_dkdv(const void *q, const void *k_cache,
                                           const void *v_cache,
                                           const int32_t *cache_seqlens,
                                           void *out, float *lse, int B, int Hq,
                                           int Hkv, int Dk, int Dv, int qLen,
                                           int kv_cap, int causal, int dtype,
                                           int num_splits, void *workspace,
                                           size_t workspace_bytes, void *stream);

/* Scratch bytes mxfa_fwd_kvcache_dkdv needs: the size query of the two-phase
 * call (SmallQ FlashAttention README, "aclnn API call"), rules as
 * mxfa_workspace_size. */
MXFA_API mxfa_status mxfa_workspace_size_dkdv(int B, int Hq, int Hkv, int Dk,
                                              int Dv, int qLen, int kv_cap,
                                              int causal, int dtype,
                                              int num_splits, size_t *bytes);

/* The plan (path, partitioning, grid, scratch size) for a problem on a
 * device with num_cus compute units (num_cus <= 0 means 256, an MI355X):
 * the record mxfa_last_plan reports for a call with the same arguments
 * (num_splits as for mxfa_fwd_kvcache_ws, since a forced partition count
 * changes the plan; causal and dtype are checked like the execute call's).
 * It lets a caller see before launching which kernel a problem takes, the
 * purpose get_last_dispatch_info serves after the fact on the MXFlashAttn
 * package page (Python API section).  Pure host code: makes no HIP runtime
 * call, so it works without a GPU. */
MXFA_API mxfa_status mxfa_plan(int B, int Hq, int Hkv, int D, int qLen,
                               int kv_cap, int causal, int dtype,
                               int num_splits, int num_cus, mxfa_plan_t *plan);

/* The plan of the last successful attention call made by this host thread:
 * the analogue of get_last_dispatch_info on the MXFlashAttn package page
 * (Python API section), whose C500 usage section asks to check which kernel
 * ran before trusting a throughput figure.
 * Returns MXFA_ERR_INVALID_ARG if plan is NULL or no call has succeeded on
 * this thread yet. */
MXFA_API mxfa_status mxfa_last_plan(mxfa_plan_t *plan);

/* Timing hook for benchmarks (no passage of the pages defines it).  After this call, every attention call made by
 * this host thread records the HIP event `before` on its stream immediately
 * before the split-KV kernel is enqueued and `after` immediately after it, so
 * hipEventElapsedTime(before, after) is that kernel's duration alone (the
 * merge kernel is excluded).  The events (hipEvent_t) are created and owned
 * by the caller and must stay valid while the hook is set.  Passing NULL for
 * both turns the hook off; passing exactly one NULL returns
 * MXFA_ERR_INVALID_ARG.  A failed event record makes the attention call
 * return MXFA_ERR_HIP. */
MXFA_API mxfa_status mxfa_set_timing_events(void *before, void *after);

/* Measurement helper, not part of attention: enqueues on `stream` one
 * streaming read of `bytes` bytes at `src` in 16-byte buffer loads by
 * num_cus * 2 workgroups of 256 threads (num_cus <= 0 means 256), each
 * streaming its own contiguous share, consecutive lanes reading consecutive
 * chunks.  nontemporal = 1 uses the
 * cache policy of the attention kernels' K/V loads (the nt bit), 0 the
 * default policy.  bytes / (duration between HIP events around the call) is
 * the practical HBM read ceiling the attention kernels are compared with.
 * src: device, 16-byte aligned, 0 < bytes <= 2^31, bytes a multiple of 16.
 * sink: one device uint32 the kernel writes only if the xor of all the data
 * equals a fixed pattern (it keeps the loads from being optimised away).
 * Returns MXFA_ERR_INVALID_ARG for a bad argument (num_cus > 4096 included),
 * MXFA_ERR_HIP if the launch fails. */
MXFA_API mxfa_status mxfa_read_probe(const void *src, size_t bytes,
                                     int nontemporal, uint32_t *sink,
                                     int num_cus, void *stream);

/* Static, human-readable text for a status value (never NULL).  It takes an
 * int so that any value, also one outside mxfa_status, can be passed across
 * the C ABI; unknown values get a generic text.  Explicit errors instead of a
 * silent fallback follow the limits section of the MXFlashAttn package page. */
MXFA_API const char *mxfa_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
MXFA_API int mxfa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFA_H_ */
