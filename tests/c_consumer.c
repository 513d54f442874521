/*
 * A plain C99 caller of the mxfa C ABI, with no Python and no torch in the
 * process: it reads one problem from a file, runs it through the two-phase
 * call of the SmallQ FlashAttention README ("aclnn API call" section: query
 * the workspace size, allocate it, enqueue on a stream, synchronise) and
 * writes the results to a second file, which the tests compare with the
 * fp64 oracle.  With the planner's partition count it also runs the call
 * with library-managed scratch and requires the same bits.
 *
 *     c_consumer <problem file> <result file>
 *
 * Problem file: int32 header[16] = {magic 0x4146584d, B, Hq, Hkv, D, qLen,
 * kv_cap, causal, dtype, has_seqlens, num_splits, page_size (0: contiguous
 * cache), max_pages, num_pages, 0, 0}, then q, k, v as 16-bit elements
 * (contiguous [B, kv_cap, Hkv, D] caches, or [num_pages, page_size, Hkv, D]
 * pools), then cache_seqlens (int32 [B], if has_seqlens) and the block table
 * (int32 [B, max_pages], if paged).
 * Result file: int32 status, int32 plan[13] (mxfa_plan_t's int fields in
 * order), int64 workspace bytes, then out (16-bit [B, qLen, Hq, D]) and lse
 * (float32 [B, Hq, qLen]).
 * Exit status: 0 on success, 1 on a library error status, 2 on bad usage or
 * file errors, 3 on a HIP runtime error, 4 if the two entry points differ.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "mxfa.h"

#define MAGIC 0x4146584d

static void hip_check(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        fprintf(stderr, "c_consumer: %s: %s\n", what, hipGetErrorString(e));
        exit(3);
    }
}

static void *read_block(FILE *f, size_t bytes) {
    void *p = malloc(bytes ? bytes : 1);
    if (!p || fread(p, 1, bytes, f) != bytes) {
        fprintf(stderr, "c_consumer: short problem file\n");
        exit(2);
    }
    return p;
}

static void *to_device(const void *host, size_t bytes) {
    void *d = NULL;
    if (bytes == 0) return NULL;
    hip_check(hipMalloc(&d, bytes), "hipMalloc");
    hip_check(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
    return d;
}

int main(int argc, char **argv) {
    int32_t h[16];
    FILE *f;
    if (argc != 3) {
        fprintf(stderr, "usage: c_consumer <problem file> <result file>\n");
        return 2;
    }
    f = fopen(argv[1], "rb");
    if (!f || fread(h, sizeof h, 1, f) != 1 || h[0] != MAGIC) {
        fprintf(stderr, "c_consumer: cannot read a problem header from %s\n", argv[1]);
        return 2;
    }
    {
        const int B = h[1], Hq = h[2], Hkv = h[3], D = h[4], qLen = h[5], kv_cap = h[6];
        const int causal = h[7], dtype = h[8], has_seqlens = h[9], num_splits = h[10];
        const int page_size = h[11], max_pages = h[12], num_pages = h[13];
        const int paged = page_size > 0;
        const size_t q_bytes = (size_t)B * qLen * Hq * D * 2;
        const size_t kv_rows = paged ? (size_t)num_pages * page_size : (size_t)B * kv_cap;
        const size_t kv_bytes = kv_rows * Hkv * D * 2;
        const size_t lse_bytes = (size_t)B * Hq * qLen * 4;
        void *hq = read_block(f, q_bytes), *hk = read_block(f, kv_bytes), *hv = read_block(f, kv_bytes);
        void *hsl = has_seqlens ? read_block(f, (size_t)B * 4) : NULL;
        void *hbt = paged ? read_block(f, (size_t)B * max_pages * 4) : NULL;
        void *q, *k, *v, *out, *out2, *ws = NULL;
        int32_t *sl, *bt;
        float *lse, *lse2;
        hipStream_t stream;
        size_t ws_bytes = 0;
        mxfa_status st;
        mxfa_plan_t plan;
        int32_t status, plan_fields[13];
        int64_t ws64;
        unsigned char *o1, *o2;
        int differ = 0;
        fclose(f);

        q = to_device(hq, q_bytes);
        k = to_device(hk, kv_bytes);
        v = to_device(hv, kv_bytes);
        sl = (int32_t *)to_device(hsl, has_seqlens ? (size_t)B * 4 : 0);
        bt = (int32_t *)to_device(hbt, paged ? (size_t)B * max_pages * 4 : 0);
        hip_check(hipMalloc(&out, q_bytes ? q_bytes : 16), "hipMalloc out");
        hip_check(hipMalloc(&out2, q_bytes ? q_bytes : 16), "hipMalloc out");
        hip_check(hipMalloc((void **)&lse, lse_bytes ? lse_bytes : 16), "hipMalloc lse");
        hip_check(hipMalloc((void **)&lse2, lse_bytes ? lse_bytes : 16), "hipMalloc lse");
        hip_check(hipStreamCreate(&stream), "hipStreamCreate");

        /* phase one: the scratch size for exactly these arguments */
        st = paged ? mxfa_workspace_size_paged(B, Hq, Hkv, D, qLen, page_size, max_pages, causal,
                                               dtype, num_splits, &ws_bytes)
                   : mxfa_workspace_size(B, Hq, Hkv, D, qLen, kv_cap, causal, dtype, num_splits,
                                         &ws_bytes);
        if (st == MXFA_OK && ws_bytes) hip_check(hipMalloc(&ws, ws_bytes), "hipMalloc workspace");
        /* phase two: enqueue on the stream, then synchronise */
        if (st == MXFA_OK)
            st = paged ? mxfa_fwd_kvcache_paged_ws(q, k, v, bt, sl, out, lse, B, Hq, Hkv, D, qLen,
                                                   num_pages, page_size, max_pages, causal, dtype,
                                                   num_splits, ws, ws_bytes, stream)
                       : mxfa_fwd_kvcache_ws(q, k, v, sl, out, lse, B, Hq, Hkv, D, qLen, kv_cap,
                                             causal, dtype, num_splits, ws, ws_bytes, stream);
        if (st != MXFA_OK) {
            fprintf(stderr, "c_consumer: %s\n", mxfa_status_string(st));
            return 1;
        }
        hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize");
        memset(&plan, 0, sizeof plan);
        mxfa_last_plan(&plan);

        o1 = (unsigned char *)malloc(q_bytes + lse_bytes + 1);
        o2 = (unsigned char *)malloc(q_bytes + lse_bytes + 1);
        if (!o1 || !o2) return 2;
        hip_check(hipMemcpy(o1, out, q_bytes, hipMemcpyDeviceToHost), "hipMemcpy out");
        hip_check(hipMemcpy(o1 + q_bytes, lse, lse_bytes, hipMemcpyDeviceToHost), "hipMemcpy lse");

        /* the library-managed entry point: same plan, so the same bits */
        if (num_splits == 0) {
            st = paged ? mxfa_fwd_kvcache_paged(q, k, v, bt, sl, out2, lse2, B, Hq, Hkv, D, qLen,
                                                num_pages, page_size, max_pages, causal, dtype,
                                                stream)
                       : mxfa_fwd_kvcache(q, k, v, sl, out2, lse2, B, Hq, Hkv, D, qLen, kv_cap,
                                          causal, dtype, stream);
            if (st != MXFA_OK) {
                fprintf(stderr, "c_consumer: %s\n", mxfa_status_string(st));
                return 1;
            }
            hip_check(hipStreamSynchronize(stream), "hipStreamSynchronize");
            hip_check(hipMemcpy(o2, out2, q_bytes, hipMemcpyDeviceToHost), "hipMemcpy out");
            hip_check(hipMemcpy(o2 + q_bytes, lse2, lse_bytes, hipMemcpyDeviceToHost),
                      "hipMemcpy lse");
            differ = memcmp(o1, o2, q_bytes + lse_bytes) != 0;
        }

        f = fopen(argv[2], "wb");
        if (!f) return 2;
        status = (int32_t)st;
        plan_fields[0] = plan.path;
        plan_fields[1] = plan.layout;
        plan_fields[2] = plan.schedule;
        plan_fields[3] = plan.rows;
        plan_fields[4] = plan.row_block;
        plan_fields[5] = plan.head_block;
        plan_fields[6] = plan.num_splits;
        plan_fields[7] = plan.chunk;
        plan_fields[8] = plan.grid_x;
        plan_fields[9] = plan.grid_y;
        plan_fields[10] = plan.grid_z;
        plan_fields[11] = plan.combine;
        plan_fields[12] = plan.num_cus;
        ws64 = (int64_t)ws_bytes;
        if (fwrite(&status, 4, 1, f) != 1 || fwrite(plan_fields, 4, 13, f) != 13 ||
            fwrite(&ws64, 8, 1, f) != 1 || fwrite(o1, 1, q_bytes + lse_bytes, f) != q_bytes + lse_bytes) {
            fprintf(stderr, "c_consumer: cannot write %s\n", argv[2]);
            return 2;
        }
        fclose(f);
        printf("c_consumer: %s, B=%d Hq=%d Hkv=%d D=%d qLen=%d %s, path %d, %d partitions, "
               "workspace %lld bytes%s\n",
               mxfa_status_string(st), B, Hq, Hkv, D, qLen, paged ? "paged" : "contiguous",
               plan.path, plan.num_splits, (long long)ws_bytes,
               num_splits == 0 ? (differ ? ", entry points DIFFER" : ", entry points agree") : "");
        if (differ) return 4;

        hip_check(hipFree(q), "hipFree");
        hip_check(hipFree(k), "hipFree");
        hip_check(hipFree(v), "hipFree");
        if (sl) hip_check(hipFree(sl), "hipFree");
        if (bt) hip_check(hipFree(bt), "hipFree");
        if (ws) hip_check(hipFree(ws), "hipFree");
        hip_check(hipFree(out), "hipFree");
        hip_check(hipFree(out2), "hipFree");
        hip_check(hipFree(lse), "hipFree");
        hip_check(hipFree(lse2), "hipFree");
        hip_check(hipStreamDestroy(stream), "hipStreamDestroy");
        free(hq); free(hk); free(hv); free(hsl); free(hbt); free(o1); free(o2);
    }
    return 0;
}
