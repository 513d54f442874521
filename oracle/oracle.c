/*
 * oracle.c -- plain fp64 CPU reference for decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness oracle for the GPU
 * library; it shares no code with it.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it.  Nothing on the product
 * path may call into it.
 *
 * What it computes (the plain definition, no tiling, no online rescaling, no
 * KV splits):
 *
 *   O = softmax(Q K^T / sqrt(headDim)) V
 *
 * as written in the interface section of the "SmallQ FlashAttention for
 * Ascend 910B" README, with the scale 1/sqrt(d) that the ops-transformer
 * article uses in its integration example.  Grouped-query attention (the GQA
 * ratios 2/4/8 listed under verified capabilities on the MXFlashAttn package
 * page) maps query head h to kv head floor(h / G), G = Hq / Hkv: the group of
 * G consecutive query heads shares one kv head.  A causal mask is aligned to
 * the bottom right: query row i (of qLen) sees key j iff j <= i + n - qLen,
 * where n is the sequence's valid cache length, so the last query row sees
 * every valid key.  The pages give no alignment rule for qLen != kvLen; this
 * is the reading taken.
 *
 * Everything is evaluated in double precision from the exact values of the
 * 16-bit inputs:
 *   1. decode q, k, v from IEEE binary16 / bfloat16 bit patterns (subnormals
 *      included) to double, exactly;
 *   2. s_j = (1/sqrt(D)) * sum_d q_d k_jd for every visible key j;
 *   3. m = max_j s_j; w_j = exp(s_j - m); l = sum_j w_j  (two-pass form);
 *   4. O_d = sum_j w_j v_jd / l;  lse = m + log(l)  (natural log);
 *   5. a row with no visible key gets O = 0 and lse = -inf.
 * Valid lengths come from cache_seqlens (clamped to [0, kv_cap]); a NULL
 * cache_seqlens means every sequence uses the whole cache.  Cache slots at or
 * beyond the valid length are never read.
 *
 * Layouts (all contiguous, row-major):
 *   q, out : [B, qLen, Hq, D]      k, v : [B, kv_cap, Hkv, D]
 *   lse    : [B, Hq, qLen]         cache_seqlens : int32 [B]
 * Keys and values may have different head dims (the SmallQ README's support
 * range lists DeepSeek V3 MLA heads, K side 192 and V side 128):
 * mxo_attention_dkdv takes q, k with Dk channels and v, out with Dv; the
 * scale is then 1/sqrt(Dk), the dimension the dot product runs over.
 *
 * Planted-mistake builds: compiling with -DMXO_MUTANT=k (k >= 1) introduces
 * one deliberate, plausible error so that the test suite can show its pins
 * catch it.  The default build (MXO_MUTANT undefined or 0) has none.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef MXO_MUTANT
#define MXO_MUTANT 0
#endif

#define MXO_FP16 0
#define MXO_BF16 1

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double mxo_fp16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    else if (e == 31)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(1024 + f), e - 25);     /* (1 + f/2^10) 2^(e-15) */
    return sign ? -mag : mag;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double mxo_bf16_to_f64(uint16_t b)
{
    const int sign = (b >> 15) & 1;
    const int e = (b >> 7) & 0xff;
    const int f = b & 0x7f;
    double mag;
    if (e == 0)
        mag = ldexp((double)f, -133);                /* subnormal: f * 2^-133 */
    else if (e == 255)
        mag = f ? NAN : INFINITY;
    else
        mag = ldexp((double)(128 + f), e - 134);     /* (1 + f/2^7) 2^(e-127) */
    return sign ? -mag : mag;
}

static double decode(uint16_t x, int dtype)
{
    return dtype == MXO_BF16 ? mxo_bf16_to_f64(x) : mxo_fp16_to_f64(x);
}

typedef struct {
    const uint16_t *q, *k, *v;
    const int32_t *seqlens;
    int B, Hq, Hkv, Dk, Dv, qLen, kv_cap, causal, dtype;
} problem_t;

static int valid_len(const problem_t *p, int b)
{
    int n = p->seqlens ? p->seqlens[b] : p->kv_cap;
    if (n < 0) n = 0;
    if (n > p->kv_cap) n = p->kv_cap;
    return n;
}

/* One output row (b, h, i).  scratch holds kv_cap doubles (scores) plus Dk
 * doubles (the decoded query row). */
static void attend_row(const problem_t *p, int b, int h, int i,
                       double *o_row, double *lse_out, double *scratch)
{
    const int Dk = p->Dk, Dv = p->Dv;
    const int G = p->Hq / p->Hkv;
#if MXO_MUTANT == 1
    const int hk = h % p->Hkv;          /* wrong GQA head mapping */
#else
    const int hk = h / G;
#endif
    const int n = valid_len(p, b);
    int last = n - 1;                   /* highest visible key index */
    if (p->causal) {
#if MXO_MUTANT == 2
        const int c = i;                /* top-left aligned mask */
#else
        const int c = i + n - p->qLen;  /* bottom-right aligned mask */
#endif
        if (c < last) last = c;
    }
    if (last < 0) {                     /* no visible key */
        for (int d = 0; d < Dv; ++d) o_row[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }
    double *s = scratch;
    double *qd = scratch + p->kv_cap;
    const int64_t qoff = (((int64_t)b * p->qLen + i) * p->Hq + h) * Dk;
    for (int d = 0; d < Dk; ++d) qd[d] = decode(p->q[qoff + d], p->dtype);

#if MXO_MUTANT == 3
    const double scale = 1.0 / (double)Dk;         /* wrong scale */
#else
    const double scale = 1.0 / sqrt((double)Dk);
#endif
    /* Pass 1: scores and their maximum. */
    double m = -INFINITY;
    for (int j = 0; j <= last; ++j) {
        const int64_t koff = (((int64_t)b * p->kv_cap + j) * p->Hkv + hk) * Dk;
        double acc = 0.0;
#if MXO_MUTANT == 4
        for (int d = 0; d < Dk - 1; ++d)           /* dropped last channel */
#else
        for (int d = 0; d < Dk; ++d)
#endif
            acc += qd[d] * decode(p->k[koff + d], p->dtype);
        s[j] = scale * acc;
        if (s[j] > m) m = s[j];
    }
    /* Pass 2: softmax weights, their sum and the weighted sum of V rows. */
    for (int d = 0; d < Dv; ++d) o_row[d] = 0.0;
    double l = 0.0;
    for (int j = 0; j <= last; ++j) {
#if MXO_MUTANT == 5
        const int jv = (j + 1 <= last) ? j + 1 : j; /* off-by-one V row */
#else
        const int jv = j;
#endif
        const double w = exp(s[j] - m);
        l += w;
        const int64_t voff = (((int64_t)b * p->kv_cap + jv) * p->Hkv + hk) * Dv;
        for (int d = 0; d < Dv; ++d)
            o_row[d] += w * decode(p->v[voff + d], p->dtype);
    }
#if MXO_MUTANT == 6
    /* forgot to normalise by l */
    *lse_out = m + log(l);
#elif MXO_MUTANT == 7
    for (int d = 0; d < Dv; ++d) o_row[d] /= l;
    *lse_out = log(l);                              /* dropped the max term */
#else
    for (int d = 0; d < Dv; ++d) o_row[d] /= l;
    *lse_out = m + log(l);
#endif
#if MXO_MUTANT == 8
    /* transposed operand: K and V swapped in the product */
    {
        const int Dm = Dk < Dv ? Dk : Dv;
        double l2 = 0.0;
        for (int d = 0; d < Dv; ++d) o_row[d] = 0.0;
        for (int j = 0; j <= last; ++j) {
            const double w = exp(s[j] - m);
            l2 += w;
            const int64_t off = (((int64_t)b * p->kv_cap + j) * p->Hkv + hk) * Dk;
            for (int d = 0; d < Dm; ++d)
                o_row[d] += w * decode(p->k[off + d], p->dtype);
        }
        for (int d = 0; d < Dv; ++d) o_row[d] /= l2;
    }
#endif
}

static int check_args(const problem_t *p)
{
    if (!p->q || !p->k || !p->v) return 1;
    if (p->B < 0 || p->qLen < 0 || p->Hq <= 0 || p->Hkv <= 0 || p->Dk <= 0 || p->Dv <= 0 ||
        p->kv_cap < 0)
        return 1;
    if (p->Hq % p->Hkv) return 1;
    if (p->dtype != MXO_FP16 && p->dtype != MXO_BF16) return 1;
    return 0;
}

/* Full attention with key / value head dims Dk / Dv: out [B,qLen,Hq,Dv] and
 * lse [B,Hq,qLen] in double.  nthreads <= 0 lets OpenMP choose.  Returns 0
 * on success, 1 on bad args, 2 if scratch memory could not be allocated. */
int mxo_attention_dkdv(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const int32_t *cache_seqlens, int B, int Hq, int Hkv, int Dk,
                       int Dv, int qLen, int kv_cap, int causal, int dtype,
                       double *out, double *lse, int nthreads)
{
    problem_t p = {q, k, v, cache_seqlens, B, Hq, Hkv, Dk, Dv, qLen, kv_cap,
                   causal ? 1 : 0, dtype};
    if (check_args(&p) || !out || !lse) return 1;
    const int64_t nrows = (int64_t)B * Hq * qLen;
    int fail = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(|: fail)
#endif
    {
        double *scratch = (double *)malloc(sizeof(double) * ((size_t)kv_cap + Dk));
        if (!scratch) {
            fail = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int64_t r = 0; r < nrows; ++r) {
                const int i = (int)(r % qLen);
                const int h = (int)((r / qLen) % Hq);
                const int b = (int)(r / ((int64_t)qLen * Hq));
                attend_row(&p, b, h, i,
                           out + (((int64_t)b * qLen + i) * Hq + h) * Dv,
                           lse + r, scratch);
            }
            free(scratch);
        }
    }
    return fail ? 2 : 0;
}

/* Full attention with one head dim D for q, k, v and out. */
int mxo_attention(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                  const int32_t *cache_seqlens, int B, int Hq, int Hkv, int D,
                  int qLen, int kv_cap, int causal, int dtype,
                  double *out, double *lse, int nthreads)
{
    return mxo_attention_dkdv(q, k, v, cache_seqlens, B, Hq, Hkv, D, D, qLen, kv_cap,
                              causal, dtype, out, lse, nthreads);
}

/* Selected rows only: rows holds nrows triples (b, h, i); out_rows is
 * [nrows, D] and lse_rows [nrows].  Used where the full problem is too large
 * for the CPU but individual rows can be checked one by one. */
int mxo_attention_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                       const int32_t *cache_seqlens, int B, int Hq, int Hkv,
                       int D, int qLen, int kv_cap, int causal, int dtype,
                       const int32_t *rows, int nrows, double *out_rows,
                       double *lse_rows, int nthreads)
{
    problem_t p = {q, k, v, cache_seqlens, B, Hq, Hkv, D, D, qLen, kv_cap,
                   causal ? 1 : 0, dtype};
    if (check_args(&p) || !rows || nrows < 0 || !out_rows || !lse_rows) return 1;
    for (int r = 0; r < nrows; ++r) {
        const int b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
        if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= qLen) return 1;
    }
    int fail = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(|: fail)
#endif
    {
        double *scratch = (double *)malloc(sizeof(double) * ((size_t)kv_cap + D));
        if (!scratch) {
            fail = 1;
        } else {
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (int r = 0; r < nrows; ++r)
                attend_row(&p, rows[3 * r], rows[3 * r + 1], rows[3 * r + 2],
                           out_rows + (int64_t)r * D, lse_rows + r, scratch);
            free(scratch);
        }
    }
    return fail ? 2 : 0;
}

int mxo_mutant_id(void) { return MXO_MUTANT; }
