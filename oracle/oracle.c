/*
 * Float64 CPU oracle for single-token (decode) grouped-query attention over a
 * paged fp16 KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check
 * and the bench's CPU-baseline leg load this code.  It shares no source,
 * header, table or helper with the GPU library, and includes none of its
 * headers.
 *
 * What it computes is the plain definition, with no blocking, fusion or
 * reordering beyond it:
 *
 *  - Page-table gather (vllm-metal kernels page, cf-1.com/news/5525226,
 *    section "什么是 Paged Attention"): token t of sequence s lives in
 *    physical page block_tables[s][t / bs], slot t mod bs.  Pool layout
 *    [num_blocks][Hkv][bs][D], fp16.
 *  - GQA grouping (same page, section "Metal 并行模型", and the voxtral.c
 *    page, dpshk.com/news/5521762, section "单 token attention 内核"): the
 *    G = Hq/Hkv query heads of a group share one KV head; query head h reads
 *    KV head h / G (consecutive heads form a group).
 *  - Softmax attention over every token t < L: z_t = scale * (q . k_t),
 *    out = sum_t exp(z_t - max z) v_t / sum_t exp(z_t - max z), computed in
 *    two passes (max, then exp-sum and weighted sum), float64 throughout.
 *    The log2-space folding that the vllm-metal page describes (section
 *    "GQA 解码内核的四个提速技巧", item 1) changes no value: 2^(z log2 e) = e^z.
 *  - Split-KV partials (same section, item 4): for each partition i of P
 *    tokens, m_i is the partition's maximum score in log2 units (max z times
 *    log2 e), l_i the partition's exp-sum relative to that maximum (a plain
 *    sum, not its log), and o_i the partition's softmax-weighted V average
 *    normalised by its own l_i.
 *  - Merge of partials: M = max m_i, w_i = l_i 2^(m_i - M),
 *    out = sum_i w_i o_i / sum_i w_i.
 *  - Several query tokens per sequence (the vllm-metal page, section "什么是
 *    Paged Attention", names a unified paged variable-length kernel for
 *    prefill and speculative decoding; the pages give no formula, so the
 *    plain causal reading is taken): sequence s contributes qlen_s =
 *    cu_q[s+1] - cu_q[s] query rows, packed at rows cu_q[s] .. cu_q[s+1]-1;
 *    its cache holds all L_s tokens, the new ones last, so query j sits at
 *    position L_s - qlen_s + j and attends to the tokens t < L_s - qlen_s +
 *    j + 1 (itself and everything before it).  A row with no such token is
 *    zeros.
 *
 * fp16 values widen to double exactly (decoded from their bits below); so do
 * the other element types of the *_dt entry points (the voxtral.c page,
 * dpshk.com/news/5521762, keeps an fp32 KV cache as the fallback of its fp16
 * one): bf16 (the upper half of an IEEE binary32) and fp32.  q, K and V share
 * one element type.
 * Build with -O2 -ffp-contract=off and no fast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_LOG2E 1.44269504088896340735992468100189214

/* IEEE 754 binary16 -> double, exactly: sign, 5-bit exponent (bias 15),
 * 10-bit fraction; exponent 0 is subnormal (no implicit 1), 31 is inf/NaN. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);               /* frac * 2^-10 * 2^-14 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 -> double, exactly: the 16 bits are the upper half of a binary32. */
double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

typedef struct {
    const void *q, *k, *v;
    int dtype;                      /* element type of q, k, v: 0 fp16, 1 bf16, 2 fp32 */
    const int32_t *block_tables, *seq_lens;
    const int32_t *cu_q;            /* variable-length queries only: [S + 1] */
    int S, Hq, Hkv, D, bs, max_blocks;
    long long num_blocks;
    double scale;
    int P, NP;                      /* partials only */
    double *out;                    /* [S][Hq][D] */
    double *m, *l, *o;              /* partials: [S][Hq][NP], [S][Hq][NP], [S][Hq][NP][D] */
    int nthreads, tid;
    int status;
} job_t;

/* Element idx of an array of the job's element type, widened to double. */
static double elem(const job_t *J, const void *base, long long idx)
{
    if (J->dtype == 1) return oracle_bf16_to_double(((const uint16_t *)base)[idx]);
    if (J->dtype == 2) return (double)((const float *)base)[idx];
    return oracle_half_to_double(((const uint16_t *)base)[idx]);
}

/* Element offset of (block, kv head g, slot j, dim 0) in a pool. */
static long long row_ptr(long long block, int g, int j, int Hkv, int bs, int D)
{
    return (((block * Hkv + g) * (long long)bs + j) * (long long)D);
}

/* Element offset of the query vector of packed query row r, head h. */
static long long q_row(const job_t *J, long long r, int h)
{
    return (r * J->Hq + h) * J->D;
}

/* KV head read by query head h. */
static int kv_head(const job_t *J, int h)
{
    int G = J->Hq / J->Hkv;
    int g = h / G;
    return g;
}

/* Scores z_t for t in [t0, t1) of query vector qrow against sequence s's keys
 * of KV head g.  Returns 0, or -1 when a page id is outside the pool. */
static int scores(const job_t *J, long long qrow, int s, int g, int t0, int t1, double *z)
{
    for (int t = t0; t < t1; ++t) {
        long long b = J->block_tables[(long long)s * J->max_blocks + t / J->bs];
        if (b < 0 || b >= J->num_blocks) return -1;
        long long krow = row_ptr(b, g, t % J->bs, J->Hkv, J->bs, J->D);
        double dot = 0.0;
        for (int d = 0; d < J->D; ++d)
            dot += elem(J, J->q, qrow + d) * elem(J, J->k, krow + d);
        z[t - t0] = J->scale * dot;
    }
    return 0;
}

/* Softmax-weighted average of V over tokens [t0, t1) with scores z, relative
 * to the maximum score zmax.  Writes sum_t e_t v_t / sum_t e_t into res and
 * returns the exp-sum sum_t e_t (e_t = exp(z_t - zmax)). */
static double weighted_v(const job_t *J, int s, int g, int t0, int t1, const double *z,
                         double zmax, double *acc, double *res)
{
    double sum = 0.0;
    for (int d = 0; d < J->D; ++d) acc[d] = 0.0;
    for (int t = t0; t < t1; ++t) {
        long long b = J->block_tables[(long long)s * J->max_blocks + t / J->bs];
        long long vrow = row_ptr(b, g, t % J->bs, J->Hkv, J->bs, J->D);
        double e = exp(z[t - t0] - zmax);
        sum += e;
        for (int d = 0; d < J->D; ++d) acc[d] += e * elem(J, J->v, vrow + d);
    }
    for (int d = 0; d < J->D; ++d) res[d] = acc[d] / sum;
    return sum;
}

static void *attention_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    int maxL = 0;
    for (int s = 0; s < J->S; ++s) if (J->seq_lens[s] > maxL) maxL = J->seq_lens[s];
    double *z = (double *)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)J->D);
    if (!z || !acc) { J->status = -2; free(z); free(acc); return NULL; }
    long long rows = (long long)J->S * J->Hq;
    for (long long r = J->tid; r < rows; r += J->nthreads) {
        int s = (int)(r / J->Hq), h = (int)(r % J->Hq);
        int L = J->seq_lens[s];
        double *dst = J->out + r * J->D;
        if (L <= 0) {                       /* empty sequence: defined as zeros */
            for (int d = 0; d < J->D; ++d) dst[d] = 0.0;
            continue;
        }
        if (scores(J, q_row(J, s, h), s, kv_head(J, h), 0, L, z) != 0) { J->status = -1; break; }
        double zmax = -INFINITY;            /* pass 1: the maximum score */
        for (int t = 0; t < L; ++t) if (z[t] > zmax) zmax = z[t];
        weighted_v(J, s, kv_head(J, h), 0, L, z, zmax, acc, dst);   /* pass 2 */
    }
    free(z);
    free(acc);
    return NULL;
}

static void *partials_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    double *z = (double *)malloc(sizeof(double) * (size_t)J->P);
    double *acc = (double *)malloc(sizeof(double) * (size_t)J->D);
    if (!z || !acc) { J->status = -2; free(z); free(acc); return NULL; }
    long long rows = (long long)J->S * J->Hq;
    for (long long r = J->tid; r < rows; r += J->nthreads) {
        int s = (int)(r / J->Hq);
        int h = (int)(r % J->Hq);
        int L = J->seq_lens[s];
        int nparts = (L + J->P - 1) / J->P;
        for (int i = 0; i < nparts && i < J->NP; ++i) {
            int t0 = i * J->P;
            int t1 = t0 + J->P < L ? t0 + J->P : L;
            if (scores(J, q_row(J, s, h), s, kv_head(J, h), t0, t1, z) != 0) { J->status = -1; goto done; }
            double zmax = -INFINITY;
            for (int t = t0; t < t1; ++t) if (z[t - t0] > zmax) zmax = z[t - t0];
            long long pi = r * J->NP + i;
            J->l[pi] = weighted_v(J, s, kv_head(J, h), t0, t1, z, zmax, acc, J->o + pi * J->D);
            J->m[pi] = ORACLE_LOG2E * zmax;
        }
    }
done:
    free(z);
    free(acc);
    return NULL;
}

/* Variable-length queries: rows are (packed query row, head); query row
 * cu_q[s] + j of sequence s attends to the tokens before position
 * L_s - qlen_s + j + 1. */
static void *varlen_worker(void *arg)
{
    job_t *J = (job_t *)arg;
    int maxL = 0;
    for (int s = 0; s < J->S; ++s) if (J->seq_lens[s] > maxL) maxL = J->seq_lens[s];
    double *z = (double *)malloc(sizeof(double) * (size_t)(maxL > 0 ? maxL : 1));
    double *acc = (double *)malloc(sizeof(double) * (size_t)J->D);
    if (!z || !acc) { J->status = -2; free(z); free(acc); return NULL; }
    long long k = 0;                        /* running (row, head) index */
    for (int s = 0; s < J->S; ++s) {
        int L = J->seq_lens[s];
        int qlen = J->cu_q[s + 1] - J->cu_q[s];
        for (int j = 0; j < qlen; ++j) {
            long long row = J->cu_q[s] + j;
            int lim = L - qlen + j + 1;     /* tokens visible to this query */
            if (lim > L) lim = L;
            for (int h = 0; h < J->Hq; ++h, ++k) {
                if (k % J->nthreads != J->tid) continue;
                double *dst = J->out + (row * J->Hq + h) * J->D;
                if (lim <= 0) {
                    for (int d = 0; d < J->D; ++d) dst[d] = 0.0;
                    continue;
                }
                if (scores(J, q_row(J, row, h), s, kv_head(J, h), 0, lim, z) != 0) {
                    J->status = -1;
                    goto done;
                }
                double zmax = -INFINITY;
                for (int t = 0; t < lim; ++t) if (z[t] > zmax) zmax = z[t];
                weighted_v(J, s, kv_head(J, h), 0, lim, z, zmax, acc, dst);
            }
        }
    }
done:
    free(z);
    free(acc);
    return NULL;
}

static int run_jobs(job_t *base, int nthreads, void *(*fn)(void *))
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    job_t jobs[256];
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = *base;
        jobs[i].nthreads = nthreads;
        jobs[i].tid = i;
        jobs[i].status = 0;
    }
    for (int i = 1; i < nthreads; ++i)
        if (pthread_create(&th[i], NULL, fn, &jobs[i]) != 0) return -3;
    fn(&jobs[0]);
    int st = jobs[0].status;
    for (int i = 1; i < nthreads; ++i) {
        pthread_join(th[i], NULL);
        if (jobs[i].status != 0) st = jobs[i].status;
    }
    return st;
}

/* out[S][Hq][D] = softmax attention of every query head over its sequence's
 * paged K/V.  Returns 0, -1 if a page id falls outside [0, num_blocks), -2 on
 * allocation failure. */
int oracle_paged_attention_dt(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *block_tables, const int32_t *seq_lens,
                              int S, int Hq, int Hkv, int D, int bs, int max_blocks,
                              long long num_blocks, double scale, int dtype, double *out,
                              int nthreads)
{
    if (dtype < 0 || dtype > 2) return -4;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.dtype = dtype;
    J.q = q; J.k = k_cache; J.v = v_cache;
    J.block_tables = block_tables; J.seq_lens = seq_lens;
    J.S = S; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.bs = bs; J.max_blocks = max_blocks;
    J.num_blocks = num_blocks; J.scale = scale; J.out = out;
    return run_jobs(&J, nthreads, attention_worker);
}

int oracle_paged_attention(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                           const int32_t *block_tables, const int32_t *seq_lens,
                           int S, int Hq, int Hkv, int D, int bs, int max_blocks,
                           long long num_blocks, double scale, double *out, int nthreads)
{
    return oracle_paged_attention_dt(q, k_cache, v_cache, block_tables, seq_lens, S, Hq, Hkv, D,
                                     bs, max_blocks, num_blocks, scale, 0, out, nthreads);
}

/* Per-partition triples for partitions i < ceil(L/P) (and i < NP); entries of
 * partitions past a sequence's end are left as they were. */
int oracle_partials_dt(const void *q, const void *k_cache, const void *v_cache,
                       const int32_t *block_tables, const int32_t *seq_lens,
                       int S, int Hq, int Hkv, int D, int bs, int max_blocks,
                       long long num_blocks, double scale, int P, int NP, int dtype,
                       double *m, double *l, double *o, int nthreads)
{
    if (P <= 0 || NP <= 0 || dtype < 0 || dtype > 2) return -4;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.dtype = dtype;
    J.q = q; J.k = k_cache; J.v = v_cache;
    J.block_tables = block_tables; J.seq_lens = seq_lens;
    J.S = S; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.bs = bs; J.max_blocks = max_blocks;
    J.num_blocks = num_blocks; J.scale = scale; J.P = P; J.NP = NP;
    J.m = m; J.l = l; J.o = o;
    return run_jobs(&J, nthreads, partials_worker);
}

int oracle_partials(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                    const int32_t *block_tables, const int32_t *seq_lens,
                    int S, int Hq, int Hkv, int D, int bs, int max_blocks,
                    long long num_blocks, double scale, int P, int NP,
                    double *m, double *l, double *o, int nthreads)
{
    return oracle_partials_dt(q, k_cache, v_cache, block_tables, seq_lens, S, Hq, Hkv, D, bs,
                              max_blocks, num_blocks, scale, P, NP, 0, m, l, o, nthreads);
}

/* out[total_q][Hq][D] for variable-length queries: sequence s has the query
 * rows cu_q[s] .. cu_q[s+1]-1 (packed [total_q][Hq][D] fp16) and its cache
 * holds L = seq_lens[s] tokens including them; row j attends causally (see
 * the header).  Same return codes as oracle_paged_attention. */
int oracle_paged_varlen_dt(const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_tables, const int32_t *seq_lens, const int32_t *cu_q,
                           int S, int Hq, int Hkv, int D, int bs, int max_blocks,
                           long long num_blocks, double scale, int dtype, double *out, int nthreads)
{
    if (dtype < 0 || dtype > 2) return -4;
    job_t J;
    memset(&J, 0, sizeof(J));
    J.dtype = dtype;
    J.q = q; J.k = k_cache; J.v = v_cache;
    J.block_tables = block_tables; J.seq_lens = seq_lens; J.cu_q = cu_q;
    J.S = S; J.Hq = Hq; J.Hkv = Hkv; J.D = D; J.bs = bs; J.max_blocks = max_blocks;
    J.num_blocks = num_blocks; J.scale = scale; J.out = out;
    return run_jobs(&J, nthreads, varlen_worker);
}

int oracle_paged_varlen(const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                        const int32_t *block_tables, const int32_t *seq_lens, const int32_t *cu_q,
                        int S, int Hq, int Hkv, int D, int bs, int max_blocks,
                        long long num_blocks, double scale, double *out, int nthreads)
{
    return oracle_paged_varlen_dt(q, k_cache, v_cache, block_tables, seq_lens, cu_q, S, Hq, Hkv, D,
                                  bs, max_blocks, num_blocks, scale, 0, out, nthreads);
}

/* Merge per-partition triples of every (s, h) into out[S][Hq][D]. */
void oracle_merge(const double *m, const double *l, const double *o, const int32_t *seq_lens,
                  int S, int Hq, int D, int P, int NP, double *out)
{
    for (long long r = 0; r < (long long)S * Hq; ++r) {
        int L = seq_lens[r / Hq];
        int nparts = (L + P - 1) / P;
        if (nparts > NP) nparts = NP;
        double *dst = out + r * D;
        for (int d = 0; d < D; ++d) dst[d] = 0.0;
        if (nparts <= 0) continue;
        double M = -INFINITY;
        for (int i = 0; i < nparts; ++i) if (m[r * NP + i] > M) M = m[r * NP + i];
        double wsum = 0.0;
        for (int i = 0; i < nparts; ++i) {
            double w = l[r * NP + i] * exp2(m[r * NP + i] - M);
            wsum += w;
            for (int d = 0; d < D; ++d) dst[d] += w * o[(r * NP + i) * D + d];
        }
        for (int d = 0; d < D; ++d) dst[d] /= wsum;
    }
}
