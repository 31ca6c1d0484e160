/* Host sanitizer driver for the float64 oracle (oracle/oracle.c): every
 * entry point on seeded random shapes, each buffer allocated to its exact
 * size, so AddressSanitizer reports any read or write past an array and
 * UndefinedBehaviorSanitizer any undefined arithmetic.  Built and run by
 * tests/test_sanitizers.py; exits 0 when every call returns 0. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_paged_attention_dt(const void *q, const void *k, const void *v, const int32_t *bt,
                              const int32_t *sl, int S, int Hq, int Hkv, int D, int bs,
                              int max_blocks, long long num_blocks, double scale, int dtype,
                              double *out, int nthreads);
int oracle_partials_dt(const void *q, const void *k, const void *v, const int32_t *bt,
                       const int32_t *sl, int S, int Hq, int Hkv, int D, int bs, int max_blocks,
                       long long num_blocks, double scale, int P, int NP, int dtype, double *m,
                       double *l, double *o, int nthreads);
int oracle_paged_varlen_dt(const void *q, const void *k, const void *v, const int32_t *bt,
                           const int32_t *sl, const int32_t *cu_q, int S, int Hq, int Hkv, int D,
                           int bs, int max_blocks, long long num_blocks, double scale, int dtype,
                           double *out, int nthreads);
void oracle_merge(const double *m, const double *l, const double *o, const int32_t *seq_lens,
                  int S, int Hq, int D, int P, int NP, double *out);

static uint64_t rng = 88172645463325252ull;
static uint32_t next(void) { rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17; return (uint32_t)rng; }
static int uni(int lo, int hi) { return lo + (int)(next() % (uint32_t)(hi - lo + 1)); }

/* a random finite value of the element type: fp16 / bf16 bit patterns of
 * small magnitude, or an fp32 */
static void fill(void *p, size_t n, int dtype) {
    for (size_t i = 0; i < n; ++i) {
        float f = ((float)(next() % 2001) - 1000.f) / 500.f;
        if (dtype == 2) { ((float *)p)[i] = f; continue; }
        uint32_t b; __builtin_memcpy(&b, &f, 4);
        if (dtype == 1) ((uint16_t *)p)[i] = (uint16_t)(b >> 16);
        else {  /* fp16: sign, exponent 13..16, mantissa */
            uint16_t h = (uint16_t)(((b >> 16) & 0x8000u) | (uint32_t)(uni(13, 16) << 10) | (next() & 0x3ffu));
            ((uint16_t *)p)[i] = h;
        }
    }
}

int main(void) {
    static const int geo[][3] = {{32, 8, 128}, {24, 4, 256}, {16, 2, 128}, {16, 16, 128}, {8, 1, 64}};
    int fails = 0;
    for (int it = 0; it < 15; ++it) {
        const int *g = geo[it % 5];
        const int Hq = g[0], Hkv = g[1], D = g[2], bs = (int[]){8, 16, 32}[it % 3];
        const int dtype = it % 3, es = dtype == 2 ? 4 : 2;
        const int S = uni(1, 4);
        int32_t *sl = malloc(sizeof(int32_t) * S), *ql = malloc(sizeof(int32_t) * S);
        int maxL = 0, need = 0;
        for (int s = 0; s < S; ++s) {
            sl[s] = (it % 7 == 0 && s == 0) ? 1 : uni(1, 600);
            ql[s] = (s == 1) ? 0 : (s == 2 ? sl[s] : uni(0, sl[s] < 5 ? sl[s] : 5));
            if (sl[s] > maxL) maxL = sl[s];
            need += (sl[s] + bs - 1) / bs;
        }
        const int mb = (maxL + bs - 1) / bs + 1;          /* one padding entry per row */
        const long long nb = need + 3;
        int32_t *bt = malloc(sizeof(int32_t) * S * mb);
        int used = 0;
        for (int s = 0; s < S; ++s)
            for (int j = 0; j < mb; ++j)
                bt[s * mb + j] = j < (sl[s] + bs - 1) / bs ? used++ : -1;
        int32_t *cu = malloc(sizeof(int32_t) * (S + 1));
        cu[0] = 0;
        for (int s = 0; s < S; ++s) cu[s + 1] = cu[s] + ql[s];
        const int T = cu[S] > 0 ? cu[S] : 1;
        void *q = malloc((size_t)es * S * Hq * D), *qv = malloc((size_t)es * T * Hq * D);
        void *k = malloc((size_t)es * nb * Hkv * bs * D), *v = malloc((size_t)es * nb * Hkv * bs * D);
        fill(q, (size_t)S * Hq * D, dtype); fill(qv, (size_t)T * Hq * D, dtype);
        fill(k, (size_t)nb * Hkv * bs * D, dtype); fill(v, (size_t)nb * Hkv * bs * D, dtype);
        double *out = malloc(sizeof(double) * S * Hq * D), *outv = malloc(sizeof(double) * T * Hq * D);
        const double scale = 0.0883883;
        fails += oracle_paged_attention_dt(q, k, v, bt, sl, S, Hq, Hkv, D, bs, mb, nb, scale, dtype, out, 1 + it % 4) != 0;
        for (int P = 256; P <= 512; P *= 2) {
            const int NP = (maxL + P - 1) / P;
            double *m = malloc(sizeof(double) * S * Hq * NP), *l = malloc(sizeof(double) * S * Hq * NP);
            double *o = malloc(sizeof(double) * S * Hq * NP * D), *mo = malloc(sizeof(double) * S * Hq * D);
            fails += oracle_partials_dt(q, k, v, bt, sl, S, Hq, Hkv, D, bs, mb, nb, scale, P, NP, dtype, m, l, o, 2) != 0;
            oracle_merge(m, l, o, sl, S, Hq, D, P, NP, mo);
            for (int i = 0; i < S * Hq * D; ++i)
                if (!(mo[i] - out[i] < 1e-9 && out[i] - mo[i] < 1e-9)) { fails++; break; }
            free(m); free(l); free(o); free(mo);
        }
        if (cu[S] > 0)
            fails += oracle_paged_varlen_dt(qv, k, v, bt, sl, cu, S, Hq, Hkv, D, bs, mb, nb, scale, dtype, outv, 3) != 0;
        free(sl); free(ql); free(bt); free(cu); free(q); free(qv); free(k); free(v); free(out); free(outv);
    }
    printf("oracle sanitizer driver: %d failures\n", fails);
    return fails != 0;
}
