/*
 * Runs the C oracle (oracle/gdn_oracle.c) under AddressSanitizer and UBSan:
 * every input and output buffer is a heap block of exactly its size, so a
 * read or write one element past any of them is reported.  A ragged batch
 * (empty, one-token and multi-chunk sequences, a GVA group of two) is run in
 * both precisions, with and without initial states and per-token states, on
 * one and on four threads; the four-thread results must equal the
 * one-thread ones bit for bit (units are independent), and the beta = 0
 * closed form S_t = exp(G_t) S_0 must hold.  Prints "OK" and exits 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gdn_oracle_forward_f64(int64_t, int32_t, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                           const float*, const float*, const float*, const float*, const float*,
                           const double*, double*, double*, double*, int32_t);
int gdn_oracle_forward_f32(int64_t, int32_t, const int32_t*, int32_t, int32_t, int32_t, int32_t,
                           const float*, const float*, const float*, const float*, const float*,
                           const float*, float*, float*, float*, int32_t);

static uint64_t rng = 88172645463325252ull;
static double uni(void) {          /* xorshift64, uniform in [0, 1) */
    rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0;
}

#define FAIL(...) do { fprintf(stderr, __VA_ARGS__); fputc('\n', stderr); return 1; } while (0)

int main(void) {
    enum { N = 4, HQK = 1, HV = 2, D = 8 };
    const int32_t cu[N + 1] = {0, 0, 1, 70, 75};
    const int64_t T = cu[N];
    const size_t nqk = (size_t)T * HQK * D, nv = (size_t)T * HV * D, ng = (size_t)T * HV;
    const size_t ns = (size_t)N * HV * D * D, nt = (size_t)T * HV * D * D;
    float* q = malloc(nqk * sizeof *q); float* k = malloc(nqk * sizeof *k);
    float* v = malloc(nv * sizeof *v); float* g = malloc(ng * sizeof *g); float* b = malloc(ng * sizeof *b);
    float* b0 = calloc(ng, sizeof *b0);
    double* s0 = malloc(ns * sizeof *s0); float* s0f = malloc(ns * sizeof *s0f);
    for (size_t i = 0; i < nqk; ++i) { q[i] = (float)(uni() - 0.5); k[i] = (float)(uni() - 0.5); }
    for (size_t i = 0; i < nv; ++i) v[i] = (float)(uni() - 0.5);
    for (size_t i = 0; i < ng; ++i) { g[i] = (float)(-uni()); b[i] = (float)uni(); }
    for (size_t i = 0; i < ns; ++i) { s0[i] = 0.02 * (uni() - 0.5); s0f[i] = (float)s0[i]; }

    double *o1 = malloc(nv * sizeof *o1), *o4 = malloc(nv * sizeof *o4);
    double *f1 = malloc(ns * sizeof *f1), *f4 = malloc(ns * sizeof *f4), *st = malloc(nt * sizeof *st);
    if (gdn_oracle_forward_f64(T, N, cu, HQK, HV, D, D, q, k, v, g, b, s0, o1, f1, st, 1)) FAIL("f64, 1 thread");
    if (gdn_oracle_forward_f64(T, N, cu, HQK, HV, D, D, q, k, v, g, b, s0, o4, f4, NULL, 4)) FAIL("f64, 4 threads");
    if (memcmp(o1, o4, nv * sizeof *o1) || memcmp(f1, f4, ns * sizeof *f1)) FAIL("thread count changed results");
    if (gdn_oracle_forward_f64(T, N, cu, HQK, HV, D, D, q, k, v, g, b, NULL, o4, NULL, NULL, 2)) FAIL("f64, no states");

    float *of = malloc(nv * sizeof *of), *ff = malloc(ns * sizeof *ff), *stf = malloc(nt * sizeof *stf);
    if (gdn_oracle_forward_f32(T, N, cu, HQK, HV, D, D, q, k, v, g, b, s0f, of, ff, stf, 3)) FAIL("f32");
    for (size_t i = 0; i < nv; ++i)
        if (!isfinite(of[i]) || fabs(of[i] - o1[i]) > 1e-4) FAIL("f32 output %zu: %g vs %g", i, of[i], o1[i]);

    /* beta = 0: pure decay of the initial state */
    if (gdn_oracle_forward_f64(T, N, cu, HQK, HV, D, D, q, k, v, g, b0, s0, o4, f4, NULL, 2)) FAIL("beta = 0");
    for (int n = 0; n < N; ++n)
        for (int h = 0; h < HV; ++h) {
            double G = 0;
            for (int t = cu[n]; t < cu[n + 1]; ++t) G += g[(size_t)t * HV + h];
            const size_t base = ((size_t)n * HV + h) * D * D;
            for (size_t e = 0; e < (size_t)D * D; ++e)
                if (fabs(f4[base + e] - exp(G) * s0[base + e]) > 1e-15) FAIL("decay closed form (%d, %d)", n, h);
        }
    /* arguments the oracle must refuse */
    const int32_t bad_cu[N + 1] = {0, 2, 1, 70, 75};
    if (gdn_oracle_forward_f64(T, N, bad_cu, HQK, HV, D, D, q, k, v, g, b, NULL, o4, NULL, NULL, 1) == 0)
        FAIL("decreasing cu_seqlens accepted");
    if (gdn_oracle_forward_f64(T, N, cu, 3, HV, D, D, q, k, v, g, b, NULL, o4, NULL, NULL, 1) == 0)
        FAIL("H_v not a multiple of H_qk accepted");

    free(q); free(k); free(v); free(g); free(b); free(b0); free(s0); free(s0f);
    free(o1); free(o4); free(f1); free(f4); free(st); free(of); free(ff); free(stf);
    puts("OK");
    return 0;
}
