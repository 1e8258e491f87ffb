/*
 * CPU oracle for the Gated DeltaNet layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  The product path never calls it; it shares no code,
 * header or constant with the HIP library.
 *
 * What it computes: the gated delta rule, one token at a time, in the plain
 * definition's order.  No page prints the recurrence; the definition in force
 * is the layer's specification, restated here.  For each sequence and value
 * head, with state S (d_v x d_k), decay alpha_t = exp(g_t) and write strength
 * beta_t:
 *
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * Expanding the first line: S_t = alpha_t S_{t-1}
 *                                + beta_t (v_t - alpha_t S_{t-1} k_t) k_t^T,
 * i.e. decay the old state, predict v_t from the decayed state, and write
 * beta times the prediction error along k_t.  That is the loop below.
 *
 * The pages this library follows (the "2080 Ti runs Qwen3.8-27B: a vLLM
 * plugin" page, section 2 "GDN prefill") use GDN as a linear-attention layer
 * whose state has a fixed size per request, checked kernel by kernel against
 * an fp32 reference; the "Qwen3.8-27B on one RTX 3090" page (section
 * "Exploiter l'architecture hybride") describes that fixed-size per-request
 * state, and the section on the 131,072-token limit keeps one state snapshot
 * per speculative token.  The per-token snapshots recorded here serve that
 * rollback use.
 *
 * Layout conventions (shared by contract with the library, not by code):
 *   q, k : [T, H_qk, d_k]   v : [T, H_v, d_v]   g, beta : [T, H_v]
 *   state: [N, H_v, d_k, d_v] holding state[a][b] = S[b][a] (d_v contiguous)
 *   out  : [T, H_v, d_v]
 *   value head h reads q/k head h / (H_v / H_qk)  (contiguous groups).
 * Sequences are packed: tokens cu_seqlens[n] .. cu_seqlens[n+1]-1.
 *
 * Inputs are float32 (bfloat16-rounded values are exactly representable);
 * the arithmetic runs in the instantiation's type: double or float.  Sums
 * run in ascending index order.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_BAD_ARGS 1
#define ORACLE_NO_MEMORY 2

/* One (sequence, value head) unit of the recurrence. */
#define DEFINE_ORACLE(real, SUFFIX, EXP)                                           \
static void unit_##SUFFIX(int64_t t0, int64_t t1, int32_t h, int32_t j,           \
                          int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,    \
                          const float* q, const float* k, const float* v,         \
                          const float* g, const float* beta,                      \
                          const real* s0, real* out, real* s_final,               \
                          real* token_states, real* H, real* p, real* delta)      \
{                                                                                 \
    const size_t dd = (size_t)d_k * (size_t)d_v;                                  \
    if (s0) memcpy(H, s0, dd * sizeof(real));                                     \
    else memset(H, 0, dd * sizeof(real));                                         \
    for (int64_t t = t0; t < t1; ++t) {                                           \
        const float* kt = k + ((size_t)t * h_qk + j) * d_k;                       \
        const float* qt = q + ((size_t)t * h_qk + j) * d_k;                       \
        const float* vt = v + ((size_t)t * h_v + h) * d_v;                        \
        const real alpha = EXP((real)g[(size_t)t * h_v + h]);                     \
        const real b = (real)beta[(size_t)t * h_v + h];                           \
        /* decay: S <- alpha S */                                                 \
        for (size_t e = 0; e < dd; ++e) H[e] *= alpha;                            \
        /* prediction p = (alpha S) k, i.e. p[c] = sum_a k[a] H[a][c] */          \
        for (int32_t c = 0; c < d_v; ++c) p[c] = 0;                               \
        for (int32_t a = 0; a < d_k; ++a) {                                       \
            const real ka = (real)kt[a];                                          \
            const real* row = H + (size_t)a * d_v;                                \
            for (int32_t c = 0; c < d_v; ++c) p[c] += ka * row[c];                \
        }                                                                         \
        /* delta = beta (v - p) */                                                \
        for (int32_t c = 0; c < d_v; ++c) delta[c] = b * ((real)vt[c] - p[c]);    \
        /* rank-one write: S <- S + delta k^T, i.e. H[a][c] += k[a] delta[c] */   \
        for (int32_t a = 0; a < d_k; ++a) {                                       \
            const real ka = (real)kt[a];                                          \
            real* row = H + (size_t)a * d_v;                                      \
            for (int32_t c = 0; c < d_v; ++c) row[c] += ka * delta[c];            \
        }                                                                         \
        /* output from the updated state: o = S q, o[c] = sum_a q[a] H[a][c] */   \
        real* ot = out + ((size_t)t * h_v + h) * d_v;                             \
        for (int32_t c = 0; c < d_v; ++c) ot[c] = 0;                              \
        for (int32_t a = 0; a < d_k; ++a) {                                       \
            const real qa = (real)qt[a];                                          \
            const real* row = H + (size_t)a * d_v;                                \
            for (int32_t c = 0; c < d_v; ++c) ot[c] += qa * row[c];               \
        }                                                                         \
        if (token_states)                                                         \
            memcpy(token_states + ((size_t)t * h_v + h) * dd, H, dd * sizeof(real)); \
    }                                                                             \
    if (s_final) memcpy(s_final, H, dd * sizeof(real));                           \
}                                                                                 \
                                                                                  \
int gdn_oracle_forward_##SUFFIX(                                                  \
    int64_t total_tokens, int32_t n_seqs, const int32_t* cu_seqlens,              \
    int32_t h_qk, int32_t h_v, int32_t d_k, int32_t d_v,                          \
    const float* q, const float* k, const float* v,                               \
    const float* g, const float* beta,                                            \
    const real* initial_state, real* out, real* final_state,                      \
    real* token_states, int32_t n_threads)                                        \
{                                                                                 \
    if (n_seqs < 0 || h_qk <= 0 || h_v <= 0 || d_k <= 0 || d_v <= 0 ||            \
        h_v % h_qk != 0 || !cu_seqlens || total_tokens < 0)                       \
        return ORACLE_BAD_ARGS;                                                   \
    if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != total_tokens)                 \
        return ORACLE_BAD_ARGS;                                                   \
    for (int32_t n = 0; n < n_seqs; ++n)                                          \
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return ORACLE_BAD_ARGS;            \
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !out))              \
        return ORACLE_BAD_ARGS;                                                   \
    const int32_t group = h_v / h_qk;                                             \
    const size_t dd = (size_t)d_k * (size_t)d_v;                                  \
    const int64_t units = (int64_t)n_seqs * h_v;                                  \
    int failed = 0;                                                               \
    if (n_threads <= 0) n_threads = 1;                                            \
    _Pragma("omp parallel num_threads(n_threads) reduction(|:failed)")            \
    {                                                                             \
        real* H = (real*)malloc(dd * sizeof(real));                               \
        real* p = (real*)malloc((size_t)d_v * sizeof(real));                      \
        real* delta = (real*)malloc((size_t)d_v * sizeof(real));                  \
        const int ok = H && p && delta;                                           \
        if (!ok) failed = 1;                                                      \
        {                                                                         \
            _Pragma("omp for schedule(dynamic, 1)")                               \
            for (int64_t u = 0; u < units; ++u) {                                 \
                if (!ok) continue;                                                \
                const int32_t n = (int32_t)(u / h_v), h = (int32_t)(u % h_v);     \
                const size_t so = ((size_t)n * h_v + h) * dd;                     \
                unit_##SUFFIX(cu_seqlens[n], cu_seqlens[n + 1], h, h / group,     \
                              h_qk, h_v, d_k, d_v, q, k, v, g, beta,              \
                              initial_state ? initial_state + so : NULL, out,     \
                              final_state ? final_state + so : NULL,              \
                              token_states, H, p, delta);                         \
            }                                                                     \
        }                                                                         \
        free(H); free(p); free(delta);                                            \
    }                                                                             \
    return failed ? ORACLE_NO_MEMORY : ORACLE_OK;                                 \
}

DEFINE_ORACLE(double, f64, exp)
DEFINE_ORACLE(float, f32, expf)

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
