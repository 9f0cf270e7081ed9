/*
 * CPU ORACLE FOR THE GATED DELTA RULE -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.
 *
 * Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
 * build, load or call this file.  It shares no code, header, table or helper with
 * the HIP library; the two meet only through the seeded input arrays.
 *
 * What it computes (fp64 throughout, inputs upcast exactly):
 *
 *   For every sequence n and value head h (key/query head hk = h % Hk, the GQA
 *   head replication named on the page "Exp 2026-07-13 -- Linear-Attention Scans
 *   on the NPU", section 4, marshaller description):
 *
 *     S <- initial_state[n, h]  (or zeros)                       S is Dv x Dk
 *     for each token t of sequence n, in order:
 *        a = exp(g[t, h])          g is the natural log of the decay alpha
 *        b = beta[t, h]
 *        S <- a * S * (I - b * k_t k_t^T) + b * v_t k_t^T
 *        o[t, h] = S q_t           (output reads the UPDATED state)
 *     final_state[n, h] <- S
 *
 *   The update-then-output order and the per-head fixed-size state follow
 *   "Empowering Hybrid Attention Models on NPUs", section 2.1 (architecture of
 *   linear-attention hybrids): the state is first updated with K_t and V_t, then
 *   the output is formed with Q_t and the updated state.  The matrix form of the
 *   update is the gated delta rule S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T)
 *   + beta_t v_t k_t^T.  No query scaling is applied.
 *
 * The product a * S * (I - b k k^T) is evaluated by distributing it:
 *   a * S * (I - b k k^T) = a * S - a * b * (S k) k^T,
 * so each token costs one matrix-vector product S k, one rank-1 update and the
 * output product S q.  This is a plain evaluation of the same expression; nothing
 * is chunked, reordered across tokens or approximated.
 *
 * A second pair of entry points (gdn_oracle_kda_*) evaluates the same rule with one
 * decay per key channel instead of one per head; see kda_token_step below.
 *
 * Parallelism: independent (sequence, value head) chains run on OpenMP threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the gated delta rule on a Dv x Dk state (row-major, key index fastest). */
static void gdn_token_step(double *S, const double *kt, const double *vt, const double *qt,
                           double a, double b, int64_t Dk, int64_t Dv, double *Sk, double *ot)
{
    /* Sk = S k_t  (uses the state before this token) */
    for (int64_t i = 0; i < Dv; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < Dk; ++j) acc += S[i * Dk + j] * kt[j];
        Sk[i] = acc;
    }
    /* S <- a*S - a*b*(S k) k^T + b * v k^T   ==   a*S*(I - b k k^T) + b v k^T */
    for (int64_t i = 0; i < Dv; ++i) {
        const double erase = a * b * Sk[i];
        const double write = b * vt[i];
        for (int64_t j = 0; j < Dk; ++j)
            S[i * Dk + j] = a * S[i * Dk + j] - erase * kt[j] + write * kt[j];
    }
    /* o_t = S q_t with the updated state */
    for (int64_t i = 0; i < Dv; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < Dk; ++j) acc += S[i * Dk + j] * qt[j];
        ot[i] = acc;
    }
}

/*
 * Packed variable-length prefill.
 *   q, k           [T_tot, Hk, Dk]
 *   v              [T_tot, Hv, Dv]
 *   g, beta        [T_tot, Hv]
 *   initial_state  [N, Hv, Dv, Dk] or NULL (zeros)
 *   cu_seqlens     [N+1], cu[0] = 0, nondecreasing, cu[N] = T_tot
 *   o              [T_tot, Hv, Dv]   (written)
 *   final_state    [N, Hv, Dv, Dk] or NULL
 *   nthreads       OpenMP threads (<= 0: runtime default)
 * Returns 0 on success, -1 on bad arguments, -2 if out of memory.
 */
int gdn_oracle_prefill_f64(const double *q, const double *k, const double *v,
                           const double *g, const double *beta,
                           const double *initial_state, const int64_t *cu_seqlens,
                           int64_t N, int64_t T_tot, int64_t Hk, int64_t Hv,
                           int64_t Dk, int64_t Dv,
                           double *o, double *final_state, int nthreads)
{
    if (N < 1 || T_tot < 0 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1 || (Hv % Hk) != 0)
        return -1;
    if (!cu_seqlens || cu_seqlens[0] != 0 || cu_seqlens[N] != T_tot) return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (T_tot > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;

    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t pairs = N * Hv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t n = p / Hv, h = p % Hv, hk = h % Hk;
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dv * Dk + 2 * Dv));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *Sk = S + Dv * Dk;
        double *ot = Sk + Dv;
        if (initial_state)
            memcpy(S, initial_state + (n * Hv + h) * Dv * Dk, sizeof(double) * (size_t)(Dv * Dk));
        else
            memset(S, 0, sizeof(double) * (size_t)(Dv * Dk));
        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            const double *kt = k + (t * Hk + hk) * Dk;
            const double *qt = q + (t * Hk + hk) * Dk;
            const double *vt = v + (t * Hv + h) * Dv;
            const double a = exp(g[t * Hv + h]);
            const double b = beta[t * Hv + h];
            gdn_token_step(S, kt, vt, qt, a, b, Dk, Dv, Sk, ot);
            memcpy(o + (t * Hv + h) * Dv, ot, sizeof(double) * (size_t)Dv);
        }
        if (final_state)
            memcpy(final_state + (n * Hv + h) * Dv * Dk, S, sizeof(double) * (size_t)(Dv * Dk));
        free(S);
    }
    return failed ? -2 : 0;
}

/*
 * One decoding token per sequence: the same recurrence with T = 1, the state updated
 * in place (token-by-token recurrence serves decoding; same page, section 2.1).
 *   q, k [B, Hk, Dk];  v [B, Hv, Dv];  g, beta [B, Hv];  state [B, Hv, Dv, Dk] in/out;
 *   o [B, Hv, Dv].
 */
int gdn_oracle_decode_step_f64(const double *q, const double *k, const double *v,
                               const double *g, const double *beta, double *state,
                               int64_t B, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv,
                               double *o, int nthreads)
{
    if (B < 1 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1 || (Hv % Hk) != 0) return -1;
    if (!q || !k || !v || !g || !beta || !state || !o) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t pairs = B * Hv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t b = p / Hv, h = p % Hv, hk = h % Hk;
        double *Sk = (double *)malloc(sizeof(double) * (size_t)(2 * Dv));
        if (!Sk) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        gdn_token_step(state + (b * Hv + h) * Dv * Dk, k + (b * Hk + hk) * Dk,
                       v + (b * Hv + h) * Dv, q + (b * Hk + hk) * Dk,
                       exp(g[b * Hv + h]), beta[b * Hv + h], Dk, Dv, Sk, Sk + Dv);
        memcpy(o + (b * Hv + h) * Dv, Sk + Dv, sizeof(double) * (size_t)Dv);
        free(Sk);
    }
    return failed ? -2 : 0;
}

/*
 * Per-key-channel decay (the KDA variant of the same delta rule, whose gate is
 * "fine-grained": one decay per key channel instead of one per head, so its
 * cumulative gate is Dk times larger -- "Empowering Hybrid Attention Models on NPUs",
 * section 2.1 and the peak-memory discussion of section 7.5).  The scalar alpha_t of
 * the gated delta rule becomes the diagonal matrix Diag(a_t), a_t[j] = exp(g[t, h, j]),
 * acting on the key index of S, applied before the erase exactly as alpha_t is:
 *
 *     S <- S Diag(a_t) (I - b k_t k_t^T) + b v_t k_t^T,     o_t = S q_t
 *
 * evaluated as  D = S Diag(a_t);  u = D k_t;  S = D - b u k_t^T + b v_t k_t^T.
 */
static void kda_token_step(double *S, const double *kt, const double *vt, const double *qt,
                           const double *gt, double b, int64_t Dk, int64_t Dv,
                           double *a, double *u, double *ot)
{
    for (int64_t j = 0; j < Dk; ++j) a[j] = exp(gt[j]);
    /* S <- S Diag(a): column j (key channel j) decays by a[j] */
    for (int64_t i = 0; i < Dv; ++i)
        for (int64_t j = 0; j < Dk; ++j) S[i * Dk + j] *= a[j];
    /* u = (S Diag(a)) k_t */
    for (int64_t i = 0; i < Dv; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < Dk; ++j) acc += S[i * Dk + j] * kt[j];
        u[i] = acc;
    }
    /* S <- S - b u k^T + b v k^T */
    for (int64_t i = 0; i < Dv; ++i) {
        const double erase = b * u[i];
        const double write = b * vt[i];
        for (int64_t j = 0; j < Dk; ++j)
            S[i * Dk + j] = S[i * Dk + j] - erase * kt[j] + write * kt[j];
    }
    /* o_t = S q_t with the updated state */
    for (int64_t i = 0; i < Dv; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < Dk; ++j) acc += S[i * Dk + j] * qt[j];
        ot[i] = acc;
    }
}

/*
 * Packed variable-length prefill with per-key-channel decay.  Arguments as for
 * gdn_oracle_prefill_f64 except  g [T_tot, Hv, Dk]  (natural log of each channel's
 * decay).
 */
int gdn_oracle_kda_prefill_f64(const double *q, const double *k, const double *v,
                               const double *g, const double *beta,
                               const double *initial_state, const int64_t *cu_seqlens,
                               int64_t N, int64_t T_tot, int64_t Hk, int64_t Hv,
                               int64_t Dk, int64_t Dv,
                               double *o, double *final_state, int nthreads)
{
    if (N < 1 || T_tot < 0 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1 || (Hv % Hk) != 0)
        return -1;
    if (!cu_seqlens || cu_seqlens[0] != 0 || cu_seqlens[N] != T_tot) return -1;
    for (int64_t n = 0; n < N; ++n)
        if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;
    if (T_tot > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;

    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t pairs = N * Hv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t n = p / Hv, h = p % Hv, hk = h % Hk;
        double *S = (double *)malloc(sizeof(double) * (size_t)(Dv * Dk + 2 * Dv + Dk));
        if (!S) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        double *u = S + Dv * Dk;
        double *ot = u + Dv;
        double *a = ot + Dv;
        if (initial_state)
            memcpy(S, initial_state + (n * Hv + h) * Dv * Dk, sizeof(double) * (size_t)(Dv * Dk));
        else
            memset(S, 0, sizeof(double) * (size_t)(Dv * Dk));
        for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
            kda_token_step(S, k + (t * Hk + hk) * Dk, v + (t * Hv + h) * Dv,
                           q + (t * Hk + hk) * Dk, g + (t * Hv + h) * Dk,
                           beta[t * Hv + h], Dk, Dv, a, u, ot);
            memcpy(o + (t * Hv + h) * Dv, ot, sizeof(double) * (size_t)Dv);
        }
        if (final_state)
            memcpy(final_state + (n * Hv + h) * Dv * Dk, S, sizeof(double) * (size_t)(Dv * Dk));
        free(S);
    }
    return failed ? -2 : 0;
}

/* One decoding token per sequence with per-key-channel decay: g [B, Hv, Dk]. */
int gdn_oracle_kda_decode_step_f64(const double *q, const double *k, const double *v,
                                   const double *g, const double *beta, double *state,
                                   int64_t B, int64_t Hk, int64_t Hv, int64_t Dk, int64_t Dv,
                                   double *o, int nthreads)
{
    if (B < 1 || Hk < 1 || Hv < 1 || Dk < 1 || Dv < 1 || (Hv % Hk) != 0) return -1;
    if (!q || !k || !v || !g || !beta || !state || !o) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int64_t pairs = B * Hv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
        const int64_t b = p / Hv, h = p % Hv, hk = h % Hk;
        double *w = (double *)malloc(sizeof(double) * (size_t)(2 * Dv + Dk));
        if (!w) {
#pragma omp atomic write
            failed = 1;
            continue;
        }
        kda_token_step(state + (b * Hv + h) * Dv * Dk, k + (b * Hk + hk) * Dk,
                       v + (b * Hv + h) * Dv, q + (b * Hk + hk) * Dk, g + (b * Hv + h) * Dk,
                       beta[b * Hv + h], Dk, Dv, w + 2 * Dv, w, w + Dv);
        memcpy(o + (b * Hv + h) * Dv, w + Dv, sizeof(double) * (size_t)Dv);
        free(w);
    }
    return failed ? -2 : 0;
}

int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
