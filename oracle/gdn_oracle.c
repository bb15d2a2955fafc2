/*
 * Frame-wise Gated DeltaNet forward scan: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this file.  It shares no
 * code with the HIP library (no headers, helpers or tables) and the HIP library
 * never calls it.
 *
 * What it computes.  The pages describe the layer only in words: a recurrent
 * layer that consumes one entire latent frame per step and keeps a fixed-size
 * state matrix, updated by a decay gate and a delta-rule correction ("NVIDIA's
 * New 2.6B World Model Generates Minute-Scale 720p Video on a Single GPU",
 * section "The Architecture: Replacing Softmax Attention at Scale"; "SANA-WM:
 * democratizing Minute-Scale World Modeling with Hybrid Linear DiT", section
 * "Methodology", item 1, which adds that GDN scans frames one by one and
 * updates a compact latent state).  The operator implemented here is the plain
 * reading of that sentence, for every batch item b and head h:
 *
 *     k^_i  = k_i / max(||k_i||_2, eps)            (per token i of frame f)
 *     G_f   = sum_i beta_i k^_i k^_i^T             (Dk x Dk)
 *     U_f   = sum_i beta_i v_i  k^_i^T             (Dv x Dk)
 *     S_f   = alpha_f * S_{f-1} (I - G_f) + U_f    (Dv x Dk, S_0 given or 0)
 *     O_f   = Q_f S_f^T                            (row i: o_i = S_f q_i)
 *
 * Every token of a frame sees the same S_{f-1} (the frame is one step) and the
 * output of a frame reads the post-update state S_f.  With N = 1 this is the
 * token-level gated delta rule.  With gates_are_logits the inputs are logits:
 * alpha = sigmoid(a), beta = sigmoid(b) / N.  With normalize_k == 0 the keys
 * are used as given (k^_i = k_i), the library's option for callers whose keys
 * already have unit norm.
 *
 * Reverse direction (reverse != 0): the same recurrence walked from the last
 * frame to the first, S entering at frame F and S_final leaving after frame 1
 * (the "bidirectional" weights on the WorldFoundry "SANA-WM" page, sections
 * "What it is for" and "Running in WorldFoundry", scan in both directions;
 * the pages do not say how the two are combined, so each direction is a scan
 * of its own):  S_f = alpha_f * S_{f+1} (I - G_f) + U_f,  O_f = Q_f S_f^T.
 *
 * Layouts (row-major, last index fastest):
 *     q, k  [B][F][N][H][Dk]      v, o  [B][F][N][H][Dv]
 *     beta  [B][F][N][H]          alpha [B][F][H]
 *     S0, S_final [B][H][Dv][Dk]  (row = value dimension)
 *
 * Each loop follows the equations literally; every sum runs over its index in
 * ascending order.  OpenMP splits only loops whose iterations write disjoint
 * outputs, so the result is bitwise independent of the thread count.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Returns 0 on success, -1 on a bad argument, -2 when scratch memory fails. */
int gdn_oracle_scan(int B, int H, int F, int N, int Dk, int Dv,
                    const double *q, const double *k, const double *v,
                    const double *beta, const double *alpha,
                    const double *S0, double eps, int gates_are_logits,
                    int normalize_k, int reverse, double *o, double *S_final)
{
    if (B < 0 || H < 0 || F < 0 || N < 0 || Dk < 1 || Dv < 1 || !(eps > 0.0))
        return -1;
    const size_t sB = (size_t)F * N * H, sF = (size_t)N * H, sN = (size_t)H;

    double *S = (double *)malloc(sizeof(double) * (size_t)Dv * Dk);
    double *T = (double *)malloc(sizeof(double) * (size_t)Dv * Dk);
    double *G = (double *)malloc(sizeof(double) * (size_t)Dk * Dk);
    double *U = (double *)malloc(sizeof(double) * (size_t)Dv * Dk);
    double *kh = (double *)malloc(sizeof(double) * ((size_t)N * Dk + 1));
    double *bt = (double *)malloc(sizeof(double) * ((size_t)N + 1));
    if (!S || !T || !G || !U || !kh || !bt) {
        free(S); free(T); free(G); free(U); free(kh); free(bt);
        return -2;
    }

    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            /* S <- S0[b,h], or zeros */
            for (int a = 0; a < Dv; ++a)
                for (int e = 0; e < Dk; ++e)
                    S[(size_t)a * Dk + e] =
                        S0 ? S0[(((size_t)b * H + h) * Dv + a) * Dk + e] : 0.0;

            for (int step = 0; step < F; ++step) {
                const int f = reverse ? F - 1 - step : step;   /* frame of this step */
                const size_t tok0 = (size_t)b * sB + (size_t)f * sF; /* token 0, head 0 */
                double al = alpha[((size_t)b * F + f) * H + h];
                if (gates_are_logits) al = sigmoid(al);

                /* per-token normalised keys and betas */
                for (int i = 0; i < N; ++i) {
                    const double *ki = k + (tok0 + (size_t)i * sN + h) * Dk;
                    double ss = 0.0;
                    for (int c = 0; c < Dk; ++c) ss += ki[c] * ki[c];
                    double nrm = sqrt(ss);
                    double den = nrm > eps ? nrm : eps;
                    if (!normalize_k) den = 1.0;   /* keys used as given */
                    for (int c = 0; c < Dk; ++c) kh[(size_t)i * Dk + c] = ki[c] / den;
                    double bi = beta[tok0 + (size_t)i * sN + h];
                    bt[i] = gates_are_logits ? sigmoid(bi) / (double)N : bi;
                }

                /* G[c][e] = sum_i beta_i kh[i][c] kh[i][e] */
#pragma omp parallel for schedule(static)
                for (int c = 0; c < Dk; ++c) {
                    double *Gc = G + (size_t)c * Dk;
                    for (int e = 0; e < Dk; ++e) Gc[e] = 0.0;
                    for (int i = 0; i < N; ++i) {
                        const double *ki = kh + (size_t)i * Dk;
                        const double s = bt[i] * ki[c];
                        for (int e = 0; e < Dk; ++e) Gc[e] += s * ki[e];
                    }
                }

                /* U[a][e] = sum_i beta_i v[i][a] kh[i][e] */
#pragma omp parallel for schedule(static)
                for (int a = 0; a < Dv; ++a) {
                    double *Ua = U + (size_t)a * Dk;
                    for (int e = 0; e < Dk; ++e) Ua[e] = 0.0;
                    for (int i = 0; i < N; ++i) {
                        const double *vi = v + (tok0 + (size_t)i * sN + h) * Dv;
                        const double *ki = kh + (size_t)i * Dk;
                        const double s = bt[i] * vi[a];
                        for (int e = 0; e < Dk; ++e) Ua[e] += s * ki[e];
                    }
                }

                /* T = S - S G ;  S <- alpha T + U */
#pragma omp parallel for schedule(static)
                for (int a = 0; a < Dv; ++a) {
                    const double *Sa = S + (size_t)a * Dk;
                    double *Ta = T + (size_t)a * Dk;
                    for (int e = 0; e < Dk; ++e) Ta[e] = Sa[e];
                    for (int c = 0; c < Dk; ++c) {
                        const double s = Sa[c];
                        const double *Gc = G + (size_t)c * Dk;
                        for (int e = 0; e < Dk; ++e) Ta[e] -= s * Gc[e];
                    }
                }
                for (size_t x = 0; x < (size_t)Dv * Dk; ++x) S[x] = al * T[x] + U[x];

                /* O[f,i,a] = sum_e q[i][e] S[a][e]  (post-update state) */
#pragma omp parallel for schedule(static)
                for (int i = 0; i < N; ++i) {
                    const double *qi = q + (tok0 + (size_t)i * sN + h) * Dk;
                    double *oi = o + (tok0 + (size_t)i * sN + h) * Dv;
                    for (int a = 0; a < Dv; ++a) {
                        const double *Sa = S + (size_t)a * Dk;
                        double acc = 0.0;
                        for (int e = 0; e < Dk; ++e) acc += qi[e] * Sa[e];
                        oi[a] = acc;
                    }
                }
            }
            if (S_final)
                memcpy(S_final + ((size_t)b * H + h) * Dv * Dk, S,
                       sizeof(double) * (size_t)Dv * Dk);
        }
    }
    free(S); free(T); free(G); free(U); free(kh); free(bt);
    return 0;
}

/* Threads an OpenMP parallel region would use (1 without OpenMP). */
int gdn_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
