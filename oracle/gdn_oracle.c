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

/*
 * Backward pass of the same scan, in fp64 loops.  Given the output gradient
 * dO = dL/dO ([B][F][N][H][Dv]) and dS_final = dL/dS_final ([B][H][Dv][Dk],
 * NULL = zeros), returns dq, dk, dv, dbeta, dalpha and dS0 in the layouts of
 * q, k, v, beta, alpha and S0 (with gates_are_logits, dbeta and dalpha are the
 * gradients of the logits).  This is the plain chain rule of the forward
 * definition above ("SANA-WM: democratizing Minute-Scale World Modeling with
 * Hybrid Linear DiT", "Problem & Motivation": the model is trained natively on
 * minute-long sequences, which needs the gradient of the scan):
 *
 *   states S_0 .. S_F are recomputed by the forward recurrence; then, with
 *   D = dL/dS_f, walking the steps backward from D = dS_final:
 *     D      += sum_i do_i q_i^T                 (frame f's outputs read S_f)
 *     dq_i    = S_f^T do_i
 *     dU_f    = D
 *     dalpha  = <D, S_{f-1} (I - G_f)>
 *     dG_f    = -alpha_f S_{f-1}^T D
 *     D      <- alpha_f D (I - G_f)^T            (dL/dS_{f-1})
 *     from G_f = sum_i beta_i k^_i k^_i^T and U_f = sum_i beta_i v_i k^_i^T:
 *       dk^_i   = beta_i (dG_f + dG_f^T) k^_i + beta_i dU_f^T v_i
 *       dv_i    = beta_i dU_f k^_i
 *       dbeta_i = k^_i^T dG_f k^_i + v_i^T dU_f k^_i
 *     from k^_i = k_i / n_i (n_i = ||k_i|| > eps):  dk_i = (dk^_i - k^_i (k^_i . dk^_i)) / n_i
 *     (n_i <= eps: dk_i = dk^_i / eps; keys used as given: dk_i = dk^_i)
 *   dS0 = D after the first step.  Logits: dlogit = dbeta sigma'(b) / N and
 *   dalpha sigma'(a).  The reverse direction walks the same steps in its own
 *   order.  Returns 0, -1 (bad argument) or -2 (no memory).
 */
int gdn_oracle_scan_bwd(int B, int H, int F, int N, int Dk, int Dv,
                        const double *q, const double *k, const double *v,
                        const double *beta, const double *alpha,
                        const double *S0, double eps, int gates_are_logits,
                        int normalize_k, int reverse,
                        const double *dO, const double *dS_final,
                        double *dq, double *dk, double *dv, double *dbeta,
                        double *dalpha, double *dS0)
{
    if (B < 0 || H < 0 || F < 0 || N < 0 || Dk < 1 || Dv < 1 || !(eps > 0.0))
        return -1;
    const size_t sB = (size_t)F * N * H, sF = (size_t)N * H, sN = (size_t)H;
    const size_t SS = (size_t)Dv * Dk;
    int status = 0;
    /* The (b, h) units are independent: each thread takes whole units, with
     * scratch of its own; the arithmetic of a unit is the same as in a plain
     * loop over the units. */
#pragma omp parallel
    {
    double *Sall = (double *)malloc(sizeof(double) * SS * ((size_t)F + 1));
    double *G = (double *)malloc(sizeof(double) * (size_t)Dk * Dk);
    double *U = (double *)malloc(sizeof(double) * SS);
    double *T = (double *)malloc(sizeof(double) * SS);
    double *Dm = (double *)malloc(sizeof(double) * SS);
    double *Dn = (double *)malloc(sizeof(double) * SS);
    double *dG = (double *)malloc(sizeof(double) * (size_t)Dk * Dk);
    double *kh = (double *)malloc(sizeof(double) * ((size_t)N * Dk + 1));
    double *nrm = (double *)malloc(sizeof(double) * ((size_t)N + 1));
    double *bt = (double *)malloc(sizeof(double) * ((size_t)N + 1));
    double *dkh = (double *)malloc(sizeof(double) * ((size_t)Dk + 1));
    const int ok = Sall && G && U && T && Dm && Dn && dG && kh && nrm && bt && dkh;
    if (!ok) {
#pragma omp atomic write
        status = -2;
    }

#pragma omp for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            if (!ok) continue;
            /* ---- forward, keeping every state: Sall[s] is the state after step s */
            for (size_t x = 0; x < SS; ++x)
                Sall[x] = S0 ? S0[((size_t)b * H + h) * SS + x] : 0.0;
            for (int step = 0; step < F; ++step) {
                const int f = reverse ? F - 1 - step : step;
                const size_t tok0 = (size_t)b * sB + (size_t)f * sF;
                double al = alpha[((size_t)b * F + f) * H + h];
                if (gates_are_logits) al = sigmoid(al);
                for (int i = 0; i < N; ++i) {
                    const double *ki = k + (tok0 + (size_t)i * sN + h) * Dk;
                    double ss = 0.0;
                    for (int c = 0; c < Dk; ++c) ss += ki[c] * ki[c];
                    const double n = sqrt(ss);
                    const double den = normalize_k ? (n > eps ? n : eps) : 1.0;
                    for (int c = 0; c < Dk; ++c) kh[(size_t)i * Dk + c] = ki[c] / den;
                    const double bi = beta[tok0 + (size_t)i * sN + h];
                    bt[i] = gates_are_logits ? sigmoid(bi) / (double)N : bi;
                }
                for (int c = 0; c < Dk; ++c)
                    for (int e = 0; e < Dk; ++e) {
                        double acc = 0.0;
                        for (int i = 0; i < N; ++i)
                            acc += bt[i] * kh[(size_t)i * Dk + c] * kh[(size_t)i * Dk + e];
                        G[(size_t)c * Dk + e] = acc;
                    }
                for (int a = 0; a < Dv; ++a)
                    for (int e = 0; e < Dk; ++e) {
                        double acc = 0.0;
                        for (int i = 0; i < N; ++i)
                            acc += bt[i] * v[(tok0 + (size_t)i * sN + h) * Dv + a] * kh[(size_t)i * Dk + e];
                        U[(size_t)a * Dk + e] = acc;
                    }
                const double *Sp = Sall + (size_t)step * SS;
                double *Sn = Sall + (size_t)(step + 1) * SS;
                for (int a = 0; a < Dv; ++a)
                    for (int e = 0; e < Dk; ++e) {
                        double t = Sp[(size_t)a * Dk + e];
                        for (int c = 0; c < Dk; ++c) t -= Sp[(size_t)a * Dk + c] * G[(size_t)c * Dk + e];
                        Sn[(size_t)a * Dk + e] = al * t + U[(size_t)a * Dk + e];
                    }
            }

            /* ---- backward */
            for (size_t x = 0; x < SS; ++x)
                Dm[x] = dS_final ? dS_final[((size_t)b * H + h) * SS + x] : 0.0;
            for (int step = F - 1; step >= 0; --step) {
                const int f = reverse ? F - 1 - step : step;
                const size_t tok0 = (size_t)b * sB + (size_t)f * sF;
                const double *Sp = Sall + (size_t)step * SS;        /* state before this step */
                const double *Sc = Sall + (size_t)(step + 1) * SS;  /* state after it */
                const double a_in = alpha[((size_t)b * F + f) * H + h];
                const double al = gates_are_logits ? sigmoid(a_in) : a_in;
                /* keys, norms and betas of the frame (as in the forward) */
                for (int i = 0; i < N; ++i) {
                    const double *ki = k + (tok0 + (size_t)i * sN + h) * Dk;
                    double ss = 0.0;
                    for (int c = 0; c < Dk; ++c) ss += ki[c] * ki[c];
                    nrm[i] = sqrt(ss);
                    const double den = normalize_k ? (nrm[i] > eps ? nrm[i] : eps) : 1.0;
                    for (int c = 0; c < Dk; ++c) kh[(size_t)i * Dk + c] = ki[c] / den;
                    const double bi = beta[tok0 + (size_t)i * sN + h];
                    bt[i] = gates_are_logits ? sigmoid(bi) / (double)N : bi;
                }
                for (int c = 0; c < Dk; ++c)
                    for (int e = 0; e < Dk; ++e) {
                        double acc = 0.0;
                        for (int i = 0; i < N; ++i)
                            acc += bt[i] * kh[(size_t)i * Dk + c] * kh[(size_t)i * Dk + e];
                        G[(size_t)c * Dk + e] = acc;
                    }
                /* D += sum_i do_i q_i^T ;  dq_i = S_f^T do_i */
                for (int i = 0; i < N; ++i) {
                    const double *doi = dO + (tok0 + (size_t)i * sN + h) * Dv;
                    const double *qi = q + (tok0 + (size_t)i * sN + h) * Dk;
                    double *dqi = dq + (tok0 + (size_t)i * sN + h) * Dk;
                    for (int a = 0; a < Dv; ++a)
                        for (int e = 0; e < Dk; ++e) Dm[(size_t)a * Dk + e] += doi[a] * qi[e];
                    for (int e = 0; e < Dk; ++e) {
                        double acc = 0.0;
                        for (int a = 0; a < Dv; ++a) acc += Sc[(size_t)a * Dk + e] * doi[a];
                        dqi[e] = acc;
                    }
                }
                /* T = S_{f-1} (I - G) ;  dalpha = <D, T> */
                double da = 0.0;
                for (int a = 0; a < Dv; ++a)
                    for (int e = 0; e < Dk; ++e) {
                        double t = Sp[(size_t)a * Dk + e];
                        for (int c = 0; c < Dk; ++c) t -= Sp[(size_t)a * Dk + c] * G[(size_t)c * Dk + e];
                        T[(size_t)a * Dk + e] = t;
                        da += Dm[(size_t)a * Dk + e] * t;
                    }
                dalpha[((size_t)b * F + f) * H + h] = gates_are_logits ? da * al * (1.0 - al) : da;
                /* dG = -alpha S_{f-1}^T D */
                for (int c = 0; c < Dk; ++c)
                    for (int e = 0; e < Dk; ++e) {
                        double acc = 0.0;
                        for (int a = 0; a < Dv; ++a) acc += Sp[(size_t)a * Dk + c] * Dm[(size_t)a * Dk + e];
                        dG[(size_t)c * Dk + e] = -al * acc;
                    }
                /* token gradients through G and U (dU = D) */
                for (int i = 0; i < N; ++i) {
                    const size_t ti = tok0 + (size_t)i * sN + h;
                    const double *khi = kh + (size_t)i * Dk;
                    const double *vi = v + ti * Dv;
                    double db = 0.0;
                    for (int c = 0; c < Dk; ++c) {
                        double acc = 0.0;               /* (dG + dG^T) k^ + dU^T v, times beta */
                        for (int e = 0; e < Dk; ++e)
                            acc += (dG[(size_t)c * Dk + e] + dG[(size_t)e * Dk + c]) * khi[e];
                        for (int a = 0; a < Dv; ++a) acc += Dm[(size_t)a * Dk + c] * vi[a];
                        dkh[c] = bt[i] * acc;
                        double gk = 0.0;                /* (dG k^)_c */
                        for (int e = 0; e < Dk; ++e) gk += dG[(size_t)c * Dk + e] * khi[e];
                        db += khi[c] * gk;
                    }
                    for (int a = 0; a < Dv; ++a) {
                        double uk = 0.0;                /* (dU k^)_a */
                        for (int e = 0; e < Dk; ++e) uk += Dm[(size_t)a * Dk + e] * khi[e];
                        dv[ti * Dv + a] = bt[i] * uk;
                        db += vi[a] * uk;
                    }
                    if (gates_are_logits) {
                        const double sg = sigmoid(beta[ti]);
                        db = db * sg * (1.0 - sg) / (double)N;
                    }
                    dbeta[ti] = db;
                    double *dki = dk + ti * Dk;
                    if (!normalize_k) {
                        for (int c = 0; c < Dk; ++c) dki[c] = dkh[c];
                    } else if (nrm[i] > eps) {
                        double proj = 0.0;
                        for (int c = 0; c < Dk; ++c) proj += khi[c] * dkh[c];
                        for (int c = 0; c < Dk; ++c) dki[c] = (dkh[c] - khi[c] * proj) / nrm[i];
                    } else {
                        for (int c = 0; c < Dk; ++c) dki[c] = dkh[c] / eps;
                    }
                }
                /* D <- alpha D (I - G)^T */
                for (int a = 0; a < Dv; ++a)
                    for (int c = 0; c < Dk; ++c) {
                        double t = Dm[(size_t)a * Dk + c];
                        for (int e = 0; e < Dk; ++e) t -= Dm[(size_t)a * Dk + e] * G[(size_t)c * Dk + e];
                        Dn[(size_t)a * Dk + c] = al * t;
                    }
                for (size_t x = 0; x < SS; ++x) Dm[x] = Dn[x];
            }
            if (dS0)
                for (size_t x = 0; x < SS; ++x) dS0[((size_t)b * H + h) * SS + x] = Dm[x];
        }
    }
    free(Sall); free(G); free(U); free(T); free(Dm); free(Dn); free(dG);
    free(kh); free(nrm); free(bt); free(dkh);
    }
    return status;
}
