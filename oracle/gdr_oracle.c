/*
 * gdr_oracle.c -- fp64 CPU oracle for the gated delta-rule forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU library is checked against.  It is plain C, slow on purpose, shares no
 * code, header, table or helper with the HIP library, and must never be
 * linked into, loaded by, or called from the product path.  Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark use it.
 *
 * What it computes (one independent recurrence per (batch, head) pair):
 * the state S is a d_k x d_v matrix (row i = key channel i, d_v contiguous),
 * the orientation in which the Kaczmarz page writes the constraint S^T k = v
 * (gist.science "Kaczmarz Linear Attention", section "Derivazione Teorica").
 * The blog summary and the textbook page write the transposed d_v x d_k
 * state; the two give identical numbers.
 *
 * For t = 0 .. T-1, starting from S = s0 (or zero):
 *   1. a_t = exp(g_t), a scalar (Gated DeltaNet) or one value per key channel
 *      (Kimi Delta Attention).  Storing g = log(alpha) <= 0 and exponentiating
 *      is the convention stated in the blog summary, section on the DPLR form.
 *   2. S~ = Diag(a_t) S : forget first.  The blog summary (Gated DeltaNet and
 *      KDA sections) orders the steps forget -> predict -> correct -> write;
 *      per key channel the decay scales a row of the d_k x d_v state, which is
 *      the right-multiplication S D_t of the d_v x d_k form (textbook page,
 *      GLA gate paragraph).
 *   3. beta_t as given, or the Kaczmarz step beta_t = eta_t / (||k_t||^2 + eps)
 *      (Kaczmarz page, "La Regola di Aggiornamento KLA").
 *   4. p_t = S~^T k_t : the prediction, taken AFTER the decay (blog summary,
 *      Gated DeltaNet section: predicting before the forget step is wrong).
 *   5. e_t = v_t - p_t : the residual (Kaczmarz page, same section).
 *   6. S = S~ + beta_t k_t e_t^T : rank-1 write of the residual.
 *   7. o_t = scale * S^T q_t : the read happens after the write, so the token
 *      sees its own write (textbook page, the read o_t = S_t q_t; blog
 *      summary, KDA step 5 and the chunked-output section where the diagonal
 *      of the read matrix is kept).
 *
 * delta_off (oracle-only switch) replaces steps 3-6 with the plain additive
 * write S = S~ + k_t v_t^T of linear attention / RetNet / Mamba-2 / GLA
 * (textbook page, update table).  It exists so that tests can pin the read
 * and decay arithmetic against brute-force causal attention.
 *
 * Inputs are float32 arrays holding exactly the values the GPU receives
 * (bf16 inputs are exactly representable in float32); all arithmetic is in
 * double.  Layouts: q,k [B,T,H,Dk]; v [B,T,H,Dv]; g [B,T,H] (scalar decay)
 * or [B,T,H,Dk] (per-channel decay); beta_or_eta [B,T,H]; s0 [B,H,Dk,Dv]
 * (may be NULL for a zero start).  Outputs: o [B,T,H,Dv] and s_final
 * [B,H,Dk,Dv], both double.  Only the flattened (b*H + h) pairs listed in
 * bh_list (all pairs when bh_list is NULL) are computed; the rest of o and
 * s_final is left untouched.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdr_oracle_abi(void) { return 1; }

int gdr_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static void oracle_one_pair(long b, long h, long B, long T, long H, long Dk, long Dv,
                            const float *q, const float *k, const float *v,
                            const float *g, const float *beta_or_eta,
                            int per_channel, int kaczmarz, double eps, double scale,
                            int delta_off, const float *s0, double *o, double *s_final,
                            double *S, double *p, double *e)
{
    (void)B;
    const size_t state_off = ((size_t)b * H + h) * Dk * Dv;
    if (s0) {
        for (long x = 0; x < Dk * Dv; ++x) S[x] = (double)s0[state_off + x];
    } else {
        memset(S, 0, sizeof(double) * Dk * Dv);
    }

    for (long t = 0; t < T; ++t) {
        const size_t row = ((size_t)b * T + t) * H + h;  /* (b, t, h) */
        const float *qt = q + row * Dk;
        const float *kt = k + row * Dk;
        const float *vt = v + row * Dv;
        double *ot = o + row * Dv;

        /* steps 1-2: forget */
        if (per_channel) {
            const float *gt = g + row * Dk;
            for (long i = 0; i < Dk; ++i) {
                const double a = exp((double)gt[i]);
                double *Si = S + i * Dv;
                for (long j = 0; j < Dv; ++j) Si[j] *= a;
            }
        } else {
            const double a = exp((double)g[row]);
            for (long x = 0; x < Dk * Dv; ++x) S[x] *= a;
        }

        if (delta_off) {
            /* plain additive write S = S~ + k v^T */
            for (long i = 0; i < Dk; ++i) {
                const double ki = (double)kt[i];
                double *Si = S + i * Dv;
                for (long j = 0; j < Dv; ++j) Si[j] += ki * (double)vt[j];
            }
        } else {
            /* step 3: write strength */
            double beta;
            if (kaczmarz) {
                double kk = 0.0;
                for (long i = 0; i < Dk; ++i) kk += (double)kt[i] * (double)kt[i];
                beta = (double)beta_or_eta[row] / (kk + eps);
            } else {
                beta = (double)beta_or_eta[row];
            }
            /* step 4: predict from the decayed state */
            for (long j = 0; j < Dv; ++j) p[j] = 0.0;
            for (long i = 0; i < Dk; ++i) {
                const double ki = (double)kt[i];
                const double *Si = S + i * Dv;
                for (long j = 0; j < Dv; ++j) p[j] += Si[j] * ki;
            }
            /* step 5: residual */
            for (long j = 0; j < Dv; ++j) e[j] = (double)vt[j] - p[j];
            /* step 6: rank-1 write */
            for (long i = 0; i < Dk; ++i) {
                const double bki = beta * (double)kt[i];
                double *Si = S + i * Dv;
                for (long j = 0; j < Dv; ++j) Si[j] += bki * e[j];
            }
        }

        /* step 7: read after write */
        for (long j = 0; j < Dv; ++j) p[j] = 0.0;
        for (long i = 0; i < Dk; ++i) {
            const double qi = (double)qt[i];
            const double *Si = S + i * Dv;
            for (long j = 0; j < Dv; ++j) p[j] += Si[j] * qi;
        }
        for (long j = 0; j < Dv; ++j) ot[j] = scale * p[j];
    }

    for (long x = 0; x < Dk * Dv; ++x) s_final[state_off + x] = S[x];
}

/* Returns 0 on success, -1 on a bad argument, -2 when memory runs out. */
int gdr_oracle_fwd(long B, long T, long H, long Dk, long Dv,
                   const float *q, const float *k, const float *v,
                   const float *g, const float *beta_or_eta,
                   int per_channel, int kaczmarz, double eps, double scale,
                   int delta_off, const float *s0,
                   double *o, double *s_final,
                   const long *bh_list, long n_bh, int n_threads)
{
    if (B < 1 || T < 0 || H < 1 || Dk < 1 || Dv < 1) return -1;
    if (!q || !k || !v || !g || !o || !s_final) return -1;
    if (!delta_off && !beta_or_eta) return -1;
    const long total = bh_list ? n_bh : B * H;
    int bad = 0;
    int oom = 0;
#ifdef _OPENMP
    if (n_threads < 1) n_threads = omp_get_max_threads();
#pragma omp parallel num_threads(n_threads) reduction(|| : bad, oom)
#endif
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)Dk * Dv);
        double *p = (double *)malloc(sizeof(double) * (size_t)Dv);
        double *e = (double *)malloc(sizeof(double) * (size_t)Dv);
        const int have_mem = (S && p && e);
        if (!have_mem) oom = 1;
        /* every thread reaches the worksharing loop, with or without memory */
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long x = 0; x < total; ++x) {
            const long bh = bh_list ? bh_list[x] : x;
            if (bh < 0 || bh >= B * H) { bad = 1; continue; }
            if (!have_mem) continue;
            oracle_one_pair(bh / H, bh % H, B, T, H, Dk, Dv, q, k, v, g, beta_or_eta,
                            per_channel, kaczmarz, eps, scale, delta_off, s0, o, s_final,
                            S, p, e);
        }
        free(S);
        free(p);
        free(e);
    }
    (void)n_threads;
    if (oom) return -2;
    return bad ? -1 : 0;
}
