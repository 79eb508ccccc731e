/*
 * kda_oracle.c -- float64 CPU oracle for the Kimi Delta Attention (KDA)
 * recurrence.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg call it; the GPU library never links, loads
 * or calls it, and it shares no code with the GPU library.
 *
 * What it computes (one head, state S with dk rows and dv columns, row-major,
 * the dv index contiguous), token by token, in the order the pages give:
 *
 *   fade   S <- Diag(alpha_t) S,   alpha_t = exp(g_t), one factor per key
 *          channel (row of S).  "Review A - Sequence and depth", Free recall,
 *          the question on KDA's three operations (fade comes first and acts
 *          per channel); "K3 Architecture Illustrated", "Combining KDA and
 *          MLA", FIG 21 (per-channel retention precedes the delta update).
 *          g is a natural-log decay ("Kimi K3 - Lesson 3 of 14 - Sequence
 *          axis": log-decay bounded in (-5, 0), tile bound stated as e^80).
 *   erase  p = S^T k_t, the value the faded state currently returns for the
 *          key (same Free recall answer; FIG 21 text on the delta update) ...
 *   write  S <- S + beta_t k_t (v_t - p)^T, i.e. S <- (I - beta_t k_t k_t^T) S
 *          + beta_t k_t v_t^T: the stored association moves toward v_t by beta_t
 *          times the gap between v_t and p ("K3 Architecture Illustrated",
 *          section "Under what conditions are RoPE, PaTH, and KDA related?":
 *          the delta rule's transition has the factor I - beta k k^T).
 *   read   o_t = S^T q_t from the updated state (the Free recall answer puts
 *          the query product after the write; FIG 21 likewise).
 *
 * The final state after the last token is S_final.  Nothing is blocked,
 * fused or reordered: each token is the four steps above in plain loops.
 *
 * Layouts (all float64, contiguous):
 *   q, k, g : [B][T][H][dk]     v, o : [B][T][H][dv]     beta : [B][T][H]
 *   S0, S_final, S : [B][H][dk][dv]
 * Heads (b, h) are independent; OpenMP runs them in parallel.
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* One token on one head.  S is dk x dv, updated in place; o receives dv values.
   q, k, g have dk values; v has dv values.  p is dv doubles of workspace. */
static void kda_token(double *S, int dk, int dv,
                      const double *q, const double *k, const double *v,
                      const double *g, double beta, double *o, double *p)
{
    /* fade: every key channel (row of S) by its own retention exp(g) */
    for (int i = 0; i < dk; ++i) {
        const double alpha = exp(g[i]);
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] *= alpha;
    }
    /* erase: the value the faded state returns for the key, p = S^T k */
    for (int j = 0; j < dv; ++j)
        p[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            p[j] += S[(size_t)i * dv + j] * k[i];
    /* write: S += beta k (v - p)^T */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            S[(size_t)i * dv + j] += beta * k[i] * (v[j] - p[j]);
    /* read from the updated state: o = S^T q */
    for (int j = 0; j < dv; ++j)
        o[j] = 0.0;
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            o[j] += S[(size_t)i * dv + j] * q[i];
}

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Token-by-token forward over T tokens for every head.
   S0 may be NULL (zero initial state); S_final may be NULL (not written).
   Returns 0, or -1 on bad sizes / allocation failure. */
int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *S0,
                   double *o, double *S_final,
                   int B, int T, int H, int dk, int dv, int nthreads)
{
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    set_threads(nthreads);
    int err = 0;
    const size_t sz = (size_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        double *S = (double *)malloc(sz * sizeof(double));
        double *p = (double *)malloc((size_t)dv * sizeof(double));
        if (!S || !p) {
            free(S);
            free(p);
            err |= 1;
            continue;
        }
        if (S0)
            memcpy(S, S0 + (size_t)bh * sz, sz * sizeof(double));
        else
            memset(S, 0, sz * sizeof(double));
        for (int t = 0; t < T; ++t) {
            const size_t row = ((size_t)b * T + t) * H + h;
            kda_token(S, dk, dv, q + row * dk, k + row * dk, v + row * dv,
                      g + row * dk, beta[row], o + row * dv, p);
        }
        if (S_final)
            memcpy(S_final + (size_t)bh * sz, S, sz * sizeof(double));
        free(S);
        free(p);
    }
    return err ? -1 : 0;
}

/* One decode step for every head: S [B][H][dk][dv] updated in place,
   q, k, g : [B][H][dk], v, o : [B][H][dv], beta : [B][H]. */
int kda_oracle_decode(const double *q, const double *k, const double *v,
                      const double *g, const double *beta, double *S, double *o,
                      int B, int H, int dk, int dv, int nthreads)
{
    if (B < 0 || H < 0 || dk <= 0 || dv <= 0)
        return -1;
    set_threads(nthreads);
    int err = 0;
    const size_t sz = (size_t)dk * dv;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : err)
    for (int bh = 0; bh < B * H; ++bh) {
        double *p = (double *)malloc((size_t)dv * sizeof(double));
        if (!p) {
            err |= 1;
            continue;
        }
        kda_token(S + (size_t)bh * sz, dk, dv, q + (size_t)bh * dk,
                  k + (size_t)bh * dk, v + (size_t)bh * dv, g + (size_t)bh * dk,
                  beta[bh], o + (size_t)bh * dv, p);
        free(p);
    }
    return err ? -1 : 0;
}

/* Threads an OpenMP parallel region would use (1 without OpenMP). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
