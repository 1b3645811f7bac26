/*
 * fp64 CPU oracle for the gated delta-rule recurrence (KDA / Complex KDA / GDN).
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code with
 * the HIP path.
 *
 * What it computes, token by token, for one sequence and one head with state
 * S in R^{dk x dv} (rows indexed by key channel, columns by value channel):
 *
 *   transition  A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
 *     (Complex KDA summary, background "diagonal-plus-rank-one transitions";
 *      the gate acts first and the rank-one delta term second)
 *   update      S_t = A_t S_{t-1} + beta_t k_t v_t^T
 *   readout     o_t = S_t^T q_t        (key-side read, Dual DeltaNet abstract)
 *
 * written in the equivalent delta form of the CyFA blog post, section 2.2,
 * with the gate applied first:
 *
 *   S'   = Diag(alpha_t) S_{t-1}
 *   pred = S'^T k_t
 *   S_t  = S' + beta_t k_t (v_t - pred)^T
 *   o_t  = S_t^T q_t
 *
 * For the scalar gate (GDN) alpha_t is one number per (token, head) applied
 * to every key channel. No query scaling and no key normalisation happen here.
 *
 * Layouts (row-major, fp64): q, k [B,T,H,dk]; v [B,T,H,dv]; gate [B,T,H,dk]
 * or [B,T,H]; beta [B,T,H]; o [B,T,H,dv]; S0, S_T [nseq,H,dk,dv]. With
 * cu_seqlens (nseq+1 offsets into T) B must be 1 and each packed sequence
 * starts from its own S0 (or zeros).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GATE_CHANNEL 0
#define GATE_SCALAR 1

/* One token of the recurrence on a dk x dv state, in place. */
static void delta_step(double *S, const double *q, const double *k, const double *v,
                       const double *alpha, int alpha_stride, double beta,
                       double *o, double *pred, int dk, int dv)
{
    int i, j;
    for (i = 0; i < dk; ++i) {
        double a = alpha[i * alpha_stride];
        for (j = 0; j < dv; ++j)
            S[i * dv + j] *= a;
    }
    for (j = 0; j < dv; ++j)
        pred[j] = 0.0;
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            pred[j] += S[i * dv + j] * k[i];
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            S[i * dv + j] += beta * k[i] * (v[j] - pred[j]);
    if (o) {
        for (j = 0; j < dv; ++j)
            o[j] = 0.0;
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                o[j] += S[i * dv + j] * q[i];
    }
}

/*
 * Forward over whole sequences. Returns 0, or -1 on a bad argument.
 * S0 and S_T may be NULL (zeros in / no state out).
 */
int kda_oracle_fwd(const double *q, const double *k, const double *v, const double *gate,
                   const double *beta, const double *S0, double *o, double *S_T,
                   int B, int H, int T, int dk, int dv, const int32_t *cu_seqlens, int nseq,
                   int gate_kind)
{
    if (!q || !k || !v || !gate || !beta || !o || B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
        return -1;
    if (gate_kind != GATE_CHANNEL && gate_kind != GATE_SCALAR)
        return -1;
    if (cu_seqlens) {
        if (B != 1 || nseq <= 0 || cu_seqlens[0] != 0 || cu_seqlens[nseq] != T)
            return -1;
    } else {
        nseq = B;
    }
    const int gdim = gate_kind == GATE_CHANNEL ? dk : 1;
    const int astride = gate_kind == GATE_CHANNEL ? 1 : 0;
    long pairs = (long)nseq * H;
    long p;
#pragma omp parallel for schedule(dynamic, 1)
    for (p = 0; p < pairs; ++p) {
        int s = (int)(p / H), h = (int)(p % H);
        long t0, t1, b;
        if (cu_seqlens) {
            b = 0;
            t0 = cu_seqlens[s];
            t1 = cu_seqlens[s + 1];
        } else {
            b = s;
            t0 = 0;
            t1 = T;
        }
        double *S = (double *)malloc(sizeof(double) * (size_t)dk * dv);
        double *pred = (double *)malloc(sizeof(double) * (size_t)dv);
        if (S0)
            memcpy(S, S0 + ((size_t)s * H + h) * dk * dv, sizeof(double) * (size_t)dk * dv);
        else
            memset(S, 0, sizeof(double) * (size_t)dk * dv);
        long t;
        for (t = t0; t < t1; ++t) {
            size_t row = ((size_t)b * T + t) * H + h;
            delta_step(S, q + row * dk, k + row * dk, v + row * dv, gate + row * gdim, astride,
                       beta[row], o + row * dv, pred, dk, dv);
        }
        if (S_T)
            memcpy(S_T + ((size_t)s * H + h) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(pred);
    }
    return 0;
}

/*
 * One recurrent decode step for N independent sequences, state updated in
 * place. q, k, gate [N,H,dk] (gate [N,H] when scalar); v [N,H,dv]; beta [N,H];
 * S [N,H,dk,dv]; o [N,H,dv].
 */
int kda_oracle_decode(const double *q, const double *k, const double *v, const double *gate,
                      const double *beta, double *S, double *o, int N, int H, int dk, int dv,
                      int gate_kind)
{
    if (!q || !k || !v || !gate || !beta || !S || !o || N <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return -1;
    if (gate_kind != GATE_CHANNEL && gate_kind != GATE_SCALAR)
        return -1;
    const int gdim = gate_kind == GATE_CHANNEL ? dk : 1;
    const int astride = gate_kind == GATE_CHANNEL ? 1 : 0;
    long pairs = (long)N * H;
    long p;
#pragma omp parallel for schedule(static)
    for (p = 0; p < pairs; ++p) {
        double *pred = (double *)malloc(sizeof(double) * (size_t)dv);
        delta_step(S + (size_t)p * dk * dv, q + (size_t)p * dk, k + (size_t)p * dk,
                   v + (size_t)p * dv, gate + (size_t)p * gdim, astride, beta[p],
                   o + (size_t)p * dv, pred, dk, dv);
        free(pred);
    }
    return 0;
}
