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

/*
 * Decoupled erase and write gates (Gated DeltaNet-2 blurb: the delta rule's
 * update split into a channel-wise erase gate and a channel-wise write gate).
 * The pages give no formula; the reading taken here keeps the update rank
 * one along k and replaces the scalar beta in its two roles:
 *
 *   S_t = (I - k_t (e_t o k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t o v_t)^T
 *
 * with the erase gate e_t in R^{dk} (per key channel: how much each channel
 * of the key takes part in reading out what is erased) and the write gate
 * w_t in R^{dv} (per value channel: how much of v is written). In delta form,
 * gate first:
 *
 *   S'   = Diag(alpha_t) S_{t-1}
 *   pred = S'^T (e_t o k_t)
 *   S_t  = S' + k_t (w_t o v_t - pred)^T
 *   o_t  = S_t^T q_t
 *
 * With e_t = beta_t 1 and w_t = beta_t 1 this is the recurrence above.
 * Layouts: erase [B,T,H,dk], write [B,T,H,dv]; the rest as for
 * kda_oracle_fwd.
 */
static void erase_write_step(double *S, const double *q, const double *k, const double *v,
                             const double *alpha, int alpha_stride, const double *erase,
                             const double *write, double *o, double *pred, int dk, int dv)
{
    int i, j;
    for (i = 0; i < dk; ++i) {
        double a = alpha[i * alpha_stride];
        for (j = 0; j < dv; ++j)
            S[i * dv + j] *= a;
    }
    for (j = 0; j < dv; ++j)
        pred[j] = 0.0;
    for (i = 0; i < dk; ++i) {
        double ek = erase[i] * k[i];
        for (j = 0; j < dv; ++j)
            pred[j] += S[i * dv + j] * ek;
    }
    for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
            S[i * dv + j] += k[i] * (write[j] * v[j] - pred[j]);
    if (o) {
        for (j = 0; j < dv; ++j)
            o[j] = 0.0;
        for (i = 0; i < dk; ++i)
            for (j = 0; j < dv; ++j)
                o[j] += S[i * dv + j] * q[i];
    }
}

int kda_oracle_fwd_ew(const double *q, const double *k, const double *v, const double *gate,
                      const double *erase, const double *write, const double *S0, double *o,
                      double *S_T, int B, int H, int T, int dk, int dv, const int32_t *cu_seqlens,
                      int nseq, int gate_kind)
{
    if (!q || !k || !v || !gate || !erase || !write || !o || B <= 0 || H <= 0 || T < 0 || dk <= 0 ||
        dv <= 0)
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
        long t0, t1, b, t;
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
        for (t = t0; t < t1; ++t) {
            size_t row = ((size_t)b * T + t) * H + h;
            erase_write_step(S, q + row * dk, k + row * dk, v + row * dv, gate + row * gdim, astride,
                             erase + row * dk, write + row * dv, o + row * dv, pred, dk, dv);
        }
        if (S_T)
            memcpy(S_T + ((size_t)s * H + h) * dk * dv, S, sizeof(double) * (size_t)dk * dv);
        free(S);
        free(pred);
    }
    return 0;
}

/* One decode step with erase and write gates: erase [N,H,dk], write [N,H,dv]. */
int kda_oracle_decode_ew(const double *q, const double *k, const double *v, const double *gate,
                         const double *erase, const double *write, double *S, double *o, int N, int H,
                         int dk, int dv, int gate_kind)
{
    if (!q || !k || !v || !gate || !erase || !write || !S || !o || N <= 0 || H <= 0 || dk <= 0 ||
        dv <= 0)
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
        erase_write_step(S + (size_t)p * dk * dv, q + (size_t)p * dk, k + (size_t)p * dk,
                         v + (size_t)p * dv, gate + (size_t)p * gdim, astride, erase + (size_t)p * dk,
                         write + (size_t)p * dv, o + (size_t)p * dv, pred, dk, dv);
        free(pred);
    }
    return 0;
}

/*
 * Reverse-mode gradient of the forward above (the chain rule applied to the
 * delta form, token by token, last token first). With the loss
 *   L = sum_t <o_t, dO_t> + <S_T, dS_T>
 * it returns dL/dq, dL/dk, dL/dv, dL/dgate, dL/dbeta and dL/dS0. The pages
 * measure forward-plus-backward training throughput of this chunkwise family
 * (Complex KDA summary, efficiency) but print no backward formulas; the
 * adjoint of each forward line, in reverse order, is:
 *
 *   forward                          adjoint (dS holds dL/dS_t on entry)
 *   o    = S_t^T q                   dS += q dO^T;   dq = S_t dO
 *   S_t  = S' + k u^T                du = dS^T k;    dk = dS u;   dS' = dS
 *   u    = beta (v - pred)           dbeta = du . (v - pred);  dv = beta du;
 *                                    dpred = -beta du
 *   pred = S'^T k                    dS' += k dpred^T;  dk += S' dpred
 *   S'   = Diag(alpha) S_{t-1}       dalpha_i = sum_j dS'_ij S_{t-1,ij};
 *                                    dS_{t-1} = Diag(alpha) dS'
 *
 * For the scalar gate dalpha is summed over i as well. The states S_{t-1}
 * before every token are kept from a forward pass (len * dk * dv doubles per
 * (sequence, head)). Gradient layouts equal the input layouts; dS_T and dS0
 * are [nseq,H,dk,dv]; dS_T may be NULL (zero) and so may dS0 (not returned).
 * Returns 0, or -1 on a bad argument or failed allocation.
 */
int kda_oracle_bwd(const double *q, const double *k, const double *v, const double *gate,
                   const double *beta, const double *S0, const double *dO, const double *dS_T,
                   double *dq, double *dk_out, double *dv_out, double *dgate, double *dbeta,
                   double *dS0, int B, int H, int T, int dk, int dv, const int32_t *cu_seqlens,
                   int nseq, int gate_kind)
{
    if (!q || !k || !v || !gate || !beta || !dO || !dq || !dk_out || !dv_out || !dgate || !dbeta ||
        B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
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
    const size_t sd = (size_t)dk * dv;
    long pairs = (long)nseq * H;
    long p;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (p = 0; p < pairs; ++p) {
        int s = (int)(p / H), h = (int)(p % H);
        long t0, t1, b, t;
        int i, j;
        if (cu_seqlens) {
            b = 0;
            t0 = cu_seqlens[s];
            t1 = cu_seqlens[s + 1];
        } else {
            b = s;
            t0 = 0;
            t1 = T;
        }
        const long len = t1 - t0;
        double *hist = (double *)malloc(sizeof(double) * sd * (size_t)(len > 0 ? len : 1));
        double *S = (double *)malloc(sizeof(double) * sd);
        double *Sp = (double *)malloc(sizeof(double) * sd);
        double *dS = (double *)malloc(sizeof(double) * sd);
        double *pred = (double *)malloc(sizeof(double) * (size_t)dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *du = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!hist || !S || !Sp || !dS || !pred || !u || !du) {
            failed = 1;
        } else {
            /* forward, keeping S_{t-1} before every token */
            if (S0)
                memcpy(S, S0 + ((size_t)s * H + h) * sd, sizeof(double) * sd);
            else
                memset(S, 0, sizeof(double) * sd);
            for (t = t0; t < t1; ++t) {
                size_t row = ((size_t)b * T + t) * H + h;
                memcpy(hist + (size_t)(t - t0) * sd, S, sizeof(double) * sd);
                delta_step(S, q + row * dk, k + row * dk, v + row * dv, gate + row * gdim,
                           gdim == dk ? 1 : 0, beta[row], NULL, pred, dk, dv);
            }
            /* backward */
            if (dS_T)
                memcpy(dS, dS_T + ((size_t)s * H + h) * sd, sizeof(double) * sd);
            else
                memset(dS, 0, sizeof(double) * sd);
            for (t = t1 - 1; t >= t0; --t) {
                size_t row = ((size_t)b * T + t) * H + h;
                const double *qt = q + row * dk, *kt = k + row * dk, *vt = v + row * dv;
                const double *ot = dO + row * dv, *at = gate + row * gdim;
                const double bt = beta[row];
                const double *Sprev = hist + (size_t)(t - t0) * sd;
                double *dqt = dq + row * dk, *dkt = dk_out + row * dk, *dvt = dv_out + row * dv;
                double *dat = dgate + row * gdim;
                /* recompute S', pred, u, S_t */
                for (i = 0; i < dk; ++i) {
                    double a = at[gdim == dk ? i : 0];
                    for (j = 0; j < dv; ++j)
                        Sp[i * dv + j] = a * Sprev[i * dv + j];
                }
                for (j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dk; ++i)
                        acc += Sp[i * dv + j] * kt[i];
                    pred[j] = acc;
                    u[j] = bt * (vt[j] - acc);
                }
                for (i = 0; i < dk; ++i)
                    for (j = 0; j < dv; ++j)
                        S[i * dv + j] = Sp[i * dv + j] + kt[i] * u[j];
                /* o_t = S_t^T q_t */
                for (i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (j = 0; j < dv; ++j) {
                        dS[i * dv + j] += qt[i] * ot[j];
                        acc += S[i * dv + j] * ot[j];
                    }
                    dqt[i] = acc;
                }
                /* S_t = S' + k u^T */
                double db = 0.0;
                for (j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dk; ++i)
                        acc += dS[i * dv + j] * kt[i];
                    du[j] = acc;
                    db += acc * (vt[j] - pred[j]);
                    dvt[j] = bt * acc;
                }
                dbeta[row] = db;
                for (i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (j = 0; j < dv; ++j)
                        acc += dS[i * dv + j] * u[j];
                    dkt[i] = acc;
                }
                /* pred = S'^T k with dpred = -beta du; then S' = Diag(alpha) S_{t-1} */
                if (gdim == 1)
                    dat[0] = 0.0;
                for (i = 0; i < dk; ++i) {
                    double a = at[gdim == dk ? i : 0];
                    double acck = 0.0, acca = 0.0;
                    for (j = 0; j < dv; ++j) {
                        double dpred = -bt * du[j];
                        double dsp = dS[i * dv + j] + kt[i] * dpred;
                        acck += Sp[i * dv + j] * dpred;
                        acca += dsp * Sprev[i * dv + j];
                        dS[i * dv + j] = a * dsp;
                    }
                    dkt[i] += acck;
                    if (gdim == dk)
                        dat[i] = acca;
                    else
                        dat[0] += acca;
                }
            }
            if (dS0)
                memcpy(dS0 + ((size_t)s * H + h) * sd, dS, sizeof(double) * sd);
        }
        free(hist);
        free(S);
        free(Sp);
        free(dS);
        free(pred);
        free(u);
        free(du);
    }
    return failed ? -1 : 0;
}

/*
 * Reverse-mode gradient of kda_oracle_fwd_ew (decoupled erase and write
 * gates; reading stated above that function). With ke = e o k and
 * u = w o v - S'^T ke, the adjoint of each forward line, last token first:
 *
 *   forward                          adjoint (dS holds dL/dS_t on entry)
 *   o    = S_t^T q                   dS += q dO^T;   dq = S_t dO
 *   S_t  = S' + k u^T                du = dS^T k;    dk = dS u;   dS' = dS
 *   u    = w o v - pred              dw = du o v;    dv = du o w;  dpred = -du
 *   pred = S'^T ke                   dS' += ke dpred^T;  dke = S' dpred;
 *                                    de = dke o k;   dk += dke o e
 *   S'   = Diag(alpha) S_{t-1}       dalpha_i = sum_j dS'_ij S_{t-1,ij};
 *                                    dS_{t-1} = Diag(alpha) dS'
 *
 * Returns dL/dq, dk, dv, dgate, derase [B,T,H,dk], dwrite [B,T,H,dv] and dS0
 * for L = sum_t <o_t, dO_t> + <S_T, dS_T>; layouts and NULL conventions as
 * for kda_oracle_bwd. Returns 0, or -1 on a bad argument or failed
 * allocation.
 */
int kda_oracle_bwd_ew(const double *q, const double *k, const double *v, const double *gate,
                      const double *erase, const double *write, const double *S0, const double *dO,
                      const double *dS_T, double *dq, double *dk_out, double *dv_out, double *dgate,
                      double *derase, double *dwrite, double *dS0, int B, int H, int T, int dk, int dv,
                      const int32_t *cu_seqlens, int nseq, int gate_kind)
{
    if (!q || !k || !v || !gate || !erase || !write || !dO || !dq || !dk_out || !dv_out || !dgate ||
        !derase || !dwrite || B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0)
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
    const size_t sd = (size_t)dk * dv;
    long pairs = (long)nseq * H;
    long p;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (p = 0; p < pairs; ++p) {
        int s = (int)(p / H), h = (int)(p % H);
        long t0, t1, b, t;
        int i, j;
        if (cu_seqlens) {
            b = 0;
            t0 = cu_seqlens[s];
            t1 = cu_seqlens[s + 1];
        } else {
            b = s;
            t0 = 0;
            t1 = T;
        }
        const long len = t1 - t0;
        double *hist = (double *)malloc(sizeof(double) * sd * (size_t)(len > 0 ? len : 1));
        double *S = (double *)malloc(sizeof(double) * sd);
        double *Sp = (double *)malloc(sizeof(double) * sd);
        double *dS = (double *)malloc(sizeof(double) * sd);
        double *pred = (double *)malloc(sizeof(double) * (size_t)dv);
        double *u = (double *)malloc(sizeof(double) * (size_t)dv);
        double *du = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!hist || !S || !Sp || !dS || !pred || !u || !du) {
            failed = 1;
        } else {
            /* forward, keeping S_{t-1} before every token */
            if (S0)
                memcpy(S, S0 + ((size_t)s * H + h) * sd, sizeof(double) * sd);
            else
                memset(S, 0, sizeof(double) * sd);
            for (t = t0; t < t1; ++t) {
                size_t row = ((size_t)b * T + t) * H + h;
                memcpy(hist + (size_t)(t - t0) * sd, S, sizeof(double) * sd);
                erase_write_step(S, q + row * dk, k + row * dk, v + row * dv, gate + row * gdim,
                                 gdim == dk ? 1 : 0, erase + row * dk, write + row * dv, NULL, pred, dk, dv);
            }
            /* backward */
            if (dS_T)
                memcpy(dS, dS_T + ((size_t)s * H + h) * sd, sizeof(double) * sd);
            else
                memset(dS, 0, sizeof(double) * sd);
            for (t = t1 - 1; t >= t0; --t) {
                size_t row = ((size_t)b * T + t) * H + h;
                const double *qt = q + row * dk, *kt = k + row * dk, *vt = v + row * dv;
                const double *et = erase + row * dk, *wt = write + row * dv;
                const double *ot = dO + row * dv, *at = gate + row * gdim;
                const double *Sprev = hist + (size_t)(t - t0) * sd;
                double *dqt = dq + row * dk, *dkt = dk_out + row * dk, *dvt = dv_out + row * dv;
                double *dat = dgate + row * gdim, *det = derase + row * dk, *dwt = dwrite + row * dv;
                /* recompute S', pred, u, S_t */
                for (i = 0; i < dk; ++i) {
                    double a = at[gdim == dk ? i : 0];
                    for (j = 0; j < dv; ++j)
                        Sp[i * dv + j] = a * Sprev[i * dv + j];
                }
                for (j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dk; ++i)
                        acc += Sp[i * dv + j] * (et[i] * kt[i]);
                    pred[j] = acc;
                    u[j] = wt[j] * vt[j] - acc;
                }
                for (i = 0; i < dk; ++i)
                    for (j = 0; j < dv; ++j)
                        S[i * dv + j] = Sp[i * dv + j] + kt[i] * u[j];
                /* o_t = S_t^T q_t */
                for (i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (j = 0; j < dv; ++j) {
                        dS[i * dv + j] += qt[i] * ot[j];
                        acc += S[i * dv + j] * ot[j];
                    }
                    dqt[i] = acc;
                }
                /* S_t = S' + k u^T;  u = w o v - pred */
                for (j = 0; j < dv; ++j) {
                    double acc = 0.0;
                    for (i = 0; i < dk; ++i)
                        acc += dS[i * dv + j] * kt[i];
                    du[j] = acc;
                    dwt[j] = acc * vt[j];
                    dvt[j] = acc * wt[j];
                }
                for (i = 0; i < dk; ++i) {
                    double acc = 0.0;
                    for (j = 0; j < dv; ++j)
                        acc += dS[i * dv + j] * u[j];
                    dkt[i] = acc;
                }
                /* pred = S'^T ke with dpred = -du; then S' = Diag(alpha) S_{t-1} */
                if (gdim == 1)
                    dat[0] = 0.0;
                for (i = 0; i < dk; ++i) {
                    double a = at[gdim == dk ? i : 0];
                    double ke = et[i] * kt[i];
                    double dke = 0.0, acca = 0.0;
                    for (j = 0; j < dv; ++j) {
                        double dpred = -du[j];
                        double dsp = dS[i * dv + j] + ke * dpred;
                        dke += Sp[i * dv + j] * dpred;
                        acca += dsp * Sprev[i * dv + j];
                        dS[i * dv + j] = a * dsp;
                    }
                    det[i] = dke * kt[i];
                    dkt[i] += dke * et[i];
                    if (gdim == dk)
                        dat[i] = acca;
                    else
                        dat[0] += acca;
                }
            }
            if (dS0)
                memcpy(dS0 + ((size_t)s * H + h) * sd, dS, sizeof(double) * sd);
        }
        free(hist);
        free(S);
        free(Sp);
        free(dS);
        free(pred);
        free(u);
        free(du);
    }
    return failed ? -1 : 0;
}
