/*
 * The C ABI used from plain C: only include/kda.h and the HIP runtime's C API,
 * no Python and no torch. Seeded fp32 inputs (a 64-bit LCG, values in the
 * configurations' ranges: unit-norm q and k, Complex-KDA-range gates with
 * exact zeros and -1, beta in [0, 2]) go through kda_chunk_fwd (fixed-length
 * batch and packed sequences) and kda_decode_step in libkda.so, and the
 * results are compared with the fp64 oracle (kda_oracle_fwd,
 * kda_oracle_decode) linked into the same program: max|x - ref| / rms(ref)
 * within 1e-4 (fp32 inputs). TEST INFRASTRUCTURE: built by the package's
 * build step, run by tests/test_gpu_c_abi.py. Prints one line per case and
 * exits 0 when every case passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "kda.h"

int kda_oracle_fwd(const double *q, const double *k, const double *v, const double *gate,
                   const double *beta, const double *S0, double *o, double *S_T, int B, int H, int T,
                   int dk, int dv, const int32_t *cu_seqlens, int nseq, int gate_kind);
int kda_oracle_decode(const double *q, const double *k, const double *v, const double *gate,
                      const double *beta, double *S, double *o, int N, int H, int dk, int dv,
                      int gate_kind);

static uint64_t rng_state;

static double uniform01(void) {
    rng_state = rng_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (double)(rng_state >> 11) * (1.0 / 9007199254740992.0);
}

static double normal01(void) {   /* Box-Muller */
    double u = uniform01(), w = uniform01();
    if (u < 1e-300) u = 1e-300;
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * w);
}

/* rows of width d, each scaled to unit norm, rounded to fp32 */
static void unit_rows(float *x, long rows, int d) {
    for (long r = 0; r < rows; ++r) {
        double n = 0.0, t[256];
        for (int i = 0; i < d; ++i) {
            t[i] = normal01();
            n += t[i] * t[i];
        }
        n = sqrt(n);
        for (int i = 0; i < d; ++i) x[r * d + i] = (float)(t[i] / n);
    }
}

static void to_f64(const float *x, double *y, size_t n) {
    for (size_t i = 0; i < n; ++i) y[i] = (double)x[i];
}

static double rel_err(const float *x, const double *ref, size_t n) {
    double d = 0.0, s = 0.0;
    for (size_t i = 0; i < n; ++i) {
        double e = fabs((double)x[i] - ref[i]);
        if (e > d || e != e) d = e;
        s += ref[i] * ref[i];
    }
    s = sqrt(s / (double)n);
    return s > 0.0 ? d / s : d;
}

#define CHECK_HIP(x)                                                      \
    do {                                                                  \
        hipError_t e_ = (x);                                              \
        if (e_ != hipSuccess) {                                           \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));       \
            return 1;                                                     \
        }                                                                 \
    } while (0)

static void *dev_copy(const void *h, size_t bytes) {
    void *d = NULL;
    if (hipMalloc(&d, bytes ? bytes : 4) != hipSuccess) return NULL;
    if (bytes && hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
    return d;
}

/* One forward case: B sequences of length T (cu == NULL) or nseq packed ones. */
static int forward_case(const char *name, int B, int H, int T, int dk, int dv, int chunk, const int32_t *cu,
                        int nseq) {
    const int N = cu ? nseq : B;
    const long rows = (long)B * T * H;
    float *q = malloc(sizeof(float) * rows * dk), *k = malloc(sizeof(float) * rows * dk);
    float *v = malloc(sizeof(float) * rows * dv), *g = malloc(sizeof(float) * rows * dk);
    float *b = malloc(sizeof(float) * rows), *S0 = malloc(sizeof(float) * (size_t)N * H * dk * dv);
    unit_rows(q, rows, dk);
    unit_rows(k, rows, dk);
    for (long i = 0; i < rows * dv; ++i) v[i] = (float)normal01();
    for (long i = 0; i < rows * dk; ++i) {
        double u = uniform01();
        g[i] = u < 0.01 ? 0.0f : (u < 0.02 ? -1.0f : (float)(2.0 * uniform01() - 1.0));
    }
    for (long i = 0; i < rows; ++i) b[i] = uniform01() < 0.01 ? 2.0f : (float)(2.0 * uniform01());
    for (long i = 0; i < (long)N * H * dk * dv; ++i) S0[i] = (float)(0.3 * normal01());

    const size_t sz_o = (size_t)rows * dv, sz_s = (size_t)N * H * dk * dv;
    float *o = malloc(sizeof(float) * sz_o), *ST = malloc(sizeof(float) * sz_s);
    void *dq = dev_copy(q, sizeof(float) * rows * dk), *dk_ = dev_copy(k, sizeof(float) * rows * dk);
    void *dv_ = dev_copy(v, sizeof(float) * rows * dv), *dg = dev_copy(g, sizeof(float) * rows * dk);
    void *db = dev_copy(b, sizeof(float) * rows), *dS0 = dev_copy(S0, sizeof(float) * sz_s);
    void *dcu = cu ? dev_copy(cu, sizeof(int32_t) * (size_t)(nseq + 1)) : NULL;
    void *dout = NULL, *dST = NULL, *ws = NULL;
    const size_t wsb = kda_chunk_fwd_workspace_bytes(B, H, T, dk, dv, chunk, cu ? nseq : 0, cu != NULL, KDA_F32);
    if (!dq || !dk_ || !dv_ || !dg || !db || !dS0 || (cu && !dcu) || wsb == 0 ||
        hipMalloc(&dout, sizeof(float) * sz_o) != hipSuccess || hipMalloc(&dST, sizeof(float) * sz_s) != hipSuccess ||
        hipMalloc(&ws, wsb) != hipSuccess) {
        fprintf(stderr, "%s: allocation failed\n", name);
        return 1;
    }
    int rc = kda_chunk_fwd(dq, dk_, dv_, dg, db, (const float *)dS0, (float *)dout, (float *)dST, B, H, T, dk, dv,
                           chunk, (const int32_t *)dcu, cu ? nseq : 0, KDA_F32, KDA_GATE_CHANNEL, ws, wsb, NULL);
    if (rc != KDA_OK) {
        fprintf(stderr, "%s: kda_chunk_fwd: %s\n", name, kda_strerror(rc));
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(o, dout, sizeof(float) * sz_o, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(ST, dST, sizeof(float) * sz_s, hipMemcpyDeviceToHost));
    uint32_t status = 0;
    CHECK_HIP(hipMemcpy(&status, ws, sizeof(status), hipMemcpyDeviceToHost));

    double *q8 = malloc(sizeof(double) * rows * dk), *k8 = malloc(sizeof(double) * rows * dk);
    double *v8 = malloc(sizeof(double) * rows * dv), *g8 = malloc(sizeof(double) * rows * dk);
    double *b8 = malloc(sizeof(double) * rows), *S08 = malloc(sizeof(double) * sz_s);
    double *ro = malloc(sizeof(double) * sz_o), *rS = malloc(sizeof(double) * sz_s);
    to_f64(q, q8, rows * dk);
    to_f64(k, k8, rows * dk);
    to_f64(v, v8, rows * dv);
    to_f64(g, g8, rows * dk);
    to_f64(b, b8, rows);
    to_f64(S0, S08, sz_s);
    if (kda_oracle_fwd(q8, k8, v8, g8, b8, S08, ro, rS, B, H, T, dk, dv, cu, nseq, 0) != 0) {
        fprintf(stderr, "%s: oracle rejected its arguments\n", name);
        return 1;
    }
    const double eo = rel_err(o, ro, sz_o), eS = rel_err(ST, rS, sz_s);
    const int ok = eo <= 1e-4 && eS <= 1e-4 && kda_chunk_fwd_status(status) == KDA_OK;
    printf("%s: B=%d H=%d T=%d dk=%d dv=%d chunk=%d sequences=%d  err o %.2e S_T %.2e  %s\n", name, B, H, T, dk, dv,
           chunk, N, eo, eS, ok ? "ok" : "FAILED");
    hipFree(dq), hipFree(dk_), hipFree(dv_), hipFree(dg), hipFree(db), hipFree(dS0), hipFree(dout), hipFree(dST);
    hipFree(ws);
    if (dcu) hipFree(dcu);
    free(q), free(k), free(v), free(g), free(b), free(S0), free(o), free(ST);
    free(q8), free(k8), free(v8), free(g8), free(b8), free(S08), free(ro), free(rS);
    return ok ? 0 : 1;
}

static int decode_case(int N, int H, int dk, int dv, int steps) {
    const long rows = (long)N * H;
    const size_t sz_s = (size_t)rows * dk * dv;
    float *S = malloc(sizeof(float) * sz_s), *o = malloc(sizeof(float) * rows * dv);
    double *S8 = malloc(sizeof(double) * sz_s), *ro = malloc(sizeof(double) * rows * dv);
    for (size_t i = 0; i < sz_s; ++i) S[i] = (float)(0.3 * normal01());
    to_f64(S, S8, sz_s);
    void *dS = dev_copy(S, sizeof(float) * sz_s), *dout = NULL;
    if (!dS || hipMalloc(&dout, sizeof(float) * rows * dv) != hipSuccess) return 1;
    double worst = 0.0;
    for (int st = 0; st < steps; ++st) {
        float *q = malloc(sizeof(float) * rows * dk), *k = malloc(sizeof(float) * rows * dk);
        float *v = malloc(sizeof(float) * rows * dv), *g = malloc(sizeof(float) * rows * dk);
        float *b = malloc(sizeof(float) * rows);
        unit_rows(q, rows, dk);
        unit_rows(k, rows, dk);
        for (long i = 0; i < rows * dv; ++i) v[i] = (float)normal01();
        for (long i = 0; i < rows * dk; ++i) g[i] = (float)(2.0 * uniform01() - 1.0);
        for (long i = 0; i < rows; ++i) b[i] = (float)(2.0 * uniform01());
        void *dq = dev_copy(q, sizeof(float) * rows * dk), *dk_ = dev_copy(k, sizeof(float) * rows * dk);
        void *dv_ = dev_copy(v, sizeof(float) * rows * dv), *dg = dev_copy(g, sizeof(float) * rows * dk);
        void *db = dev_copy(b, sizeof(float) * rows);
        if (!dq || !dk_ || !dv_ || !dg || !db) return 1;
        int rc = kda_decode_step(dq, dk_, dv_, dg, db, (float *)dS, (float *)dout, N, H, dk, dv, KDA_F32,
                                 KDA_GATE_CHANNEL, NULL);
        if (rc != KDA_OK) {
            fprintf(stderr, "decode: %s\n", kda_strerror(rc));
            return 1;
        }
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(o, dout, sizeof(float) * rows * dv, hipMemcpyDeviceToHost));
        double *q8 = malloc(sizeof(double) * rows * dk), *k8 = malloc(sizeof(double) * rows * dk);
        double *v8 = malloc(sizeof(double) * rows * dv), *g8 = malloc(sizeof(double) * rows * dk);
        double *b8 = malloc(sizeof(double) * rows);
        to_f64(q, q8, rows * dk);
        to_f64(k, k8, rows * dk);
        to_f64(v, v8, rows * dv);
        to_f64(g, g8, rows * dk);
        to_f64(b, b8, rows);
        if (kda_oracle_decode(q8, k8, v8, g8, b8, S8, ro, N, H, dk, dv, 0) != 0) return 1;
        const double e = rel_err(o, ro, (size_t)rows * dv);
        if (e > worst || e != e) worst = e;
        hipFree(dq), hipFree(dk_), hipFree(dv_), hipFree(dg), hipFree(db);
        free(q), free(k), free(v), free(g), free(b), free(q8), free(k8), free(v8), free(g8), free(b8);
    }
    CHECK_HIP(hipMemcpy(S, dS, sizeof(float) * sz_s, hipMemcpyDeviceToHost));
    const double eS = rel_err(S, S8, sz_s);
    const int ok = worst <= 1e-4 && eS <= 1e-4;
    printf("decode: N=%d H=%d dk=%d dv=%d steps=%d  worst err o %.2e S %.2e  %s\n", N, H, dk, dv, steps, worst, eS,
           ok ? "ok" : "FAILED");
    hipFree(dS), hipFree(dout);
    free(S), free(o), free(S8), free(ro);
    return ok ? 0 : 1;
}

int main(void) {
    int dev_count = 0;
    CHECK_HIP(hipGetDeviceCount(&dev_count));
    if (dev_count < 1) {
        fprintf(stderr, "no GPU\n");
        return 2;
    }
    printf("libkda version %d\n", kda_version());
    rng_state = 20261204ULL;
    int fails = 0;
    fails += forward_case("forward", 2, 3, 157, 64, 32, 32, NULL, 0);
    fails += forward_case("forward", 1, 2, 300, 128, 64, 64, NULL, 0);
    const int32_t cu[5] = {0, 37, 37, 38, 171};
    fails += forward_case("forward packed", 1, 2, 171, 32, 16, 16, cu, 4);
    fails += decode_case(5, 3, 64, 32, 4);
    printf("%s\n", fails ? "FAILED" : "all cases ok");
    return fails ? 1 : 0;
}
