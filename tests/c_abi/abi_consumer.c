/*
 * A plain C consumer of libfp4 (include/fp4.h): the library used through its
 * C ABI alone, with the HIP runtime for device memory, checked against the C
 * oracle (test infrastructure). Quantizes X (64 x 256) and W (48 x 256) to
 * NVFP4 with round-to-nearest, multiplies them (Y = X W^T, FP32 out), and
 * compares the codes, scale bytes and tensor scales bit for bit and Y within
 * 1e-5 * sum |a_k b_k| per element. Exit status 0 and "abi consumer ok" on
 * success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fp4.h"
#include "fp4_oracle.h"

#define CHECK_HIP(x)                                                             \
    do {                                                                         \
        hipError_t e_ = (x);                                                     \
        if (e_ != hipSuccess) {                                                  \
            fprintf(stderr, "HIP error %d at line %d\n", (int)e_, __LINE__);     \
            return 2;                                                            \
        }                                                                        \
    } while (0)
#define CHECK_FP4(x)                                                             \
    do {                                                                         \
        fp4_status s_ = (x);                                                     \
        if (s_ != FP4_OK) {                                                      \
            fprintf(stderr, "fp4 error: %s at line %d\n", fp4_status_str(s_), __LINE__); \
            return 3;                                                            \
        }                                                                        \
    } while (0)

enum { M = 64, N = 48, K = 256 };

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double next_uniform(void)
{
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 9007199254740992.0;
}

typedef struct {
    uint8_t* codes;
    uint8_t* scales;
    float* amax;
    float* tscale;
} dev_q;

static int quantize_one(const float* host, int rows, fp4_tensor* t, dev_q* d, float** dsrc)
{
    CHECK_HIP(hipMalloc((void**)dsrc, sizeof(float) * rows * K));
    CHECK_HIP(hipMemcpy(*dsrc, host, sizeof(float) * rows * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMalloc((void**)&d->codes, fp4_codes_bytes(rows, K)));
    CHECK_HIP(hipMalloc((void**)&d->scales, fp4_scales_bytes(rows, K, FP4_NVFP4)));
    CHECK_HIP(hipMalloc((void**)&d->amax, 4));
    CHECK_HIP(hipMalloc((void**)&d->tscale, 4));
    memset(t, 0, sizeof(*t));
    t->codes = d->codes;
    t->scales = d->scales;
    t->amax = d->amax;
    t->tscale = d->tscale;
    t->fmt = FP4_NVFP4;
    CHECK_FP4(fp4_quantize(*dsrc, FP4_DTYPE_F32, rows, K, K, FP4_AXIS_COLS, FP4_RTN, 0, 0, 0, t, NULL));
    return 0;
}

static int compare_quant(const fp4_tensor* t, int rows, const float* host, const char* name)
{
    size_t nc = fp4_codes_bytes(rows, K), ns = fp4_scales_bytes(rows, K, FP4_NVFP4);
    uint8_t* gc = malloc(nc);
    uint8_t* gs = malloc(ns);
    uint8_t* oc = calloc(nc, 1);
    uint8_t* os = calloc(ns, 1);
    float gsg = 0, oam = 0, osg = 0;
    CHECK_HIP(hipMemcpy(gc, t->codes, nc, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gs, t->scales, ns, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&gsg, t->tscale, 4, hipMemcpyDeviceToHost));
    if (o_quantize(host, 0, rows, K, K, O_AXIS_COLS, O_FMT_NVFP4, O_RTN, 0, 0, 0, 0, 0, 0.0f, oc, os,
                   &oam, &osg) != 0) {
        fprintf(stderr, "%s: oracle rejected the input\n", name);
        return 4;
    }
    int bad = memcmp(gc, oc, nc) != 0 || memcmp(gs, os, ns) != 0 || gsg != osg;
    free(gc); free(gs); free(oc); free(os);
    if (bad) {
        fprintf(stderr, "%s: GPU quantization differs from the oracle\n", name);
        return 5;
    }
    return 0;
}

int main(void)
{
    static float x[M * K], w[N * K];
    for (int i = 0; i < M * K; ++i) x[i] = (float)(4.0 * (next_uniform() - 0.5));
    for (int i = 0; i < N * K; ++i) w[i] = (float)(0.1 * (next_uniform() - 0.5));
    x[5 * K + 7] = 40.0f; /* an outlier */

    fp4_tensor tx, tw;
    dev_q dx, dw;
    float *sx, *sw, *dy;
    int rc;
    if ((rc = quantize_one(x, M, &tx, &dx, &sx))) return rc;
    if ((rc = quantize_one(w, N, &tw, &dw, &sw))) return rc;
    CHECK_HIP(hipMalloc((void**)&dy, sizeof(float) * M * N));
    CHECK_FP4(fp4_gemm(&tx, &tw, FP4_DTYPE_F32, dy, N, NULL));
    static float y[M * N];
    CHECK_HIP(hipMemcpy(y, dy, sizeof(y), hipMemcpyDeviceToHost)); /* synchronizes the null stream */

    if ((rc = compare_quant(&tx, M, x, "X"))) return rc;
    if ((rc = compare_quant(&tw, N, w, "W"))) return rc;

    /* reference: FP64 product of the oracle's exact dequantizations */
    static uint8_t cx[M * K / 2], scx[M * K / 16], cw[N * K / 2], scw[N * K / 16];
    static double ax[M * K], bw[N * K];
    float amx, sgx, amw, sgw;
    o_quantize(x, 0, M, K, K, O_AXIS_COLS, O_FMT_NVFP4, O_RTN, 0, 0, 0, 0, 0, 0.0f, cx, scx, &amx, &sgx);
    o_quantize(w, 0, N, K, K, O_AXIS_COLS, O_FMT_NVFP4, O_RTN, 0, 0, 0, 0, 0, 0.0f, cw, scw, &amw, &sgw);
    o_dequantize_f64(cx, scx, M, K, O_FMT_NVFP4, sgx, ax);
    o_dequantize_f64(cw, scw, N, K, O_FMT_NVFP4, sgw, bw);
    double worst = 0.0;
    for (int i = 0; i < M; ++i)
        for (int j = 0; j < N; ++j) {
            double ref = 0.0, s = 0.0;
            for (int k = 0; k < K; ++k) {
                ref += ax[i * K + k] * bw[j * K + k];
                s += fabs(ax[i * K + k] * bw[j * K + k]);
            }
            double err = fabs((double)y[i * N + j] - ref);
            double frac = s > 0 ? err / (1e-5 * s) : (err == 0 ? 0 : INFINITY);
            if (frac > worst) worst = frac;
        }
    if (!(worst <= 1.0)) {
        fprintf(stderr, "GEMM error %.3g of the 1e-5 sum|ab| bound\n", worst);
        return 6;
    }
    hipFree(sx); hipFree(sw); hipFree(dy);
    hipFree(dx.codes); hipFree(dx.scales); hipFree(dx.amax); hipFree(dx.tscale);
    hipFree(dw.codes); hipFree(dw.scales); hipFree(dw.amax); hipFree(dw.tscale);
    printf("abi consumer ok (GEMM worst error %.3g of the bound)\n", worst);
    return 0;
}
