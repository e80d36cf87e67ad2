/*
 * A plain C consumer of libfp4 (include/fp4.h): the library used through its
 * C ABI alone, with the HIP runtime for device memory, checked against the C
 * oracle (test infrastructure). Quantizes X (64 x 256) and W (48 x 256) to
 * NVFP4 with round-to-nearest, multiplies them (Y = X W^T, FP32 out), and
 * compares the codes, scale bytes and tensor scales bit for bit and Y within
 * 1e-5 * sum |a_k b_k| per element. Then the GEMM with raw operands, which
 * the library quantizes into the caller's workspace: for both formats, both
 * roundings, with and without the rotation, and each operand stored K-major
 * (layout N) or transposed (layout T), the product and the workspace's codes
 * and scale bytes must equal those of fp4_quantize followed by a GEMM of the
 * quantized operands, bit for bit. Last, X as two 32-row shards (the
 * transposed quantization with stochastic rounding, the shards' amaxes
 * reduced by max on the host): each shard's codes and scale bytes must be its
 * columns of the oracle's quantization of the whole X. Exit status 0 and
 * "abi consumer ok" on success.
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

/* One raw-operand case: the stored matrix of an operand (rows x K for
 * layout N, K x rows for layout T) on the device. */
typedef struct {
    float* dev;
    int rows, layout;
} raw_src;

static int upload_raw(const float* logical, int rows, int layout, raw_src* r)
{
    float* h = malloc(sizeof(float) * rows * K);
    for (int i = 0; i < rows; ++i)
        for (int k = 0; k < K; ++k) {
            if (layout == FP4_LAYOUT_N) h[i * K + k] = logical[i * K + k];
            else h[k * rows + i] = logical[i * K + k];
        }
    CHECK_HIP(hipMalloc((void**)&r->dev, sizeof(float) * rows * K));
    CHECK_HIP(hipMemcpy(r->dev, h, sizeof(float) * rows * K, hipMemcpyHostToDevice));
    free(h);
    r->rows = rows;
    r->layout = layout;
    return 0;
}

static void fill_raw(fp4_operand* o, const raw_src* r, int fmt, int rnd, uint64_t seed, int had,
                     uint32_t signs)
{
    memset(o, 0, sizeof(*o));
    o->kind = FP4_OPERAND_RAW;
    o->dtype = FP4_DTYPE_F32;
    o->data = r->dev;
    o->rows = r->rows;
    o->k = K;
    o->ld = r->layout == FP4_LAYOUT_N ? K : r->rows;
    o->layout = r->layout;
    o->fmt = fmt;
    o->rnd = rnd;
    o->seed = seed;
    o->index_offset = rnd == FP4_SR ? 64 : 0;
    o->had_on = had;
    o->had_signs = signs;
}

/* fp4_quantize of a raw operand into its own buffers, as the reference path. */
static int quantize_raw(const fp4_operand* o, fp4_tensor* t)
{
    int B = o->fmt == FP4_NVFP4 ? 16 : 32;
    memset(t, 0, sizeof(*t));
    CHECK_HIP(hipMalloc((void**)&t->codes, (size_t)o->rows * K / 2));
    CHECK_HIP(hipMalloc((void**)&t->scales, (size_t)o->rows * K / B));
    if (o->fmt == FP4_NVFP4) {
        CHECK_HIP(hipMalloc((void**)&t->amax, 4));
        CHECK_HIP(hipMalloc((void**)&t->tscale, 4));
    }
    t->fmt = o->fmt;
    t->had_on = o->had_on;
    t->had_signs = o->had_signs;
    int64_t R = o->layout == FP4_LAYOUT_N ? o->rows : K;
    int64_t C = o->layout == FP4_LAYOUT_N ? K : o->rows;
    CHECK_FP4(fp4_quantize(o->data, FP4_DTYPE_F32, R, C, o->ld,
                           o->layout == FP4_LAYOUT_N ? FP4_AXIS_COLS : FP4_AXIS_ROWS, (fp4_rounding)o->rnd,
                           o->seed, o->index_offset, 0, t, NULL));
    return 0;
}

static void free_q(fp4_tensor* t)
{
    hipFree(t->codes); hipFree(t->scales);
    if (t->amax) hipFree(t->amax);
    if (t->tscale) hipFree(t->tscale);
}

static int same_device_bytes(const void* a, const void* b, size_t n)
{
    uint8_t* ha = malloc(n);
    uint8_t* hb = malloc(n);
    int same = hipMemcpy(ha, a, n, hipMemcpyDeviceToHost) == hipSuccess &&
               hipMemcpy(hb, b, n, hipMemcpyDeviceToHost) == hipSuccess && memcmp(ha, hb, n) == 0;
    free(ha); free(hb);
    return same;
}

static int raw_operand_cases(const float* x, const float* w)
{
    int cases = 0;
    float* y_raw;
    float* y_ref;
    CHECK_HIP(hipMalloc((void**)&y_raw, sizeof(float) * M * N));
    CHECK_HIP(hipMalloc((void**)&y_ref, sizeof(float) * M * N));
    for (int la = 0; la < 2; ++la)
        for (int lb = 0; lb < 2; ++lb) {
            raw_src ra, rb;
            if (upload_raw(x, M, la, &ra) || upload_raw(w, N, lb, &rb)) return 10;
            for (int fmt = 0; fmt < 2; ++fmt)
                for (int rnd = 0; rnd < 2; ++rnd)
                    for (int had = 0; had < 2; ++had) {
                        uint32_t signs = fp4_hadamard_signs(5);
                        fp4_operand a, b;
                        fill_raw(&a, &ra, fmt, rnd, 11, had, signs);
                        fill_raw(&b, &rb, fmt, rnd, 12, had, signs);
                        size_t need = fp4_gemm_workspace_bytes(&a, &b);
                        if (need == 0) {
                            fprintf(stderr, "raw operands reported no workspace\n");
                            return 11;
                        }
                        uint8_t* ws;
                        CHECK_HIP(hipMalloc((void**)&ws, need));
                        if (fp4_gemm(&a, &b, FP4_DTYPE_F32, y_raw, N, ws, need - 1, NULL) != FP4_ERR_WORKSPACE) {
                            fprintf(stderr, "a workspace one byte short was accepted\n");
                            return 12;
                        }
                        CHECK_FP4(fp4_gemm(&a, &b, FP4_DTYPE_F32, y_raw, N, ws, need, NULL));
                        fp4_tensor qa, qb;
                        if (quantize_raw(&a, &qa) || quantize_raw(&b, &qb)) return 13;
                        fp4_operand oa, ob;
                        memset(&oa, 0, sizeof(oa));
                        memset(&ob, 0, sizeof(ob));
                        oa.kind = ob.kind = FP4_OPERAND_QUANTIZED;
                        oa.q = &qa;
                        ob.q = &qb;
                        CHECK_FP4(fp4_gemm(&oa, &ob, FP4_DTYPE_F32, y_ref, N, NULL, 0, NULL));
                        CHECK_HIP(hipDeviceSynchronize());
                        /* workspace layout: A codes, A scales, (NVFP4: A amax, tscale), then B's */
                        int B = fmt == FP4_NVFP4 ? 16 : 32;
                        size_t up = 256;
                        size_t ca = ((size_t)M * K / 2 + up - 1) / up * up;
                        size_t sa = ((size_t)M * K / B + up - 1) / up * up;
                        size_t a_bytes = ca + sa + (fmt == FP4_NVFP4 ? up : 0);
                        size_t cb = ((size_t)N * K / 2 + up - 1) / up * up;
                        size_t sb = ((size_t)N * K / B + up - 1) / up * up;
                        int ok = same_device_bytes(y_raw, y_ref, sizeof(float) * M * N) &&
                                 same_device_bytes(ws, qa.codes, (size_t)M * K / 2) &&
                                 same_device_bytes(ws + ca, qa.scales, (size_t)M * K / B) &&
                                 same_device_bytes(ws + a_bytes, qb.codes, (size_t)N * K / 2) &&
                                 same_device_bytes(ws + a_bytes + cb, qb.scales, (size_t)N * K / B);
                        if (ok && fmt == FP4_NVFP4)
                            ok = same_device_bytes(ws + ca + sa + 4, qa.tscale, 4) &&
                                 same_device_bytes(ws + a_bytes + cb + sb + 4, qb.tscale, 4);
                        if (!ok) {
                            fprintf(stderr, "raw-operand GEMM differs from quantize-then-GEMM: layouts %d %d, "
                                            "fmt %d, rnd %d, rotation %d\n", la, lb, fmt, rnd, had);
                            return 14;
                        }
                        free_q(&qa);
                        free_q(&qb);
                        hipFree(ws);
                        ++cases;
                    }
            hipFree(ra.dev);
            hipFree(rb.dev);
        }
    hipFree(y_raw);
    hipFree(y_ref);
    return cases == 32 ? 0 : 15;
}

/* X (M x K) in two row shards, quantized along the rows (out: K x rows) with
 * SR and the whole tensor's indices and amax. */
static int shard_case(const float* x)
{
    enum { SH = M / 2 };
    float* dx;
    float* damax;
    CHECK_HIP(hipMalloc((void**)&dx, sizeof(float) * M * K));
    CHECK_HIP(hipMemcpy(dx, x, sizeof(float) * M * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMalloc((void**)&damax, 2 * sizeof(float)));
    for (int h = 0; h < 2; ++h)
        CHECK_FP4(fp4_tensor_amax(dx + h * SH * K, FP4_DTYPE_F32, SH, K, K, damax + h, NULL));
    float am[2];
    CHECK_HIP(hipMemcpy(am, damax, sizeof(am), hipMemcpyDeviceToHost));
    const float amax = am[0] > am[1] ? am[0] : am[1]; /* the all-reduce(max) */

    static uint8_t wc[K * M / 2], ws[K * M / 16];
    float wam, wsg;
    if (o_quantize(x, 0, M, K, K, O_AXIS_ROWS, O_FMT_NVFP4, O_SR, 11, 0, 0, 0, 0, 0.0f, wc, ws, &wam, &wsg) != 0)
        return 20;
    int bad = 0;
    for (int h = 0; h < 2; ++h) {
        dev_q d;
        CHECK_HIP(hipMalloc((void**)&d.codes, fp4_codes_bytes(K, SH)));
        CHECK_HIP(hipMalloc((void**)&d.scales, fp4_scales_bytes(K, SH, FP4_NVFP4)));
        CHECK_HIP(hipMalloc((void**)&d.amax, 4));
        CHECK_HIP(hipMalloc((void**)&d.tscale, 4));
        CHECK_HIP(hipMemcpy(d.amax, &amax, 4, hipMemcpyHostToDevice));
        fp4_tensor t;
        memset(&t, 0, sizeof(t));
        t.codes = d.codes;
        t.scales = d.scales;
        t.amax = d.amax;
        t.tscale = d.tscale;
        t.fmt = FP4_NVFP4;
        CHECK_FP4(fp4_quantize_shard(dx + h * SH * K, FP4_DTYPE_F32, SH, K, K, h * SH, M, FP4_AXIS_ROWS, FP4_SR,
                                     11, 0, 1, &t, NULL, NULL));
        static uint8_t gc[K * SH / 2], gs[K * SH / 16];
        float gsg;
        CHECK_HIP(hipMemcpy(gc, d.codes, sizeof(gc), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(gs, d.scales, sizeof(gs), hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(&gsg, d.tscale, 4, hipMemcpyDeviceToHost));
        for (int r = 0; r < K; ++r) {
            bad |= memcmp(gc + r * (SH / 2), wc + r * (M / 2) + h * (SH / 2), SH / 2) != 0;
            bad |= memcmp(gs + r * (SH / 16), ws + r * (M / 16) + h * (SH / 16), SH / 16) != 0;
        }
        bad |= gsg != wsg;
        hipFree(d.codes); hipFree(d.scales); hipFree(d.amax); hipFree(d.tscale);
    }
    hipFree(dx);
    hipFree(damax);
    if (bad) {
        fprintf(stderr, "a shard differs from its slice of the whole tensor's quantization\n");
        return 21;
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
    fp4_operand ox, ow;
    memset(&ox, 0, sizeof(ox));
    memset(&ow, 0, sizeof(ow));
    ox.kind = ow.kind = FP4_OPERAND_QUANTIZED;
    ox.q = &tx;
    ow.q = &tw;
    if (fp4_gemm_workspace_bytes(&ox, &ow) != 0) {
        fprintf(stderr, "quantized operands need no workspace\n");
        return 7;
    }
    CHECK_FP4(fp4_gemm(&ox, &ow, FP4_DTYPE_F32, dy, N, NULL, 0, NULL));
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
    if ((rc = raw_operand_cases(x, w))) return rc;
    if ((rc = shard_case(x))) return rc;
    hipFree(sx); hipFree(sw); hipFree(dy);
    hipFree(dx.codes); hipFree(dx.scales); hipFree(dx.amax); hipFree(dx.tscale);
    hipFree(dw.codes); hipFree(dw.scales); hipFree(dw.amax); hipFree(dw.tscale);
    printf("abi consumer ok (GEMM worst error %.3g of the bound; 32 raw-operand GEMMs equal to "
           "quantize-then-GEMM; two SR shards equal to their slices)\n", worst);
    return 0;
}
