/*
 * fp4_oracle.c -- plain CPU oracle for block-scaled FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark; never by the GPU product path, with
 * which it shares no code.
 *
 * Written for readability, not speed: every rounding decision is taken by
 * enumerating the candidate values of the target format and picking the
 * nearest one, so the reader can check each step against the definitions.
 * Build: gcc -O2 -ffp-contract=off -fopenmp (no fast-math), so every float
 * operation below is one IEEE-754 binary32 operation rounded to nearest even.
 *
 * Sources (the web pages this method is described on):
 *  - Robots Atlas, "FP4", section Components (E2M1 format; NVFP4; MXFP4;
 *    block scaling) and section How it works (two-level scaling, Hadamard
 *    rotation, stochastic rounding of gradients).
 *  - "FP4 All the Way: Fully Quantized Training of LLMs", Key points and
 *    Summary (NVFP4 choice; round-to-nearest forward, stochastic rounding in
 *    backward and update passes).
 *  - "Quartet: Native FP4 Training Can Be Optimal for Large Language
 *    Models", Approach (MXFP4 with block-wise Hadamard rotations).
 * Readings of what the pages leave open (scale rules, tie rules, the random
 * stream and its indexing, the rotation's normalisation) are stated at each
 * function.
 */
#include "fp4_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* E2M1 (Robots Atlas "FP4", Components / E2M1 format).                      */
/* Bit layout S | E1 E0 | M, exponent bias 1, E=0 encodes the subnormal 0.5. */
/* ------------------------------------------------------------------------ */
double o_e2m1_value(unsigned code4)
{
    unsigned s = (code4 >> 3) & 1u;
    unsigned e = (code4 >> 1) & 3u;
    unsigned m = code4 & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : (1.0 + 0.5 * (double)m) * ldexp(1.0, (int)e - 1);
    return s ? -mag : mag;
}

/* Round-to-nearest onto the E2M1 magnitudes; a tie goes to the code whose
 * mantissa bit is 0 ("even"), as IEEE round-to-nearest-even does. */
unsigned o_e2m1_rtn_mag(float a)
{
    unsigned best = 0;
    double bestd = fabs((double)a - o_e2m1_value(0));
    for (unsigned c = 1; c < 8; ++c) {
        double d = fabs((double)a - o_e2m1_value(c));
        if (d < bestd || (d == bestd && (c & 1u) == 0)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* Stochastic rounding onto the E2M1 magnitudes. A value on the grid is kept.
 * Otherwise, with lo < a < hi its grid neighbours and p = (a-lo)/(hi-lo),
 * the result is hi when the 16-bit draw and p's first 16 fraction bits carry
 * out of a 16-bit add, h16 + floor(p * 2^16) >= 2^16, else lo; so
 * P(hi) = floor(p * 2^16) / 2^16, at most 2^-16 below p, and the expected
 * result equals a up to 2^-16 of a grid step. */
unsigned o_e2m1_sr_mag(float a, uint32_t h16)
{
    unsigned lo = 0;
    for (unsigned c = 0; c < 8; ++c) {
        double g = o_e2m1_value(c);
        if (g == (double)a) return c;
        if (g < (double)a) lo = c;
    }
    if (lo == 7) return 7; /* a > 6 does not occur: callers clamp to 6 */
    unsigned hi = lo + 1;
    double glo = o_e2m1_value(lo), ghi = o_e2m1_value(hi);
    double p = ((double)a - glo) / (ghi - glo); /* exact: a power-of-two step */
    double pf = floor(p * 65536.0);
    return ((double)(h16 & 0xFFFFu) + pf >= 65536.0) ? hi : lo;
}

/* ------------------------------------------------------------------------ */
/* E4M3 block scale (Robots Atlas "FP4", Components / NVFP4; Hyperparameters */
/* scale factor format). OCP "fn" variant: bias 7, no infinities, max 448,   */
/* 0x7F / 0xFF are NaN, subnormals m * 2^-9.                                 */
/* ------------------------------------------------------------------------ */
double o_e4m3_value(unsigned byte)
{
    unsigned s = (byte >> 7) & 1u;
    unsigned e = (byte >> 3) & 15u;
    unsigned m = byte & 7u;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = (double)m * ldexp(1.0, -9);
    else
        mag = (1.0 + (double)m / 8.0) * ldexp(1.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Nearest finite non-negative E4M3 value to t >= 0; ties to the even
 * mantissa (even byte); anything above the largest finite value saturates to
 * 448 (0x7E). The block scale is always rounded to nearest, never
 * stochastically. */
unsigned o_e4m3_encode(float t)
{
    if (!(t >= 0.0f)) return 0; /* callers never pass negative or NaN */
    if ((double)t > 448.0) return 0x7E;
    unsigned best = 0;
    double bestd = fabs((double)t);
    for (unsigned b = 1; b <= 0x7E; ++b) {
        double d = fabs((double)t - o_e4m3_value(b));
        if (d < bestd || (d == bestd && (b & 1u) == 0)) {
            best = b;
            bestd = d;
        }
    }
    return best;
}

/* ------------------------------------------------------------------------ */
/* E8M0 block scale (Robots Atlas "FP4", Components / MXFP4): a bare power  */
/* of two 2^(byte-127). Reading of "brings the block into FP4-representable  */
/* range": the smallest power of two that maps the block's largest magnitude */
/* to at most 6, i.e. amax_b/6 rounded up to a power of two.                 */
/* ------------------------------------------------------------------------ */
int o_e8m0_exponent(float amax_b)
{
    for (int e = -127; e <= 127; ++e)
        if (6.0 * ldexp(1.0, e) >= (double)amax_b) return e;
    return 127;
}

double o_e8m0_value(unsigned byte)
{
    if ((byte & 0xFFu) == 0xFFu) return NAN;
    return ldexp(1.0, (int)(byte & 0xFFu) - 127);
}

uint16_t o_f32_to_bf16_rne(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

float o_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 counter-based generator (Salmon, Moraes, Dror, Shaw,        */
/* "Parallel random numbers: as easy as 1, 2, 3", SC'11). One round maps    */
/* (c0,c1,c2,c3) with key (k0,k1) to                                        */
/*   (hi(M1*c2)^c1^k0, lo(M1*c2), hi(M0*c0)^c3^k1, lo(M0*c0));               */
/* the key advances by the Weyl constants between rounds.                    */
/* ------------------------------------------------------------------------ */
void o_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)M0 * (uint64_t)c0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += W0;
        k1 += W1;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The stochastic-rounding stream: element `index` (row-major position in the
 * quantized orientation plus the caller's offset) uses 16 bits of Philox
 * output. One Philox call (counter = index / 8, key = seed) serves 8
 * consecutive elements; element index uses word (index/2) % 4, low half for
 * even index, high half for odd. */
uint32_t o_sr_draw16(uint64_t seed, uint64_t index)
{
    uint64_t call = index >> 3;
    uint32_t ctr[4] = {(uint32_t)call, (uint32_t)(call >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    o_philox4x32_10(ctr, key, out);
    uint32_t w = out[(index >> 1) & 3u];
    return (index & 1u) ? (w >> 16) : (w & 0xFFFFu);
}

/* The rotation's sign mask: word 0 of Philox at counter (0,0,0,1), a counter
 * the element stream never uses. */
uint32_t o_hadamard_signs(uint64_t seed)
{
    uint32_t ctr[4] = {0u, 0u, 0u, 1u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    o_philox4x32_10(ctr, key, out);
    return out[0];
}

/* ------------------------------------------------------------------------ */
/* Block-wise random-sign Hadamard rotation (Quartet, Approach; Robots Atlas */
/* "FP4", How it works). y = c * H32 * (D x), D = diag(+-1) from the mask    */
/* bits (bit j set: negate x_j), H32 the Sylvester-ordered Hadamard matrix   */
/* H[i][j] = (-1)^popcount(i & j), c = 2^-2.5 rounded to FP32 so that c*H32  */
/* is orthonormal up to that rounding. The butterfly stages run h = 1, 2, 4, */
/* 8, 16, each sum and difference one FP32 operation.                        */
/* ------------------------------------------------------------------------ */
void o_fwht32(float x[32], uint32_t signs)
{
    const float c = (float)ldexp(sqrt(2.0), -3); /* 2^-2.5 */
    for (int j = 0; j < 32; ++j)
        if ((signs >> j) & 1u) x[j] = -x[j];
    for (int h = 1; h < 32; h <<= 1) {
        for (int i = 0; i < 32; ++i) {
            if ((i & h) == 0) {
                float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
        }
    }
    for (int j = 0; j < 32; ++j) x[j] = x[j] * c;
}

/* The random Hadamard transform for NVFP4 (Robots Atlas "FP4", How it       */
/* works: random Hadamard transforms are one of the stabilizers of FP4       */
/* training, not tied to one format). Reading: like the MXFP4 rotation, it   */
/* spans exactly one scale block, so here 16 elements:                       */
/* y = (1/4) * H16 * (D x), D from bits 0..15 of the mask, butterfly stages  */
/* h = 1, 2, 4, 8 in FP32. The normalisation 16^-1/2 = 1/4 is exact.         */
void o_fwht16(float x[16], uint32_t signs)
{
    for (int j = 0; j < 16; ++j)
        if ((signs >> j) & 1u) x[j] = -x[j];
    for (int h = 1; h < 16; h <<= 1) {
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                float a = x[i], b = x[i + h];
                x[i] = a + b;
                x[i + h] = a - b;
            }
        }
    }
    for (int j = 0; j < 16; ++j) x[j] = x[j] * 0.25f;
}

/* The inverse rotation. c*H*D is orthonormal (up to the rounding of c), so */
/* its inverse is its transpose D*H*c (H is symmetric): the same butterfly   */
/* stages on y, the product with c, then the signs. Used to read a rotated   */
/* quantization back in the tensor's own domain.                             */
void o_unfwht32(float y[32], uint32_t signs)
{
    const float c = (float)ldexp(sqrt(2.0), -3); /* 2^-2.5 */
    for (int h = 1; h < 32; h <<= 1) {
        for (int i = 0; i < 32; ++i) {
            if ((i & h) == 0) {
                float a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
        }
    }
    for (int j = 0; j < 32; ++j) y[j] = y[j] * c;
    for (int j = 0; j < 32; ++j)
        if ((signs >> j) & 1u) y[j] = -y[j];
}

void o_unfwht16(float y[16], uint32_t signs)
{
    for (int h = 1; h < 16; h <<= 1) {
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                float a = y[i], b = y[i + h];
                y[i] = a + b;
                y[i + h] = a - b;
            }
        }
    }
    for (int j = 0; j < 16; ++j) y[j] = y[j] * 0.25f;
    for (int j = 0; j < 16; ++j)
        if ((signs >> j) & 1u) y[j] = -y[j];
}

/* ------------------------------------------------------------------------ */
/* Tensors.                                                                  */
/* ------------------------------------------------------------------------ */
static float load_elem(const void* src, int src_bf16, int64_t i)
{
    if (src_bf16) return o_bf16_to_f32(((const uint16_t*)src)[i]);
    return ((const float*)src)[i];
}

float o_tensor_amax(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld)
{
    float amax = 0.0f;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            float a = fabsf(load_elem(src, src_bf16, r * ld + c));
            if (a > amax) amax = a;
        }
    return amax;
}

/* NVFP4 two-level scaling (Robots Atlas "FP4", How it works / NVFP4): the
 * FP32 tensor scale maps the tensor amax onto the product of the largest
 * E2M1 magnitude and the largest E4M3 value, s_g = amax / (6 * 448); an
 * all-zero tensor takes s_g = 1. */
/* NVFP4 tensor scale (Robots Atlas "FP4", How it works: the per-tensor FP32
 * scale of two-level scaling): amax / (6 * 448). Degenerate tensors: an amax
 * of 0, or below 2^-100, takes s_g = 1. For such a tensor every block scale
 * then encodes to E4M3 0 and every code is a signed zero; without the floor
 * s_g could be 0 or subnormal and the block scale's reciprocal 0/0 or
 * infinite. Above it, s_g >= 2^-112 and every nonzero decoded block scale
 * times s_g stays a normal FP32 number. */
static float nv_tensor_scale(float amax)
{
    if (amax < 0x1p-100f) return 1.0f;
    return amax / 2688.0f;
}

static double scale_value(const uint8_t* scales, int64_t i, int fmt);

/* Quantization noise of a quantized tensor (FP4 All the Way, Summary: the
 * gradient norm set against the quantization noise). x holds the values that
 * were quantized (after the rotation, when it is on), rows x cols in the
 * quantized orientation. out[0] = sum x^2, out[1] = sum (xhat - x)^2 with xhat
 * the exact value the code and scales stand for (e2m1 * sdec * s_g, or
 * e2m1 * 2^e): every product is exact in FP64 (at most 31 significant bits),
 * the difference and the sums are FP64 roundings. Rows are summed in order. */
static void quant_noise(const float* x, const uint8_t* codes, const uint8_t* scales,
                        int64_t rows, int64_t cols, int fmt, float sg, double out[2])
{
    const int B = (fmt == O_FMT_NVFP4) ? 16 : 32;
    double* part = (double*)calloc((size_t)(2 * rows), sizeof(double));
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double g = 0.0, e = 0.0;
        for (int64_t c = 0; c < cols; ++c) {
            int64_t pos = r * cols + c;
            unsigned code = (codes[pos >> 1] >> ((pos & 1) * 4)) & 15u;
            double xhat = o_e2m1_value(code) * scale_value(scales, r * (cols / B) + c / B, fmt);
            if (fmt == O_FMT_NVFP4) xhat *= (double)sg;
            double xv = (double)x[pos];
            double d = xhat - xv;
            g += xv * xv;
            e += d * d;
        }
        part[2 * r] = g;
        part[2 * r + 1] = e;
    }
    out[0] = 0.0;
    out[1] = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        out[0] += part[2 * r];
        out[1] += part[2 * r + 1];
    }
    free(part);
}

/* Block scale "amax/6" of a block with amax amax_b: returns the scale byte and
 * sets the element multiplier r.
 * NVFP4: E4M3 scale relative to the tensor scale, rounded to nearest; the
 * element multiplier is the reciprocal of the full decoded scale, rounded once
 * (zero scale -> zero). MXFP4: the power of two of o_e8m0_exponent. */
static unsigned block_scale(float amax_b, int fmt, float sg, float* rcp)
{
    if (fmt == O_FMT_NVFP4) {
        float q = amax_b / 6.0f;
        q = q / sg;
        unsigned sbyte = o_e4m3_encode(q);
        float sdec = (float)o_e4m3_value(sbyte);
        float d = sdec * sg;
        *rcp = (d == 0.0f) ? 0.0f : 1.0f / d;
        return sbyte;
    }
    int e = o_e8m0_exponent(amax_b);
    *rcp = (float)ldexp(1.0, -e);
    return (unsigned)(e + 127);
}

/* The E2M1 code of x with element multiplier rcp: RTN, or SR with the 16-bit
 * draw of element index idx under seed. */
static unsigned encode_elem(float x, float rcp, int rnd, uint64_t seed, uint64_t idx)
{
    float v = x * rcp;
    float a = fabsf(v);
    if (a > 6.0f) a = 6.0f;
    unsigned mag = (rnd == O_SR) ? o_e2m1_sr_mag(a, o_sr_draw16(seed, idx)) : o_e2m1_rtn_mag(a);
    return (signbit(v) ? 8u : 0u) | mag;
}

/* Code nibble at packed position pos (element 2t in the low nibble of byte t). */
static void put_code(uint8_t* codes, int64_t pos, unsigned code)
{
    uint8_t* byte = &codes[pos >> 1];
    if ((pos & 1) == 0)
        *byte = (uint8_t)((*byte & 0xF0u) | code);
    else
        *byte = (uint8_t)((*byte & 0x0Fu) | (code << 4));
}

static int quantize_impl(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld,
                         int axis, int fmt, int rnd, uint64_t seed, uint64_t index_offset,
                         int had_on, uint32_t had_signs, int amax_given, float amax_in,
                         uint8_t* codes, uint8_t* scales, float* amax_out, float* sg_out,
                         double* noise)
{
    if (!src || !codes || !scales || R <= 0 || C <= 0 || ld < C) return -1;
    if (fmt != O_FMT_NVFP4 && fmt != O_FMT_MXFP4) return -1;
    const int B = (fmt == O_FMT_NVFP4) ? 16 : 32;
    const int64_t rows_q = (axis == O_AXIS_ROWS) ? C : R;
    const int64_t cols_q = (axis == O_AXIS_ROWS) ? R : C;
    if (cols_q % B != 0) return -1;

    /* Load into FP32 in the quantized orientation (a transpose is an exact
     * copy). Non-finite inputs are outside the contract. */
    float* t = (float*)malloc((size_t)(rows_q * cols_q) * sizeof(float));
    if (!t) return -3;
    int bad = 0;
#pragma omp parallel for reduction(| : bad)
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c) {
            float v = load_elem(src, src_bf16, r * ld + c);
            if (!isfinite(v)) bad = 1;
            if (axis == O_AXIS_ROWS)
                t[c * cols_q + r] = v;
            else
                t[r * cols_q + c] = v;
        }
    if (bad) {
        free(t);
        return -2;
    }

    /* The rotation (when on) acts on every block along the blocked axis before
     * anything else: the tensor amax of NVFP4 is that of the rotated tensor,
     * the values the scales have to cover. */
    const int64_t nblk = cols_q / B;
    if (had_on) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows_q; ++r)
            for (int64_t b = 0; b < nblk; ++b) {
                float* blk = t + r * cols_q + b * B;
                if (B == 16)
                    o_fwht16(blk, had_signs);
                else
                    o_fwht32(blk, had_signs);
            }
    }

    float sg = 1.0f;
    if (fmt == O_FMT_NVFP4) {
        float amax = amax_given ? amax_in : o_tensor_amax(t, 0, rows_q, cols_q, cols_q);
        sg = nv_tensor_scale(amax);
        if (amax_out) *amax_out = amax;
        if (sg_out) *sg_out = sg;
    }

#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows_q; ++r) {
        for (int64_t b = 0; b < nblk; ++b) {
            float x[32];
            for (int j = 0; j < B; ++j) x[j] = t[r * cols_q + b * B + j];

            float amax_b = 0.0f;
            for (int j = 0; j < B; ++j)
                if (fabsf(x[j]) > amax_b) amax_b = fabsf(x[j]);

            float rcp;
            unsigned sbyte = block_scale(amax_b, fmt, sg, &rcp);
            scales[r * nblk + b] = (uint8_t)sbyte;

            for (int j = 0; j < B; ++j) {
                uint64_t idx = index_offset + (uint64_t)(r * cols_q + b * B + j);
                put_code(codes, r * cols_q + b * B + j, encode_elem(x[j], rcp, rnd, seed, idx));
            }
        }
    }
    if (noise) quant_noise(t, codes, scales, rows_q, cols_q, fmt, sg, noise);
    free(t);
    return 0;
}

int o_quantize(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld,
               int axis, int fmt, int rnd, uint64_t seed, uint64_t index_offset,
               int had_on, uint32_t had_signs, int amax_given, float amax_in,
               uint8_t* codes, uint8_t* scales, float* amax_out, float* sg_out)
{
    return quantize_impl(src, src_bf16, R, C, ld, axis, fmt, rnd, seed, index_offset, had_on,
                         had_signs, amax_given, amax_in, codes, scales, amax_out, sg_out, NULL);
}

int o_quantize_noise(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld,
                     int axis, int fmt, int rnd, uint64_t seed, uint64_t index_offset,
                     int had_on, uint32_t had_signs, int amax_given, float amax_in,
                     uint8_t* codes, uint8_t* scales, float* amax_out, float* sg_out,
                     double noise[2])
{
    if (!noise) return -1;
    return quantize_impl(src, src_bf16, R, C, ld, axis, fmt, rnd, seed, index_offset, had_on,
                         had_signs, amax_given, amax_in, codes, scales, amax_out, sg_out, noise);
}

/* Two-dimensional block quantization (Robots Atlas "FP4", How it works: two-
 * dimensional quantization among the stabilizers). Reading: square B x B
 * blocks (B = 16 NVFP4, 32 MXFP4), one scale per block from the block's amax
 * by the same rule as a 1-D block, so that the matrix and its transpose are
 * the same quantization. Element index for SR: row-major position in the
 * R x C source + index_offset, for both outputs, so out_t is exactly the
 * transpose of out. Outputs in the layouts of o_quantize:
 *   codes   [R][C/2], scales   [R][C/B]   (the block's byte on each of its rows)
 *   codes_t [C][R/2], scales_t [C][R/B]   (the transpose) */
int o_quantize_2d(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld, int fmt, int rnd,
                  uint64_t seed, uint64_t index_offset, int amax_given, float amax_in,
                  uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                  float* amax_out, float* sg_out)
{
    if (!src || !codes || !scales || !codes_t || !scales_t || R <= 0 || C <= 0 || ld < C) return -1;
    if (fmt != O_FMT_NVFP4 && fmt != O_FMT_MXFP4) return -1;
    const int B = (fmt == O_FMT_NVFP4) ? 16 : 32;
    if (R % B != 0 || C % B != 0) return -1;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; ++c)
            if (!isfinite(load_elem(src, src_bf16, r * ld + c))) return -2;

    float sg = 1.0f;
    if (fmt == O_FMT_NVFP4) {
        float amax = amax_given ? amax_in : o_tensor_amax(src, src_bf16, R, C, ld);
        sg = nv_tensor_scale(amax);
        if (amax_out) *amax_out = amax;
        if (sg_out) *sg_out = sg;
    }
#pragma omp parallel for schedule(static)
    for (int64_t br = 0; br < R / B; ++br) {
        for (int64_t bc = 0; bc < C / B; ++bc) {
            float amax_b = 0.0f;
            for (int i = 0; i < B; ++i)
                for (int j = 0; j < B; ++j) {
                    float a = fabsf(load_elem(src, src_bf16, (br * B + i) * ld + bc * B + j));
                    if (a > amax_b) amax_b = a;
                }
            float rcp;
            unsigned sbyte = block_scale(amax_b, fmt, sg, &rcp);
            for (int i = 0; i < B; ++i) {
                int64_t r = br * B + i, c0 = bc * B;
                scales[r * (C / B) + bc] = (uint8_t)sbyte;
                scales_t[(c0 + i) * (R / B) + br] = (uint8_t)sbyte;
                for (int j = 0; j < B; ++j) {
                    int64_t c = c0 + j;
                    unsigned code = encode_elem(load_elem(src, src_bf16, r * ld + c), rcp, rnd, seed,
                                                index_offset + (uint64_t)(r * C + c));
                    put_code(codes, r * C + c, code);
                    put_code(codes_t, c * R + r, code);
                }
            }
        }
    }
    return 0;
}

static double scale_value(const uint8_t* scales, int64_t i, int fmt)
{
    return (fmt == O_FMT_NVFP4) ? o_e4m3_value(scales[i]) : o_e8m0_value(scales[i]);
}

int o_dequantize_f32(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int fmt, float sg, float* out)
{
    const int B = (fmt == O_FMT_NVFP4) ? 16 : 32;
    if (cols % B != 0) return -1;
#pragma omp parallel for
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t pos = r * cols + c;
            unsigned code = (codes[pos >> 1] >> ((pos & 1) * 4)) & 15u;
            double q = o_e2m1_value(code);
            double s = scale_value(scales, r * (cols / B) + c / B, fmt);
            if (fmt == O_FMT_NVFP4) {
                float qs = (float)(q * s); /* exact: at most 6 significant bits */
                out[pos] = qs * sg;
            } else {
                out[pos] = (float)(q * s); /* exact power-of-two scaling */
            }
        }
    return 0;
}

int o_dequantize_f64(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int fmt, float sg, double* out)
{
    const int B = (fmt == O_FMT_NVFP4) ? 16 : 32;
    if (cols % B != 0) return -1;
#pragma omp parallel for
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t pos = r * cols + c;
            unsigned code = (codes[pos >> 1] >> ((pos & 1) * 4)) & 15u;
            double q = o_e2m1_value(code);
            double s = scale_value(scales, r * (cols / B) + c / B, fmt);
            out[pos] = (fmt == O_FMT_NVFP4) ? q * s * (double)sg : q * s;
        }
    return 0;
}

/* Dequantize, then undo the block rotation the quantization applied        */
/* (had_on): each block of B values in the quantized orientation goes        */
/* through o_unfwht (B = 16 for NVFP4, 32 for MXFP4), so the result          */
/* approximates the source tensor itself rather than its rotation.           */
int o_dequantize_unrotated_f32(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                               int fmt, float sg, uint32_t had_signs, float* out)
{
    const int B = (fmt == O_FMT_NVFP4) ? 16 : 32;
    int rc = o_dequantize_f32(codes, scales, rows, cols, fmt, sg, out);
    if (rc != 0) return rc;
#pragma omp parallel for
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; c += B) {
            if (B == 16) o_unfwht16(out + r * cols + c, had_signs);
            else o_unfwht32(out + r * cols + c, had_signs);
        }
    return 0;
}

int o_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
