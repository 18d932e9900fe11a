/*
 * convrot_oracle.c -- plain CPU oracle (TEST INFRASTRUCTURE ONLY; see the
 * header for who may load it and for the sources it follows).
 *
 * Compiled with: gcc -O3 -ffp-contract=off -fno-fast-math -fopenmp
 * Every floating-point operation below is a single IEEE binary32 operation in
 * round-to-nearest-even; fmaf() appears only where the pinned definition uses
 * a fused multiply-add.  Loops are written in the order the definition states;
 * OpenMP only splits independent rows between threads.
 */
#include "convrot_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static float u32_as_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_as_u32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bf16_to_f32(uint16_t b) { return u32_as_f32((uint32_t)b << 16); }

static int is_pow2_le(int g, int max) { return g >= 1 && g <= max && (g & (g - 1)) == 0; }

/* ---------------------------------------------------------------------------
 * Rotation.  [KEY] stores W_rot = W H^T and rotates x_rot = x H online.  The
 * pages' two statements of the identity place H and H^T differently; with the
 * normalised Sylvester matrix H is symmetric and orthogonal, so both hold.
 * H is block-diagonal over contiguous groups of g input channels ([LOAD]: the
 * per-partition input size must be divisible by the group size).
 * ------------------------------------------------------------------------- */

/* Closed form: H_g[i][j] = (-1)^popcount(i & j) / sqrt(g). */
int orc_hadamard(int g, double *h)
{
    if (!is_pow2_le(g, 4096)) return -1;
    double c = 1.0 / sqrt((double)g);
    for (int i = 0; i < g; ++i)
        for (int j = 0; j < g; ++j)
            h[(int64_t)i * g + j] = (__builtin_popcount((unsigned)(i & j)) & 1) ? -c : c;
    return 0;
}

/* Normalisation constant of H_g as an FP32 value: fl(1/sqrt(g)). */
float orc_norm_const(int g) { return (float)(1.0 / sqrt((double)g)); }

/* Unnormalised fast Walsh-Hadamard transform of each group of g values:
 * u = v * (sqrt(g) H_g).  Pinned order: strides h = 1, 2, 4, ..., g/2 in
 * ascending order; at stride h every pair (i, i+h) with (i & h) == 0 becomes
 * (v_i + v_{i+h}, v_i - v_{i+h}).  The 1/sqrt(g) factor is not applied here:
 * it cancels out of the codes and enters only the scale (orc_quant_row). */
void orc_fwht_groups(float *v, int64_t n, int g)
{
    for (int64_t base = 0; base + g <= n; base += g) {
        float *b = v + base;
        for (int h = 1; h < g; h <<= 1)
            for (int i = 0; i < g; ++i)
                if ((i & h) == 0) {
                    float p = b[i], q = b[i + h];
                    b[i] = p + q;
                    b[i + h] = p - q;
                }
    }
}

/* ---------------------------------------------------------------------------
 * SwiGLU, [SWI]: the down projection's quantizer forms silu(gate) * up and
 * keeps it in FP32 (not rounded to BF16).  The pages do not say how silu is
 * evaluated; the pinned reading is silu(gamma) = gamma * 1/(1 + e^{-gamma})
 * with e^{-gamma} and the reciprocal computed by the two fixed procedures
 * below, so that a GPU can reproduce every bit.
 * ------------------------------------------------------------------------- */

/* e^{-gc} for gc in [-80, 80] by Cody-Waite reduction (W. J. Cody and
 * W. Waite, Software Manual for the Elementary Functions, 1980):
 *   t  = -gc
 *   kf = rint(fl(t * LOG2E))                          (nearest, ties to even)
 *   r  = fma(kf, -LN2_HI, t)   -- exact: LN2_HI has 16 significant bits
 *   r  = fma(kf, -LN2_LO, r)
 *   p  = 1 + r + r^2/2! + ... + r^7/7!   (Horner, one fmaf per degree)
 *   E  = p * 2^kf                         (exact: the result stays normal)
 * Constants: LOG2E = fl(log2 e); LN2_HI = round(ln2 * 2^16) / 2^16;
 * LN2_LO = fl(ln2 - LN2_HI); C_n = fl(1/n!).                                */
static const float LOG2E = 0x1.715476p+0f;
static const float LN2_HI = 0x1.62e4p-1f;
static const float LN2_LO = 0x1.7f7d1cp-20f;
static const float TAYLOR[8] = {
    0x1p+0f, 0x1p+0f, 0x1p-1f, 0x1.555556p-3f,
    0x1.555556p-5f, 0x1.111112p-7f, 0x1.6c16c2p-10f, 0x1.a01a02p-13f,
};

float orc_exp_neg(float gc)
{
    float t = -gc;
    float kf = rintf(t * LOG2E);
    float r = fmaf(kf, -LN2_HI, t);
    r = fmaf(kf, -LN2_LO, r);
    float p = TAYLOR[7];
    for (int n = 6; n >= 0; --n) p = fmaf(p, r, TAYLOR[n]);
    return ldexpf(p, (int)kf);
}

/* 1/d for d in [1, 2^116]: seed y0 = bits(RCP_MAGIC - bits(d)) (maximum
 * relative error 5.05e-2 over a binade; the constant minimises that error and
 * was found by exhaustive search), then three Newton-Raphson steps
 *   e = fma(-d, y, 1);  y = fma(y, e, y).                                   */
static const uint32_t RCP_MAGIC = 0x7ef311c2u;

float orc_rcp(float d)
{
    float y = u32_as_f32(RCP_MAGIC - f32_as_u32(d));
    for (int it = 0; it < 3; ++it) {
        float e = fmaf(-d, y, 1.0f);
        y = fmaf(y, e, y);
    }
    return y;
}

/* silu(gamma) = gl * rcp(1 + e^{-gc}) with gl = max(gamma, -80) and
 * gc = min(gl, 80).  The clamps keep every intermediate finite and normal.
 * The upper one changes nothing (1 + e^{-gc} rounds to 1 for gc >= 80, so
 * silu(gamma) = gamma there); the lower one sets silu(gamma) = silu(-80)
 * (about -1.4e-33) for every gamma below -80, where the true value is smaller
 * still in magnitude. */
float orc_silu(float gamma)
{
    float gl = gamma < -80.0f ? -80.0f : gamma;
    float gc = gl > 80.0f ? 80.0f : gl;
    float e = orc_exp_neg(gc);
    float d = 1.0f + e;
    return gl * orc_rcp(d);
}

void orc_exp_neg_v(const float *x, int64_t n, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_exp_neg(x[i]);
}

void orc_rcp_v(const float *x, int64_t n, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_rcp(x[i]);
}

void orc_silu_v(const uint16_t *gate_bf16, int64_t n, float *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) y[i] = orc_silu(bf16_to_f32(gate_bf16[i]));
}

/* ---------------------------------------------------------------------------
 * Quantization.  [KEY]: the activation is quantized per token to INT8 on the
 * same symmetric grid as the weight; [LOAD]: per-output-row weight scale
 * stored as F32 [out, 1].  Symmetric absmax quantization with scale
 * amax/127 and round-half-even; codes lie in [-127, 127].
 *
 * Pinned FP32 reading, with u the unnormalised rotated row and c = fl(1/sqrt g):
 *   A = max_k |u_k|                          (exact)
 *   s = fl(fl(A * c) / 127)                  -- fl(A * c) equals the absmax of
 *                                               the FP32-normalised row, since
 *                                               rounding is monotone
 *   A == 0:  s = 0 and every code is 0
 *   else:    r = fl(127 / A)                  (one division per row)
 *            q_k = round-half-even(u_k * r)   of the exact product u_k * r,
 *                  clamped to [-127, 127] (never active: |u_k| <= A)
 * The codes equal round(127 * x_rot_k / amax(x_rot)); the normalisation
 * cancels, so it is applied to the scale only.
 * ------------------------------------------------------------------------- */
void orc_quant_row(const float *u, int64_t k, int g, int8_t *q, float *s)
{
    float a = 0.0f;
    for (int64_t i = 0; i < k; ++i) {
        float m = fabsf(u[i]);
        if (m > a) a = m;
    }
    if (a == 0.0f) {
        *s = 0.0f;
        memset(q, 0, (size_t)k);
        return;
    }
    float an = a * orc_norm_const(g);
    *s = an / 127.0f;
    float r = 127.0f / a;
    for (int64_t i = 0; i < k; ++i) {
        /* u * r is exact in double (24 + 24 significant bits). */
        double v = nearbyint((double)u[i] * (double)r);
        if (v > 127.0) v = 127.0;
        if (v < -127.0) v = -127.0;
        q[i] = (int8_t)v;
    }
}

/* Activation value a_k of one row, FP32 ([SWI] for act = 1). */
static void act_row(const uint16_t *xr, int64_t k, int act, float *a)
{
    if (act == 0) {
        for (int64_t i = 0; i < k; ++i) a[i] = bf16_to_f32(xr[i]);
    } else {
        for (int64_t i = 0; i < k; ++i) {
            float gate = bf16_to_f32(xr[i]);
            float up = bf16_to_f32(xr[k + i]);
            a[i] = orc_silu(gate) * up;
        }
    }
}

static int check_act_args(int64_t ldx, int64_t m, int64_t k, int act, int g)
{
    if (m < 0 || k <= 0 || !is_pow2_le(g, 4096) || k % g) return -1;
    if (act != 0 && act != 1) return -1;
    if (ldx < (act ? 2 * k : k)) return -1;
    return 0;
}

/* The rotated row as values: the pages define x H over the reals, where a zero
 * has no sign.  Reading: an exact zero of u is written as +0 (u + 0 changes no
 * other value; the codes and scales never see the sign of a zero). */
int orc_act_rotate(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, int act,
                   int g, float *u)
{
    if (check_act_args(ldx, m, k, act, g)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < m; ++r) {
        float *ur = u + r * k;
        act_row(x + r * ldx, k, act, ur);
        orc_fwht_groups(ur, k, g);
        for (int64_t j = 0; j < k; ++j) ur[j] = ur[j] + 0.0f;
    }
    return 0;
}

int orc_act_quant(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, int act,
                  int g, int8_t *q, float *s)
{
    if (check_act_args(ldx, m, k, act, g)) return -1;
#pragma omp parallel
    {
        float *u = (float *)malloc((size_t)k * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < m; ++r) {
            act_row(x + r * ldx, k, act, u);
            orc_fwht_groups(u, k, g);
            orc_quant_row(u, k, g, q + r * k, s + r);
        }
        free(u);
    }
    return 0;
}

/* [LOAD] weight preparation: W_rot = W H^T (H symmetric, so the same
 * blockwise transform as the activation), then per-row symmetric INT8. */
int orc_weight_prep(const float *w, int64_t n, int64_t k, int g, int8_t *q,
                    float *s)
{
    if (n < 0 || k <= 0 || !is_pow2_le(g, 4096) || k % g) return -1;
#pragma omp parallel
    {
        float *u = (float *)malloc((size_t)k * sizeof(float));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n; ++r) {
            memcpy(u, w + r * k, (size_t)k * sizeof(float));
            orc_fwht_groups(u, k, g);
            orc_quant_row(u, k, g, q + r * k, s + r);
        }
        free(u);
    }
    return 0;
}

/* [KEY], "Measured results": INT8 x INT8 products accumulated in int32.
 * Exact; |acc| <= 127^2 * k fits int32 for k <= 133143. */
void orc_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t m, int64_t n,
                  int64_t k, int32_t *acc)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < m; ++i) {
        const int8_t *xr = xq + i * k;
        for (int64_t j = 0; j < n; ++j) {
            const int8_t *wr = wq + j * k;
            int32_t sum = 0;
            for (int64_t t = 0; t < k; ++t) sum += (int32_t)xr[t] * (int32_t)wr[t];
            acc[i * n + j] = sum;
        }
    }
}

/* Round-to-nearest-even FP32 -> BF16 (finite inputs). */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = f32_as_u32(f);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

/* Dequant: the int32 accumulator times the token scale times the row scale,
 * rounded to BF16.  Pinned order: (f32(acc) * sx[m]) * sw[n], each product
 * rounded to FP32, then one BF16 rounding. */
void orc_dequant_bf16(const int32_t *acc, const float *sx, const float *sw,
                      int64_t m, int64_t n, uint16_t *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            float v = (float)acc[i * n + j]; /* int32 -> FP32, nearest even */
            v = v * sx[i];
            v = v * sw[j];
            y[i * n + j] = orc_f32_to_bf16(v);
        }
}

/* Epilogue with the optional bias and residual of a linear layer.
 * comfy-kitchen PR #277, "Changes": the INT8 linear is tested with bias and
 * residual; comfy-kitchen PR #248, commit list: input activations and
 * residuals are fused into the kernels.  The pages do not fix the FP32 order;
 * the reading taken is one FP32 sum in the epilogue, then one BF16 rounding:
 *   t = fl(fl(f32(acc) * sx[m]) * sw[n]);  t = fl(t + bias[n]);
 *   t = fl(t + f32(res[m, n]));  y = bf16(t)
 * bias is F32 [n] (may be NULL), res is BF16 [m, n] row-major (may be NULL). */
void orc_epilogue_bf16(const int32_t *acc, const float *sx, const float *sw,
                       const float *bias, const uint16_t *res, int64_t m, int64_t n,
                       uint16_t *y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            float v = (float)acc[i * n + j];
            v = v * sx[i];
            v = v * sw[j];
            if (bias) v = v + bias[j];
            if (res) v = v + bf16_to_f32(res[i * n + j]);
            y[i * n + j] = orc_f32_to_bf16(v);
        }
}

/* [SWI] "Motivation": the unfused path writes silu(gate) * up to HBM in BF16
 * (silu rounded to BF16 first, then the product rounded to BF16). */
void orc_eager_swiglu_bf16(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                           uint16_t *a)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < m; ++r)
        for (int64_t i = 0; i < k; ++i) {
            float gate = bf16_to_f32(x[r * ldx + i]);
            float up = bf16_to_f32(x[r * ldx + k + i]);
            float sg = bf16_to_f32(orc_f32_to_bf16(orc_silu(gate)));
            a[r * k + i] = orc_f32_to_bf16(sg * up);
        }
}
