/*
 * convrot_oracle.h -- plain CPU oracle of the ConvRot INT8 linear and the
 * SwiGLU MLP block built on it.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library under swiglu_mlp_amd/) never calls it and shares no code,
 * header, table or constant generator with it.
 *
 * Sources (cited by page title and section):
 *  [KEY]   comfy-kitchen PR #277 "Add FP16 tensor-core fallback for int8_linear
 *          on devices without INT8 tensor cores", section "The key observation":
 *          W_rot = W H^T is stored, x_rot = x H is formed online, the GEMM runs
 *          in the rotated basis, and the activation is quantized to INT8 on the
 *          same grid as the weight.  Section "Measured results": int32
 *          accumulation on the INT8 path.
 *  [SWI]   sglang PR #44196 (comfy_kitchen_swiglu_mlp), sections "Motivation"
 *          and "Accuracy Tests": packed [gate | up] GEMM, then a down
 *          projection whose quantizer applies silu(gate) * up kept in FP32.
 *  [LOAD]  sglang PR #35994 report "[diffusion] Load serialized Comfy ConvRot
 *          INT8 DiTs", section on the key source excerpts: per-output-channel
 *          (per_channel=True, convrot=True) INT8 weights with an F32 [out, 1]
 *          row scale; in_features must be divisible by the rotation group.
 *
 * Where the pages leave the FP32 operation order open, this oracle pins one
 * reading; every such reading is listed beside the function that makes it.
 * All arithmetic is IEEE binary32 round-to-nearest-even with no contraction
 * (the file is compiled with -ffp-contract=off); fmaf() is used only where a
 * fused multiply-add is part of the pinned definition.
 */
#ifndef CONVROT_ORACLE_H
#define CONVROT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Normalised Sylvester Hadamard H_g (g a power of two), g*g doubles, row-major. */
int orc_hadamard(int g, double *h);

/* Pinned elementary functions (exported so the test-suite can pin them). */
float orc_exp_neg(float gc);      /* e^{-gc} for gc in [-80, 80]            */
float orc_rcp(float d);           /* 1/d for d >= 1 (normal, finite)        */
float orc_silu(float gamma);      /* silu in FP32 as pinned below           */
float orc_norm_const(int g);      /* fl(1/sqrt(g))                          */
uint16_t orc_f32_to_bf16(float f);/* round-to-nearest-even                  */

void orc_exp_neg_v(const float *x, int64_t n, float *y);
void orc_rcp_v(const float *x, int64_t n, float *y);
void orc_silu_v(const uint16_t *gate_bf16, int64_t n, float *y);

/* In-place unnormalised FWHT of each contiguous group of g floats. */
void orc_fwht_groups(float *v, int64_t n, int g);

/* One row: amax, scale and codes from the unnormalised rotated values u. */
void orc_quant_row(const float *u, int64_t k, int g, int8_t *q, float *s);

/* Activation quantizer.  act = 0: x is [m, ldx] BF16, row r reads x[r, 0:k].
 * act = 1 (swiglu): row r reads gate = x[r, 0:k], up = x[r, k:2k].
 * Writes q [m, k] int8 and s [m] float.  Returns 0, or -1 on bad arguments. */
int orc_act_quant(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, int act,
                  int g, int8_t *q, float *s);

/* Rotated-but-unquantized FP32 activation (unnormalised), for diagnostics;
 * an exact zero is written as +0. */
int orc_act_rotate(const uint16_t *x, int64_t ldx, int64_t m, int64_t k, int act,
                   int g, float *u);

/* Weight preparation: W [n, k] FP32 -> W_q [n, k] int8 + s_w [n] float. */
int orc_weight_prep(const float *w, int64_t n, int64_t k, int g, int8_t *q,
                    float *s);

/* Exact int32 GEMM: acc[m, n] = sum_k xq[m, k] * wq[n, k]. */
void orc_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t m, int64_t n,
                  int64_t k, int32_t *acc);

/* Dequant epilogue: y = bf16(fl(fl(f32(acc) * sx[m]) * sw[n])). */
void orc_dequant_bf16(const int32_t *acc, const float *sx, const float *sw,
                      int64_t m, int64_t n, uint16_t *y);

/* Epilogue with optional F32 bias [n] and BF16 residual [m, n] (either may be
 * NULL): y = bf16(fl(fl(fl(fl(f32(acc) * sx[m]) * sw[n]) + bias[n]) + res[m, n])). */
void orc_epilogue_bf16(const int32_t *acc, const float *sx, const float *sw,
                       const float *bias, const uint16_t *res, int64_t m, int64_t n,
                       uint16_t *y);

/* Eager (unfused) SwiGLU activation: a = bf16(bf16(silu(gate)) * up),
 * written back as BF16 [m, k]; the path the fused quantizer replaces. */
void orc_eager_swiglu_bf16(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                           uint16_t *a);

#ifdef __cplusplus
}
#endif
#endif
