/*
 * ck.h -- C ABI of the MI355X (gfx950) ConvRot INT8 linear and SwiGLU MLP.
 *
 * What the library computes (sources cited by page title and section):
 *
 *  - comfy-kitchen PR #277 "Add FP16 tensor-core fallback for int8_linear on
 *    devices without INT8 tensor cores", section "The key observation": the
 *    weight is stored pre-rotated, W_rot = W H^T; the activation is rotated
 *    online, x_rot = x H; the GEMM runs in the rotated basis, so
 *    y = x W^T = x_rot W_rot^T and no inverse rotation is applied to y.  The
 *    activation is quantized to INT8 on the same grid as the weight.  Section
 *    "Measured results": INT8 x INT8 products are accumulated in int32.
 *  - sglang PR #35994 report "[diffusion] Load serialized Comfy ConvRot INT8
 *    DiTs", key source excerpts: INT8 weights [out_features, in_features] with
 *    an F32 per-output-channel scale [out_features, 1] (per_channel=True,
 *    convrot=True); in_features must be divisible by the rotation group.
 *  - sglang PR #44196 (comfy_kitchen_swiglu_mlp), section "Motivation": the MLP
 *    runs as one packed [gate | up] int8_linear and a down projection whose
 *    quantizer applies the SwiGLU (input_act="swiglu"); section "Accuracy
 *    Tests": silu(gate) * up is kept in FP32, not rounded to BF16 first.
 *
 * H is block-diagonal over contiguous groups of `group` input channels, each
 * block the normalised Sylvester Hadamard matrix of that size.
 *
 * Numerics (identical, bit for bit, to the CPU oracle shipped with the tests):
 *  - rotation: unnormalised fast Walsh-Hadamard transform per group, strides
 *    1, 2, 4, ... ascending, FP32; the 1/sqrt(group) factor enters the scale;
 *  - per row: A = max |u|; scale = fl(fl(A * fl(1/sqrt(group))) / 127);
 *    codes = round-half-even(u * fl(127 / A)) of the exact product, in
 *    [-127, 127]; an all-zero row gets scale 0 and zero codes;
 *  - SwiGLU: a = silu(gate) * up in FP32 with a fixed exp/reciprocal procedure;
 *  - output: y = bf16_rne(fl(fl(f32(acc) * x_scale[m]) * w_scale[n])).
 *
 * Conventions shared by every entry point:
 *  - All pointers are DEVICE pointers (HBM) except where stated; tensors are
 *    row-major with a contiguous last dimension.  BF16 values are passed as
 *    their 16-bit patterns (uint16_t).  W is [out_features, in_features]
 *    (torch.nn.Linear layout).
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    workspace.  The library never allocates, frees or synchronises.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues kernels on that stream and returns; results are visible after the
 *    caller synchronises the stream.
 *  - Errors: every argument is checked on the host before anything is
 *    enqueued; a failed check returns a non-zero ck_status and enqueues
 *    nothing.  A failed launch returns CK_EHIP.  A fault inside a kernel
 *    surfaces at the caller's next synchronisation.
 *  - Shapes: m >= 0 (m == 0 is a no-op that returns CK_OK), n >= 0 (n == 0 is
 *    a no-op), k >= 1.  group is a power of two in [1, 256] dividing k; k is a
 *    multiple of 64 and at most CK_MAX_K; n is a multiple of 16.  Pointers are
 *    16-byte aligned; leading dimensions are multiples of 8 elements.
 *  - INT8 operand layouts (`layout` arguments), for an int8 matrix A [R, K]:
 *      CK_LAYOUT_ROWS     row-major, A[r][k] at byte r * K + k (R * K bytes).
 *      CK_LAYOUT_BLOCKED  rows padded to R_pad = ck_blocked_rows(R) (a multiple
 *                         of 256); 1 KB blocks, block (r / 32, k / 32) at byte
 *                         ((r / 32) * (K / 32) + k / 32) * 1024, and inside a
 *                         block A[r][k] at ((k % 32) / 16) * 512 + (r % 32) * 16
 *                         + k % 16.  R_pad * K bytes; padding rows are never
 *                         read into valid outputs.  A block is one 32-row x
 *                         32-byte MFMA operand fragment in lane order, so the
 *                         GEMM streams whole kilobytes from HBM into LDS and
 *                         reads LDS without bank conflicts.
 *    The blocked layout is the fast path; the row-major one is the serialized
 *    checkpoint format (sglang PR #35994 report, key source excerpts).
 */
#ifndef CK_H
#define CK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ck_status {
    CK_OK = 0,
    CK_EINVAL = 1,       /* null pointer, unknown act, misaligned pointer      */
    CK_ESHAPE = 2,       /* negative size, k % group, k % 64, n % 16, ld < k   */
    CK_EUNSUPPORTED = 3, /* group not a power of two <= 256, k > CK_MAX_K      */
    CK_EWORKSPACE = 4,   /* workspace too small or null                        */
    CK_EHIP = 5          /* the HIP runtime reported an error at launch        */
} ck_status;

typedef enum ck_act {
    CK_ACT_NONE = 0,     /* a = x                                              */
    CK_ACT_SWIGLU = 1    /* a = silu(x[:, 0:k]) * x[:, k:2k]  (gate, then up)  */
} ck_act;

typedef enum ck_layout {
    CK_LAYOUT_ROWS = 0,    /* row-major int8 [R, K]                             */
    CK_LAYOUT_BLOCKED = 1, /* 1 KB fragment blocks, rows padded to 256          */
    CK_LAYOUT_DECODE = 2   /* weights only, m <= 64: rows and scales interleaved */
} ck_layout;

/* Largest in_features: 127 * 127 * k must fit an int32 accumulator and one
 * activation row (k FP32 values) must fit the quantizer's LDS. */
#define CK_MAX_K 32768

/* Largest element count of one int8 operand or output buffer addressed with
 * 32-bit offsets by the GEMM kernels. */
#define CK_MAX_ELEMS 0x7fffffffLL

/* Library version string (static storage). */
const char *ck_version(void);

/* Human-readable name of a status code (static storage). */
const char *ck_status_str(ck_status s);

/* Weight preparation (done once per weight, at load).
 * Source: sglang PR #35994 report, key source excerpts (online quantization
 * with per_channel=True, convrot=True, stochastic_rounding=0, giving an I8
 * weight and an F32 [out_features, 1] scale); comfy-kitchen PR #277, "The key
 * observation" (the stored matrix is W H^T).
 *   w        [n, k] FP32, read
 *   w_q      [n, k] int8, written: codes of W H^T, row-quantized
 *   w_scale  [n]    FP32, written: one scale per output row
 * Errors: CK_EINVAL on null pointers; CK_ESHAPE/CK_EUNSUPPORTED on shapes. */
ck_status ck_weight_prep(const float *w, int64_t n, int64_t k, int32_t group,
                         int8_t *w_q, float *w_scale, void *stream);

/* Padded row count and byte size of an int8 [rows, k] matrix in the blocked
 * layout (0 for rows <= 0 or k <= 0). */
int64_t ck_blocked_rows(int64_t rows);
size_t ck_blocked_size(int64_t rows, int64_t k);

/* Decode layout (CK_LAYOUT_DECODE) of a weight [n, k] with its row scales,
 * for calls with m <= 64 (token-at-a-time decoding).  Source: comfy-kitchen
 * PR #248 "Performance improvements for qwen 3.x (Part 2)", "Description": at
 * small M the layer streams its weights, and interleaving the weights with
 * their scales makes that stream linear.  Each group of 16 rows b is one
 * contiguous region of 64 + 16 k bytes at byte b * (64 + 16 k): the 16 FP32
 * row scales of rows 16 b .. 16 b + 15, then k / 64 chunks of 1 KB, chunk c
 * holding W[16 b + r][64 c + 16 q + e] at byte 64 + 1024 c + 256 q + 16 r + e
 * (q < 4, r < 16, e < 16): one 16 x 64-byte MFMA operand in lane order.
 * A call with w_q in this layout ignores w_scale (it may be NULL); its
 * activation codes use the blocked layout.  m > 64 returns CK_EUNSUPPORTED.
 * ck_decode_size: bytes of the layout (0 for n <= 0 or k <= 0). */
size_t ck_decode_size(int64_t n, int64_t k);

/* Row-major codes and scales -> decode layout (done once, at load).
 *   w_q [n, k] int8 and w_scale [n] FP32 (from ck_weight_prep), read
 *   w_dec  ck_decode_size(n, k) bytes, written */
ck_status ck_weight_pack_decode(const int8_t *w_q, const float *w_scale, int64_t n,
                                int64_t k, void *w_dec, void *stream);

/* One-time relayout of prepared weights into the blocked layout.
 * Source: comfy-kitchen PR #248 "Performance improvements for qwen 3.x
 * (Part 2)", "Description" (weights are relaid out once so the GEMM reads them
 * linearly); the input is the serialized I8 [out_features, in_features] weight
 * of sglang PR #35994 report, key source excerpts.
 *   w_q      [n, k] int8 row-major, read
 *   w_blk    ck_blocked_size(n, k) bytes, written (padding rows zeroed) */
ck_status ck_weight_pack(const int8_t *w_q, int64_t n, int64_t k, int8_t *w_blk,
                         void *stream);

/* Activation quantizer: optional SwiGLU, rotation, per-token INT8.
 * Source: comfy-kitchen PR #277, "The key observation" (x_rot = x H, INT8 on
 * the weight's grid); sglang PR #44196, "Motivation" and "Accuracy Tests"
 * (input_act="swiglu", silu(gate) * up in FP32).
 *   x        [m, ldx] BF16, read.  act == CK_ACT_NONE: row r uses x[r, 0:k],
 *            ldx >= k.  act == CK_ACT_SWIGLU: gate = x[r, 0:k],
 *            up = x[r, k:2k], ldx >= 2k.
 *   x_q      int8 codes, written, in `layout` (below)
 *   x_scale  [m]    FP32, written */
ck_status ck_act_quant(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                       int32_t act, int32_t group, int32_t layout, int8_t *x_q,
                       float *x_scale, void *stream);
/*   layout   CK_LAYOUT_ROWS: x_q is [m, k] (m * k bytes); CK_LAYOUT_BLOCKED:
 *            x_q is ck_blocked_size(m, k) bytes (padding rows not written). */

/* ConvRot int8_linear: y = dequant(act_quant(x) . w_q^T) (+ bias + residual).
 * Source: comfy-kitchen PR #277, "The key observation" and "Measured results";
 * sglang PR #44196, "Motivation" (int8_linear(..., input_act="swiglu")).
 * Bias and residual: comfy-kitchen PR #277, "Changes" (the INT8 linear is
 * tested with bias and residual) and PR #248's commit list (residuals fused
 * into the kernels).
 *   x, ldx, act   as ck_act_quant
 *   w_q      int8 weight codes from ck_weight_prep (CK_LAYOUT_ROWS),
 *            ck_weight_pack (CK_LAYOUT_BLOCKED) or ck_weight_pack_decode
 *            (CK_LAYOUT_DECODE, m <= 64), read
 *   w_scale  [n]    FP32 from ck_weight_prep, read (ignored, may be NULL,
 *            with CK_LAYOUT_DECODE)
 *   bias     [n]    FP32, read, 16-byte aligned, or NULL
 *   residual [m, n] BF16 row-major (row stride n), read, 8-byte aligned, or
 *            NULL; it may be y itself (each element is read before it is
 *            written) but must not otherwise overlap y.
 *            Epilogue order: t = fl(fl(f32(acc) * x_scale[m]) * w_scale[n]);
 *            t = fl(t + bias[n]); t = fl(t + f32(residual[m, n])); y = bf16(t),
 *            round-to-nearest-even.
 *   layout   layout of w_q; the activation codes use the same one (blocked
 *            for CK_LAYOUT_DECODE)
 *   y        [m, n] BF16, written (row stride n)
 *   workspace  device buffer, 256-byte aligned, clobbered, of
 *            ck_int8_linear_workspace_size(m, k, n) bytes.  It holds x_q and
 *            x_scale (the first R(ck_blocked_size(m, k)) + R(4 m) bytes, R:
 *            rounded up to a multiple of 256; a smaller workspace is
 *            CK_EWORKSPACE) and, past them, the int32 partial sums of the
 *            split-K GEMM that CK_LAYOUT_BLOCKED uses for few output tiles
 *            (m >= 48, k >= 8192, tiles for only part of the CUs); a
 *            workspace without room for those runs the same shape unsplit.
 *            With CK_LAYOUT_BLOCKED or CK_LAYOUT_DECODE at m <= 2 (k <= 8192,
 *            or k <= 16384 with SwiGLU), group 64, 128 or 256, the quantizer runs
 *            inside the GEMM kernel and the workspace is left untouched (it is
 *            still required).  Every path gives the same result bit for bit. */
ck_status ck_int8_linear(const uint16_t *x, int64_t ldx, int32_t act,
                         const int8_t *w_q, const float *w_scale, const float *bias,
                         const uint16_t *residual, int32_t layout,
                         int64_t m, int64_t n, int64_t k, int32_t group,
                         uint16_t *y, void *workspace, size_t workspace_bytes,
                         void *stream);
size_t ck_int8_linear_workspace_size(int64_t m, int64_t k, int64_t n);

/* ck_int8_linear without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It allocates nothing; the activation
 * codes and row scales go to a scratch buffer of CK_NOALLOC_SCRATCH_BYTES
 * that the library holds in device memory, one per GPU, reserved when the
 * library's code is loaded on that GPU and kept until the process ends.
 *   Arguments, results and errors as ck_int8_linear, on the calling thread's
 *   current device (`stream` must belong to it), with one more limit: when
 *   x_q and x_scale (R(ck_blocked_size(m, k)) + R(4 m) bytes, R as there)
 *   exceed CK_NOALLOC_SCRATCH_BYTES the call returns CK_EWORKSPACE and
 *   enqueues nothing (64 MiB holds m = 4096 rows at k = 16384); the split-K
 *   partials use the rest of the buffer when they fit.  CK_EHIP if the
 *   scratch's device address cannot be queried.
 *   Every call on one GPU uses that GPU's one buffer, and the buffer keeps
 *   the last call's contents: calls that may overlap on one GPU (different
 *   streams, or host threads without an order between them) race on it and
 *   must not be issued.  Calls in one stream are ordered and safe. */
#define CK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
size_t ck_noalloc_scratch_bytes(void);
ck_status ck_int8_linear_noalloc(const uint16_t *x, int64_t ldx, int32_t act,
                                 const int8_t *w_q, const float *w_scale, const float *bias,
                                 const uint16_t *residual, int32_t layout,
                                 int64_t m, int64_t n, int64_t k, int32_t group,
                                 uint16_t *y, void *stream);

/* The INT8 GEMM with its dequant epilogue alone (the second half of
 * ck_int8_linear), for callers that hold quantized activations.
 *   x_q, w_q int8 codes in `layout` (both), x_scale [m], w_scale [n] FP32,
 *   read; bias, residual as ck_int8_linear (either may be NULL); y [m, n]
 *   BF16 written. */
ck_status ck_int8_gemm_bf16(const int8_t *x_q, const float *x_scale,
                            const int8_t *w_q, const float *w_scale,
                            const float *bias, const uint16_t *residual,
                            int32_t layout, int64_t m, int64_t n, int64_t k,
                            uint16_t *y, void *stream);

/* SwiGLU MLP block: y = int8_linear(int8_linear(x, W_gu), W_down, swiglu).
 * Source: sglang PR #44196, "Motivation" and "Modifications" (one packed
 * [gate | up] GEMM whose gate rows come first, then the down projection that
 * applies silu(gate) * up inside its quantizer); "Accuracy Tests" (the stacked
 * GEMM does the same per-column arithmetic as two separate projections).
 *   x      [m, h]  BF16, read
 *   w_gu   [2i, h] int8 + s_gu [2i] FP32: rows 0..i-1 gate, i..2i-1 up
 *   w_down [h, i]  int8 + s_down [h] FP32
 *   layout layout of both weights (and of the internal activation codes;
 *          with CK_LAYOUT_DECODE, m <= 64, s_gu and s_down may be NULL)
 *   y      [m, h]  BF16, written
 *   workspace  ck_swiglu_mlp_workspace_size(m, h, i) bytes, 256-byte
 *          aligned; clobbered (x codes/scales, the [m, 2i] BF16 gate|up
 *          output, its codes/scales, then room for the split-K partials either
 *          GEMM takes with CK_LAYOUT_BLOCKED as in ck_int8_linear; a workspace
 *          short of that room, but holding the rest, runs both unsplit; with
 *          CK_LAYOUT_BLOCKED or CK_LAYOUT_DECODE at the fewest rows a stage's
 *          quantizer runs inside its GEMM, as in ck_int8_linear, and its codes
 *          are not written). */
ck_status ck_swiglu_mlp(const uint16_t *x, const int8_t *w_gu, const float *s_gu,
                        const int8_t *w_down, const float *s_down, int32_t layout,
                        int64_t m, int64_t h, int64_t i, int32_t group, uint16_t *y,
                        void *workspace, size_t workspace_bytes, void *stream);
size_t ck_swiglu_mlp_workspace_size(int64_t m, int64_t h, int64_t i);

/* ---- W8A16: INT8 weights, BF16 activations (no activation quantization) ----
 * Source: comfy-kitchen PR #277, "Notes for the reviewer": a variant that keeps
 * the rotated activation in 16-bit floating point instead of quantizing it to
 * INT8 (a different quantization grid, closer to the float32 result), with
 * the INT8 weights widened on the fly; "The key observation": the GEMM runs in
 * the rotated basis, so the widened W_rot is used as it is.  On this target
 * the activation type is BF16 and the product accumulates in FP32.
 *
 * BF16 blocked layout (activations of these calls): rows padded to a multiple
 * of 256; the 32 values k = 32 j .. 32 j + 31 of the 32-row block r / 32 are
 * 2 KB at byte ((r / 32) * (k / 32) + j) * 2048, value (r, k) inside at byte
 * ((k % 16) / 8) * 1024 + ((k % 32) / 16) * 512 + (r % 32) * 16 + (k % 8) * 2:
 * two 1 KB BF16 MFMA operands that pair with one 1 KB block of the INT8
 * blocked weight. */

/* Rotated activation in BF16: a (= x, or silu(gate) * up for CK_ACT_SWIGLU,
 * in FP32), u = the unnormalised blockwise FWHT of a (as ck_act_quant),
 * x_rot = bf16(fl(u * fl(1 / sqrt(group))) + 0): an exact zero is +0.
 *   layout  CK_LAYOUT_ROWS: x_rot [m, k] row-major; CK_LAYOUT_BLOCKED: the
 *           BF16 blocked layout, ck_blocked_size(m, k) * 2 bytes (the padding
 *           rows are not written)
 * Errors as ck_act_quant. */
ck_status ck_act_rotate_bf16(const uint16_t *x, int64_t ldx, int64_t m, int64_t k,
                             int32_t act, int32_t group, int32_t layout, uint16_t *x_rot,
                             void *stream);

/* y[m, n] = bf16(fl(acc[m, n] * w_scale[n]) (+ bias[n]) (+ residual[m, n])),
 * acc = sum_k x_rot[m, k] * w_q[n, k] accumulated in FP32 (order unspecified;
 * every product is exact in FP32).  x_rot in the BF16 blocked layout, w_q in
 * CK_LAYOUT_BLOCKED (ck_weight_pack); bias and residual as ck_int8_linear.
 * k % 64 == 0, n % 16 == 0.  Errors: CK_EINVAL on null or misaligned
 * pointers; CK_ESHAPE on shapes; CK_EUNSUPPORTED past the 32-bit extents. */
ck_status ck_w8a16_gemm_bf16(const uint16_t *x_rot, const int8_t *w_q, const float *w_scale,
                             const float *bias, const uint16_t *residual, int64_t m, int64_t n,
                             int64_t k, uint16_t *y, void *stream);

/* The W8A16 linear: ck_act_rotate_bf16 (blocked) into the workspace, then
 * ck_w8a16_gemm_bf16.  Arguments as ck_int8_linear with w_q in
 * CK_LAYOUT_BLOCKED; workspace of ck_int8_linear_w8a16_workspace_size(m, k)
 * bytes, 256-byte aligned, clobbered.  At m <= 2 (k <= 8192, or k <= 16384
 * with CK_ACT_SWIGLU; group 64, 128 or 256) one kernel rotates the rows
 * itself and the workspace is left untouched; the output is the same bits. */
ck_status ck_int8_linear_w8a16(const uint16_t *x, int64_t ldx, int32_t act, const int8_t *w_q,
                               const float *w_scale, const float *bias, const uint16_t *residual,
                               int64_t m, int64_t n, int64_t k, int32_t group, uint16_t *y,
                               void *workspace, size_t workspace_bytes, void *stream);
size_t ck_int8_linear_w8a16_workspace_size(int64_t m, int64_t k);

/* The SwiGLU MLP block with W8A16 linears (as ck_swiglu_mlp, with both
 * rotated activations kept in BF16): rotate x, the packed [gate | up] W8A16
 * GEMM to BF16, then silu(gate) * up rotated to BF16 and the down W8A16 GEMM.
 * Weights in CK_LAYOUT_BLOCKED; workspace of
 * ck_swiglu_mlp_w8a16_workspace_size(m, h, i) bytes, 256-byte aligned.  At
 * the sizes where ck_int8_linear_w8a16 is one kernel, each stage's rotation
 * runs inside its GEMM and the rotated activations are not written. */
ck_status ck_swiglu_mlp_w8a16(const uint16_t *x, const int8_t *w_gu, const float *s_gu,
                              const int8_t *w_down, const float *s_down, int64_t m, int64_t h,
                              int64_t i, int32_t group, uint16_t *y, void *workspace,
                              size_t workspace_bytes, void *stream);
size_t ck_swiglu_mlp_w8a16_workspace_size(int64_t m, int64_t h, int64_t i);

/* ---- test hooks: the same device code with its intermediate exposed ---- */

/* Raw int32 accumulators acc[m, n] = sum_k x_q[m, k] * w_q[n, k] from the
 * production GEMM kernels (comfy-kitchen PR #277, "Measured results"). */
ck_status ck_int8_gemm_i32(const int8_t *x_q, const int8_t *w_q, int32_t layout,
                           int64_t m, int64_t n, int64_t k, int32_t *acc,
                           void *stream);

/* Raw FP32 accumulators acc[m, n] of the W8A16 GEMM (operands as
 * ck_w8a16_gemm_bf16). */
ck_status ck_w8a16_gemm_f32(const uint16_t *x_rot, const int8_t *w_q, int64_t m, int64_t n,
                            int64_t k, float *acc, void *stream);

/* FP32 silu of n BF16 gate values, by the quantizer's own device function
 * (sglang PR #44196, "Accuracy Tests": silu kept in FP32). */
ck_status ck_silu_f32(const uint16_t *gate, int64_t n, float *out, void *stream);

/* Unnormalised rotated activation u [m, k] FP32 (before quantization), by the
 * quantizer's own device code (comfy-kitchen PR #277, "The key observation");
 * an exact zero is written as +0. */
ck_status ck_act_rotate_f32(const uint16_t *x, int64_t ldx, int64_t m,
                            int64_t k, int32_t act, int32_t group, float *u,
                            void *stream);

/* ---- measurement hooks: what the chip delivers, for the rooflines ----
 * These compute nothing the path uses.  bench.py times them beside the path's
 * kernels (MI355X is power-limited: its INT8 rate depends on the operand bits,
 * and its HBM rate on the traffic pattern). */

/* INT8 MFMA loop: one 256-thread workgroup per CU; each wave repeats `iters`
 * times 16 independent v_mfma_i32_32x32x32_i8 (65,536 ops each) on operand
 * fragments taken from `ops` (16 KB of INT8 codes, device, 16-byte aligned).
 * lds != 0: each wave also reads 8 fragments (8 KB) from LDS per 16 MFMAs,
 * the operand traffic of the 256 x 256 GEMM tile.  ops per call:
 * ck_probe_mfma_workgroups() * 4 * iters * 16 * 65536.  sink: device int32
 * [ck_probe_mfma_workgroups() * 256], never written for real operand data.
 * Errors: CK_EINVAL on null or misaligned pointers, CK_ESHAPE on iters < 0 or
 * odd (the loop alternates two operand register sets). */
int64_t ck_probe_mfma_workgroups(void);
ck_status ck_probe_mfma_i8(const int8_t *ops, int64_t iters, int32_t lds, int32_t *sink,
                           void *stream);

/* Stream with a quantizer's traffic and trivial compute: m rows; row r
 * reads read_bytes at src + r * ld_bytes and writes write_bytes at
 * dst + r * write_bytes (a flat grid-stride loop over the 16-byte chunks).  read_bytes % 16 == 0, read_bytes <= 65536,
 * write_bytes % 8 == 0, write_bytes / 8 <= read_bytes / 16,
 * ld_bytes >= read_bytes, ld_bytes % 16 == 0; src 16-byte and dst 8-byte
 * aligned.  Errors: CK_EINVAL (pointers), CK_ESHAPE (sizes),
 * CK_EUNSUPPORTED (more than 2^31 rows). */
ck_status ck_probe_stream_rows(const void *src, int64_t ld_bytes, int64_t m, int64_t read_bytes,
                               int64_t write_bytes, void *dst, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* CK_H */
