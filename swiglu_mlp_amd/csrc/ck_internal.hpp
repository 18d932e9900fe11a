// ck_internal.hpp -- launchers shared between the kernel translation units and
// the C ABI layer.  Each launcher only enqueues work on `st`; argument checks
// are done by the caller (api.hip) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ck_device.hpp"

namespace ck {

// Rotation + per-row INT8 quantization of m rows of k values.
// kind: 0 = BF16 x[r, 0:k]; 1 = BF16 [gate | up] with SwiGLU; 2 = FP32 rows.
// u_out != nullptr selects the diagnostic variant that writes the unnormalised
// rotated FP32 rows instead of codes and scales.
// blocked: write the codes in the blocked layout (rows padded to 256, see
// include/ck.h) instead of row-major.
hipError_t launch_quant_rows(int kind, const void* src, int64_t ld, int64_t m, int64_t k, int g,
                             int8_t* q, float* s, float* u_out, bool blocked, hipStream_t st);

// Rotation of m rows of k values (kind 0 or 1 as above) to BF16
// x_rot = bf16(fl(u * fl(1/sqrt(g)))), u the unnormalised blockwise FWHT;
// written row-major [m, k] or, blocked, in the BF16 blocked layout.
hipError_t launch_rotate_bf16(int kind, const void* src, int64_t ld, int64_t m, int64_t k, int g,
                              uint16_t* out, bool blocked, hipStream_t st);

// The decode-layout GEMM with the activation quantizer fused in front, for the
// fewest rows (m <= 2): act 0 (BF16 x [m, ldx], k <= 8192) or 1 (BF16
// [gate | up] [m, ldx] with SwiGLU, k <= 16384), g in {64, 128, 256}.
// Writes y = bf16(fl(fl(f32(acc) * sx[m]) * sw[n])) (+ ex) with the codes and
// scales launch_quant_rows would have written.
bool use_fused_decode(int act, int64_t m, int64_t k, int g);
hipError_t launch_gemm_dec_fused(int act, const uint16_t* x, int64_t ldx, int64_t m, int64_t k, int g,
                                 const int8_t* wq, const float* sw, bool dec, int64_t n, uint16_t* y,
                                 hipStream_t st, EpiExtra ex = EpiExtra{});
// The W8A16 linear at the same sizes (use_fused_decode): the BF16 rotation
// inside the few-row W8A16 GEMM, W in the blocked layout with its row scales sw.
hipError_t launch_gemm_w8a16_fused(int act, const uint16_t* x, int64_t ldx, int64_t m, int64_t k, int g,
                                   const int8_t* wq, const float* sw, int64_t n, uint16_t* y, hipStream_t st,
                                   EpiExtra ex = EpiExtra{});

// Row-major [n, k] int8 -> blocked layout, padding rows zero-filled.
hipError_t launch_pack_blocked(const int8_t* w, int64_t n, int64_t k, int8_t* out, hipStream_t st);

// FP32 silu of n BF16 values (the quantizer's device function).
hipError_t launch_silu(const uint16_t* g, int64_t n, float* out, hipStream_t st);

// y[m, n] = bf16(fl(fl(f32(x_q . w_q^T) * sx[m]) * sw[n])); both operands in
// the row-major or the blocked layout.
// `ex` adds an optional bias and residual before the BF16 rounding.
// layout: 0 rows, 1 blocked, 2 decode (W only; the activation codes are blocked).
// ws / ws_bytes: optional room for split-K partials (blocked layout; see
// gemm_splitk_bytes); without it every shape runs unsplit.
hipError_t launch_gemm_bf16(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                            int64_t m, int64_t n, int64_t k, uint16_t* y, int layout, hipStream_t st,
                            EpiExtra ex = EpiExtra{}, void* ws = nullptr, size_t ws_bytes = 0);

// acc[m, n] = x_q . w_q^T in int32.
hipError_t launch_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                           int32_t* acc, int layout, hipStream_t st);

// Blocked-layout GEMM (gemm_blk.hip).
hipError_t launch_gemm_blk(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                           int64_t m, int64_t n, int64_t k, void* out, bool out_i32, int num_cu,
                           hipStream_t st, EpiExtra ex = EpiExtra{});

// Split-K form of the blocked BF16 GEMM for few-tile shapes (gemm_blk.hip):
// gemm_splitk_bytes is the int32 partial buffer its plan needs on the current
// device (0: no split for this shape).  launch_gemm_blk_splitk enqueues the
// split GEMM and its reduction, with the partials in ws, and returns true, or
// returns false without enqueuing anything when the shape takes no split or
// ws is smaller than the plan needs (*err: the launch status).
size_t gemm_splitk_bytes(int64_t m, int64_t n, int64_t k);
bool launch_gemm_blk_splitk(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, int64_t m,
                            int64_t n, int64_t k, uint16_t* y, hipStream_t st, EpiExtra ex, void* ws,
                            size_t ws_bytes, hipError_t* err);

// W8A16 GEMM (gemm_blk.hip): x_rot BF16 in the BF16 blocked layout, W INT8
// blocked; y = bf16(fl(acc * sw[n])) with FP32 accumulation, or (out_f32) the
// raw FP32 accumulators.
hipError_t launch_gemm_w8a16(const uint16_t* x_rot, const int8_t* wq, const float* sw, int64_t m,
                             int64_t n, int64_t k, void* out, bool out_f32, hipStream_t st,
                             EpiExtra ex = EpiExtra{});

// Blocked-layout GEMM for m <= 64 (gemm_small.hip): streams the weights once.
// decode: W in the decode layout (sw unused).
hipError_t launch_gemm_small(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                             int64_t m, int64_t n, int64_t k, void* out, bool out_i32, hipStream_t st,
                             EpiExtra ex = EpiExtra{}, bool decode = false);

// W8A16 for m <= 64 (gemm_small.hip): x_rot in the BF16 blocked layout, W blocked.
hipError_t launch_gemm_small_w8a16(const uint16_t* x_rot, const int8_t* wq, const float* sw, int64_t m,
                                   int64_t n, int64_t k, void* out, bool out_f32, hipStream_t st,
                                   EpiExtra ex = EpiExtra{});

// Row-major codes + scales -> decode layout (include/ck.h).
hipError_t launch_pack_decode(const int8_t* w, const float* sw, int64_t n, int64_t k, void* out,
                              hipStream_t st);

// Largest m of a call with weights in the decode layout.
constexpr int64_t kDecodeMaxM = 64;
// Largest m the weight-streaming kernel takes (eight 16-row fragments).
constexpr int64_t kSmallMaxM = 128;

// Blocked-layout GEMMs take the weight-streaming kernel when m <= 32, or when
// m <= kSmallMaxM and it runs at most one workgroup per CU (n <= 16 * CUs).
bool use_small_kernel(int64_t m, int64_t n);

int num_cus();

// Measurement kernels (probe.hip): the INT8 MFMA loop on one workgroup per CU
// (optionally reading 0.5 KB of LDS per MFMA), and a row stream with a given
// read / write byte count per row.
hipError_t launch_probe_mfma(const void* ops, int64_t iters, bool lds, int32_t* sink, hipStream_t st);
hipError_t launch_probe_stream(const void* src, int64_t ld_bytes, int64_t m, int64_t read_bytes, int64_t write_bytes,
                               void* dst, hipStream_t st);

// Persistent large-tile GEMM (256 x bn tiles, bn = 256 or 192), one workgroup
// per CU; writes BF16 y (with scales) or int32 acc (out_i32).
hipError_t launch_gemm_big(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                           int64_t m, int64_t n, int64_t k, void* out, bool out_i32, int bn,
                           int num_cu, hipStream_t st, EpiExtra ex = EpiExtra{});

}  // namespace ck
