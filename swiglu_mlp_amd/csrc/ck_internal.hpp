// ck_internal.hpp -- launchers shared between the kernel translation units and
// the C ABI layer.  Each launcher only enqueues work on `st`; argument checks
// are done by the caller (api.hip) before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck {

// Rotation + per-row INT8 quantization of m rows of k values.
// kind: 0 = BF16 x[r, 0:k]; 1 = BF16 [gate | up] with SwiGLU; 2 = FP32 rows.
// u_out != nullptr selects the diagnostic variant that writes the unnormalised
// rotated FP32 rows instead of codes and scales.
hipError_t launch_quant_rows(int kind, const void* src, int64_t ld, int64_t m, int64_t k, int g,
                             int8_t* q, float* s, float* u_out, hipStream_t st);

// FP32 silu of n BF16 values (the quantizer's device function).
hipError_t launch_silu(const uint16_t* g, int64_t n, float* out, hipStream_t st);

// y[m, n] = bf16(fl(fl(f32(x_q . w_q^T) * sx[m]) * sw[n])).
hipError_t launch_gemm_bf16(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                            int64_t m, int64_t n, int64_t k, uint16_t* y, hipStream_t st);

// acc[m, n] = x_q . w_q^T in int32.
hipError_t launch_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                           int32_t* acc, hipStream_t st);

}  // namespace ck
