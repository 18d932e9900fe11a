// probe.hip -- measurement kernels for the ceilings the path is measured
// against on MI355X (gfx950): an INT8 MFMA loop and a stream with a
// quantizer's read/write bytes.  They compute nothing the path uses; bench.py
// times them to state what the chip delivers under its power limit and for a
// given traffic pattern.
#include "ck_internal.hpp"

namespace ck {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// One 256-thread workgroup per CU, 16 independent 32 x 32 x 32 INT8 MFMA
// accumulators per wave with operands from `ops` (16 KB of codes staged in
// LDS).  LDS: every 16 MFMAs each wave also reads 8 operand fragments (1 KB
// each) from LDS for the next 16, the 0.5 KB per MFMA of the 256 x 256 GEMM
// tile, into the other of two register sets (no copies: a register an MFMA
// still reads is never overwritten).  The sink store never happens for real
// data; it keeps the MFMAs.
template <bool LDS>
__global__ __launch_bounds__(256) void mfma_loop_kernel(const v4i* __restrict__ ops, int iters, int* __restrict__ sink)
{
    __shared__ v4i buf[1024];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    for (int i = t; i < 1024; i += 256) buf[i] = ops[i];
    __syncthreads();
    v4i a[2][4], b[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[0][i] = a[1][i] = buf[i * 64 + lane];
        b[0][i] = b[1][i] = buf[(i + 4) * 64 + lane];
    }
    v16i acc[16];
#pragma unroll
    for (int f = 0; f < 16; ++f) acc[f] = v16i{};
    for (int it = 0; it < iters; it += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (LDS) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    a[h ^ 1][i] = buf[(((it + h + wave) & 1) * 512 + i * 64 + lane) & 1023];
                    b[h ^ 1][i] = buf[(((it + h + wave) & 1) * 512 + (i + 4) * 64 + lane) & 1023];
                }
            }
#pragma unroll
            for (int f = 0; f < 16; ++f)
                acc[f] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[h][f & 3], b[h][f >> 2], acc[f], 0, 0, 0);
        }
    }
    int s = 0;
#pragma unroll
    for (int f = 0; f < 16; ++f)
#pragma unroll
        for (int e = 0; e < 16; ++e) s ^= acc[f][e];
    if (s == 0x7fffffff) sink[blockIdx.x * 256 + t] = s;
}

// Rows of a quantizer's traffic: row r reads nr 16-byte chunks at
// src + r * ld_bytes and writes nw 8-byte chunks at dst + r * nw * 8 (nw <=
// nr), output chunk c folded from input chunk c.  A flat grid-stride stream
// over the m * nr chunks: consecutive threads take consecutive chunks, rows
// follow each other with no gap in the work, one load in flight per thread,
// kStreamWgsPerCu 256-thread workgroups per CU.  (Measured on 37.8 MB after a
// MALL flush: 2048 or 4096 workgroups of 256 threads and 256 of 1024 give the
// same time, and 4 or 8 loads in flight per thread no better.)
constexpr int kStreamWgsPerCu = 8;

__global__ __launch_bounds__(256) void stream_rows_kernel(const char* __restrict__ src, int64_t ld_bytes, int m,
                                                          int nr, int nw, uint2* __restrict__ dst)
{
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x, nt = (int64_t)gridDim.x * 256;
    int64_t row = t / nr;
    int c = (int)(t % nr);
    const int64_t drow = nt / nr;
    const int dc = (int)(nt % nr);
    while (row < m) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + row * ld_bytes + (int64_t)c * 16);
        if (c < nw) dst[row * nw + c] = make_uint2(v.x ^ v.z, v.y ^ v.w);
        row += drow;
        c += dc;
        if (c >= nr) {
            c -= nr;
            ++row;
        }
    }
}

}  // namespace

hipError_t launch_probe_mfma(const void* ops, int64_t iters, bool lds, int32_t* sink, hipStream_t st)
{
    const int n = num_cus();
    if (lds)
        hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(n), dim3(256), 0, st, static_cast<const v4i*>(ops), (int)iters,
                           sink);
    else
        hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(n), dim3(256), 0, st, static_cast<const v4i*>(ops), (int)iters,
                           sink);
    return hipGetLastError();
}

hipError_t launch_probe_stream(const void* src, int64_t ld_bytes, int64_t m, int64_t read_bytes, int64_t write_bytes,
                               void* dst, hipStream_t st)
{
    const int64_t chunks = m * (read_bytes / 16);
    const int64_t wgs = std::min<int64_t>((chunks + 255) / 256, (int64_t)kStreamWgsPerCu * num_cus());
    hipLaunchKernelGGL(stream_rows_kernel, dim3((unsigned)wgs), dim3(256), 0, st, static_cast<const char*>(src),
                       ld_bytes, (int)m, (int)(read_bytes / 16), (int)(write_bytes / 8), static_cast<uint2*>(dst));
    return hipGetLastError();
}

}  // namespace ck
