// gemm_fused.hip -- the few-row INT8 GEMM (decode or blocked weights) with the
// activation quantizer in front of it, in one kernel, for the fewest token rows.
//
// Sources: comfy-kitchen PR #277, "The key observation" (x_rot = x H, per-token
// INT8, y = x_rot W_rot^T with int32 accumulation); sglang PR #44196,
// "Motivation" and "Accuracy Tests" (input_act="swiglu": silu(gate) * up kept
// in FP32 inside the quantizer); comfy-kitchen PR #248 "Performance
// improvements for qwen 3.x (Part 2)", "Description" (at small M the layer is
// bound by streaming the weights).
//
// At a few token rows the activation is a few KB and its quantization is a
// separate launch of one or a few workgroups, which costs more than the
// arithmetic.  Here every workgroup of the decode GEMM (one per 16 weight rows)
// quantizes the rows itself, into LDS, with the quantizer's own FP32 steps
// (ck_device.hpp), so its codes and scales are those ck_act_quant writes:
// the rotation stays inside 16- or 32-lane groups and the row absmax is an
// exact maximum, so the result does not depend on the team's width (here the
// whole workgroup, 512 lanes).  The row data is loaded first, then the
// workgroup's first two batches of weights, so the weight stream is already in
// flight while the rows are rotated and quantized.  After that the loop is the
// few-row GEMM's (gemm_small.hip) with the activation fragments read from LDS.
//
// Every workgroup repeats the quantization, so it pays off only while that
// work is smaller than the launch it saves.  Measured (MI355X, c5's MLP at
// decode sizes, both weights in the decode layout, after a 512 MB read that
// evicts the MALL): at M = 1, 41.0 us with separate quantizers, 35.6 with the
// x quantizer fused, 29.8 with both; at M = 2, 41.5 -> 37.7 us with the x
// quantizer fused; at M = 3 and 4 the fused x quantizer is slower back to
// back (31.7 -> 34.2 us, 31.9 -> 37.4 us).  The SwiGLU variant repeats
// silu, the rotation and the absmax of whole rows of i values in each
// workgroup; at M = 2 it still gains a little (37.5 -> 35.8 us).  So both
// variants take up to 2 rows.
#include "ck_device.hpp"
#include "ck_internal.hpp"

namespace ck {
namespace fused {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int WAVES = 8;
constexpr int NT = WAVES * 64;   // threads per workgroup, all of them one quantizer team
[[maybe_unused]] constexpr int U = 8;             // 64-byte k-chunks per batch per wave
[[maybe_unused]] constexpr int PAD = 16;          // bytes after each LDS code row (spreads the 16 rows' banks)

// ACT 0: x BF16 [M, ldx]; ACT 1: [gate | up] BF16 [M, ldx] with SwiGLU; up to
// 2 rows.  CH: 8-element chunks per lane, K <= 8 * NT * CH.
template <int ACT>
struct FusedCfg {
    static constexpr int MAXR = 2;
};

// The rows' raw BF16 data: lane tid holds chunks c = j * NT + tid (8 values
// each) of row m < MAXR, zeros past the row or past M; for SwiGLU (ACT 1) also
// the up half, which starts at column K.
template <int ACT, int MAXR, int CH>
__device__ __forceinline__ void load_rows(const uint16_t* __restrict__ x, int64_t ldx, int M, int K, int tid,
                                          uint4 (&rg)[MAXR][CH], uint4 (&ru)[ACT ? MAXR : 1][ACT ? CH : 1])
{
    const int k8 = K >> 3;
#pragma unroll
    for (int m = 0; m < MAXR; ++m) {
        const uint16_t* rp = x + (int64_t)(m < M ? m : 0) * ldx;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = j * NT + tid;
            const bool ok = m < M && c < k8;
            rg[m][j] = ok ? *reinterpret_cast<const uint4*>(rp + c * 8) : make_uint4(0u, 0u, 0u, 0u);
            if constexpr (ACT)
                ru[m][j] = ok ? *reinterpret_cast<const uint4*>(rp + K + c * 8) : make_uint4(0u, 0u, 0u, 0u);
        }
    }
}

// Row m's values in FP32, the quantizer's first step: x, or silu(gate) * up.
template <int ACT, int MAXR, int CH>
__device__ __forceinline__ void row_values(int m, const uint4 (&rg)[MAXR][CH],
                                           const uint4 (&ru)[ACT ? MAXR : 1][ACT ? CH : 1], float (&v)[CH][8])
{
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const uint32_t w[4] = {rg[m][j].x, rg[m][j].y, rg[m][j].z, rg[m][j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[j][2 * e] = bf16_lo(w[e]);
            v[j][2 * e + 1] = bf16_hi(w[e]);
        }
        if constexpr (ACT) {
            const uint32_t wu[4] = {ru[m][j].x, ru[m][j].y, ru[m][j].z, ru[m][j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[j][2 * e] = silu_f32(w[e] << 16) * bf16_lo(wu[e]);
                v[j][2 * e + 1] = silu_f32(w[e] & 0xffff0000u) * bf16_hi(wu[e]);
            }
        }
    }
}

// DEC: W in the decode layout (scales in each group's header); else in the
// blocked layout with its row scales sw (n_rows: its padded row count).
template <int ACT, int LOG_G, int CH, bool DEC>
__global__ __launch_bounds__(NT) void gemm_dec_fused_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int8_t* __restrict__ wq, const float* __restrict__ sw,
    int M, int N, int K, int n_rows, float cg, void* __restrict__ out, EpiExtra ex)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int G = 1 << LOG_G;
    constexpr int MAXR = FusedCfg<ACT>::MAXR;
    constexpr int KMAX = 8 * NT * CH;
    __shared__ __attribute__((aligned(16))) int8_t xs[MAXR * (KMAX + PAD)];
    __shared__ float sxs[MAXR];
    __shared__ float wmax[WAVES];
    __shared__ v4i red[WAVES][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = blockIdx.x;       // 16-row group of W (output columns 16 nb ..)
    const int KC = K >> 6;           // 64-byte k-chunks
    const int k8 = K >> 3;           // 8-element chunks of a row
    const int xs_stride = K + PAD;

    // ---- the rows' raw BF16 data (issued first: the quantizer waits on it,
    // not on the weight loads issued after it) --------------------------------
    uint4 rg[MAXR][CH], ru[ACT ? MAXR : 1][ACT ? CH : 1];
    load_rows<ACT, MAXR, CH>(x, ldx, M, K, tid, rg, ru);

    // ---- the first two batches of this workgroup's weight stream -----------
    // W in the decode layout (include/ck.h): chunk j of group nb is the 1 KB at
    // nb * grp_bytes + 64 + 1024 j; lane l's 16 bytes hold row l % 16, k-bytes
    // 64 j + 16 (l / 16) .. + 16.  In the blocked layout the same 16 bytes sit
    // in 1 KB block 2 j + c / 2 of the 32-row block nb / 2, half c % 2 (c = l /
    // 16), at row offset 16 (l % 16), + 256 for the odd 16-row group.  Batch b
    // covers chunks wave + WAVES (U b + u).
    const uint32_t grp_bytes = 64u + 16u * (uint32_t)K;
    const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wq, (short)0, DEC ? (int)((uint32_t)(N / 16) * grp_bytes) : n_rows * K, 0x00020000);
    const int cq = lane >> 4;
    const uint32_t w_base = DEC ? (uint32_t)nb * grp_bytes + 64u + (uint32_t)lane * 16u
                                : (uint32_t)((nb >> 1) * (K >> 5)) * 1024u + (uint32_t)(nb & 1) * 256u +
                                      (uint32_t)((cq >> 1) * 1024 + (cq & 1) * 512 + (lane & 15) * 16);
    const uint32_t w_step = DEC ? 1024u : 2048u;
    auto load_w = [&](int b, v4i (&w)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = wave + WAVES * (U * b + u);
            w[u] = __builtin_amdgcn_raw_buffer_load_b128(rs_w, j < KC ? w_base + (uint32_t)j * w_step : kBufferOutside,
                                                         0, 0);
        }
    };
    const int batches = (KC + WAVES * U - 1) / (WAVES * U);
    v4i wa[U], wb[U];
    __builtin_amdgcn_sched_barrier(0);   // keep the row loads ahead of the weight loads
    load_w(0, wa);
    if (batches > 1) load_w(1, wb);

    // ---- quantize the rows into LDS (the quantizer's steps, team = NT) -----
#pragma unroll
    for (int m = 0; m < MAXR; ++m) {
        if (m >= M) break;
        float v[CH][8];
        row_values<ACT, MAXR, CH>(m, rg, ru, v);
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            fwht_in_lane<G>(v[j]);
            fwht_cross_lane<G>(v[j], tid);
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
        }
        amax = fmaxf(amax, swizzle_xor<1>(amax));
        amax = fmaxf(amax, swizzle_xor<2>(amax));
        amax = fmaxf(amax, swizzle_xor<4>(amax));
        amax = fmaxf(amax, swizzle_xor<8>(amax));
        amax = fmaxf(amax, swizzle_xor<16>(amax));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        if (lane == 0) wmax[wave] = amax;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < WAVES; ++w) amax = fmaxf(amax, wmax[w]);
        // s = fl(fl(A * c_g) / 127); r = fl(127 / A), or 0 for an all-zero row
        const float scale = (amax * cg) / 127.0f;
        const float r = amax > 0.0f ? 127.0f / amax : 0.0f;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = j * NT + tid;
            uint32_t b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) b[i] = code_bits(v[j][i], r);
            if (c < k8)
                *reinterpret_cast<uint2*>(xs + m * xs_stride + c * 8) =
                    make_uint2(pack4(b[0], b[1], b[2], b[3]), pack4(b[4], b[5], b[6], b[7]));
        }
        if (tid == 0) sxs[m] = scale;
        __syncthreads();   // codes visible; wmax free for the next row
    }

    // ---- the weight stream against the LDS codes ---------------------------
    // activation fragment of chunk j: lane l holds row l % 16 (rows past M
    // read row M - 1; their outputs are not stored), k-bytes 64 j + 16 (l / 16)
    const int r16 = lane & 15;
    const int xrow = r16 < M ? r16 : M - 1;
    const int8_t* xl = xs + xrow * xs_stride + (lane >> 4) * 16;
    v4i acc = {0, 0, 0, 0};
    auto compute = [&](int b, const v4i (&w)[U]) {
        v4i xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = wave + WAVES * (U * b + u);
            xv[u] = j < KC ? *reinterpret_cast<const v4i*>(xl + j * 64) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u], xv[u], acc, 0, 0, 0);
    };
    for (int b = 0; b < batches; b += 2) {
        compute(b, wa);
        if (b + 2 < batches) load_w(b + 2, wa);
        if (b + 1 >= batches) break;
        compute(b + 1, wb);
        if (b + 3 < batches) load_w(b + 3, wb);
    }

    // ---- sum the waves' partial accumulators (in wave order) ----------------
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4i t = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) t += red[w][lane];

    // ---- epilogue: lane l holds D[n = 4 (l / 16) + i][m = l % 16], i < 4 ----
    const int m = r16;
    const int n = nb * 16 + 4 * (lane >> 4);
    const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(out, (short)0, M * N * 2, 0x00020000);
    const float4 s4 = DEC ? *reinterpret_cast<const float4*>(wq + (size_t)nb * grp_bytes + 16 * (lane >> 4))
                          : *reinterpret_cast<const float4*>(sw + n);
    const float sxm = sxs[xrow];
    float y0 = ((float)t[0] * sxm) * s4.x;
    float y1 = ((float)t[1] * sxm) * s4.y;
    float y2 = ((float)t[2] * sxm) * s4.z;
    float y3 = ((float)t[3] * sxm) * s4.w;
    epi_extra4(y0, y1, y2, y3, ex, xrow, n, N);
    const u32x2 d = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
    const uint32_t row = (uint32_t)m * (uint32_t)N + (uint32_t)n;
    __builtin_amdgcn_raw_buffer_store_b64(d, rs_o, m < M ? row * 2u : kBufferOutside, 0, 0);
#endif  // __HIP_DEVICE_COMPILE__
}

// ---- W8A16 ---------------------------------------------------------------
// The same fusion for the W8A16 linear (comfy-kitchen PR #277, "Notes for the
// reviewer": the activation rotated but kept in BF16): every workgroup of the
// few-row W8A16 GEMM (gemm_small.hip; 16 weight rows in the blocked layout)
// rotates the rows into LDS as BF16, x_rot = bf16(fl(u * c_g)), the rotation
// kernel's own FP32 steps, then streams its weights against them.  No absmax,
// so no reduction across the team before the codes are known.  Each wave
// takes the k-chunks wave + 8 i in increasing order and does the two BF16
// MFMAs of a chunk in the same order as the few-row kernel, and the waves are
// summed in the same order, so the output equals the two-launch path's bit for
// bit.
constexpr int PADH = 8;   // BF16 values after each LDS row (16 bytes)

template <int ACT, int LOG_G, int CH>
__global__ __launch_bounds__(NT) void gemm_w8a16_fused_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, const int8_t* __restrict__ wq, const float* __restrict__ sw,
    int M, int N, int K, int n_rows, float cg, void* __restrict__ out, EpiExtra ex)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int G = 1 << LOG_G;
    constexpr int MAXR = FusedCfg<ACT>::MAXR;
    constexpr int KMAX = 8 * NT * CH;
    __shared__ __attribute__((aligned(16))) uint16_t xs[MAXR * (KMAX + PADH)];
    __shared__ v4f red[WAVES][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = blockIdx.x;       // 16-row group of W (output columns 16 nb ..)
    const int KB = K >> 5;           // 1 KB blocks per 32-row block of W
    const int KC = K >> 6;           // 64-value k-chunks
    const int k8 = K >> 3;
    const int xs_stride = K + PADH;

    uint4 rg[MAXR][CH], ru[ACT ? MAXR : 1][ACT ? CH : 1];
    load_rows<ACT, MAXR, CH>(x, ldx, M, K, tid, rg, ru);

    // W in the blocked layout: the 16 bytes of lane l = 16 c + r for chunk j
    // (row r of the group, k = 64 j + 16 c ..) sit in 1 KB block 2 j + c / 2 of
    // the 32-row block nb / 2, half c % 2, at row offset 16 r (+ 256 for the
    // odd 16-row group).
    const int r16 = lane & 15;
    const int cq = lane >> 4;
    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc((void*)wq, (short)0, n_rows * K, 0x00020000);
    const uint32_t w_base = (uint32_t)((nb >> 1) * KB) * 1024u + (uint32_t)(nb & 1) * 256u +
                            (uint32_t)((cq >> 1) * 1024 + (cq & 1) * 512 + r16 * 16);
    auto load_w = [&](int b, v4i (&w)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = wave + WAVES * (U * b + u);
            w[u] = __builtin_amdgcn_raw_buffer_load_b128(rs_w, j < KC ? w_base + (uint32_t)j * 2048u : kBufferOutside,
                                                         0, 0);
        }
    };
    const int batches = (KC + WAVES * U - 1) / (WAVES * U);
    v4i wa[U], wb[U];
    __builtin_amdgcn_sched_barrier(0);   // keep the row loads ahead of the weight loads
    load_w(0, wa);
    if (batches > 1) load_w(1, wb);

    // ---- rotate the rows into LDS (the rotation kernel's steps) ------------
#pragma unroll
    for (int m = 0; m < MAXR; ++m) {
        if (m >= M) break;
        float v[CH][8];
        row_values<ACT, MAXR, CH>(m, rg, ru, v);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            fwht_in_lane<G>(v[j]);
            fwht_cross_lane<G>(v[j], tid);
            const int c = j * NT + tid;
            const uint4 h = make_uint4(rot_bf16x2(v[j][0], v[j][1], cg), rot_bf16x2(v[j][2], v[j][3], cg),
                                       rot_bf16x2(v[j][4], v[j][5], cg), rot_bf16x2(v[j][6], v[j][7], cg));
            if (c < k8) *reinterpret_cast<uint4*>(xs + m * xs_stride + c * 8) = h;
        }
    }
    __syncthreads();

    // ---- the weight stream against the LDS rows ----------------------------
    // lane l's activation pieces of chunk j: row l % 16 (rows past M read row
    // M - 1; their outputs are not stored), k = 64 j + 16 (l / 16) + 8 s, s < 2
    const int xrow = r16 < M ? r16 : M - 1;
    const uint16_t* xl = xs + xrow * xs_stride + cq * 16;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](int b, const v4i (&w)[U]) {
        v4i xv[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = wave + WAVES * (U * b + u);
            const bool ok = j < KC;
            xv[u][0] = ok ? *reinterpret_cast<const v4i*>(xl + j * 64) : v4i{0, 0, 0, 0};
            xv[u][1] = ok ? *reinterpret_cast<const v4i*>(xl + j * 64 + 8) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bf16x8_t w0 = widen8(w[u][0], w[u][1]), w1 = widen8(w[u][2], w[u][3]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w0, __builtin_bit_cast(bf16x8_t, xv[u][0]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w1, __builtin_bit_cast(bf16x8_t, xv[u][1]), acc, 0, 0, 0);
        }
    };
    for (int b = 0; b < batches; b += 2) {
        compute(b, wa);
        if (b + 2 < batches) load_w(b + 2, wa);
        if (b + 1 >= batches) break;
        compute(b + 1, wb);
        if (b + 3 < batches) load_w(b + 3, wb);
    }

    // ---- sum the waves' partial accumulators (in wave order) ----------------
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    v4f t = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) t += red[w][lane];

    // ---- epilogue: lane l holds D[n = 4 (l / 16) + i][m = l % 16], i < 4 ----
    const int m = r16;
    const int n = nb * 16 + 4 * cq;
    const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(out, (short)0, M * N * 2, 0x00020000);
    const float4 s4 = *reinterpret_cast<const float4*>(sw + n);
    float y0 = t[0] * s4.x;
    float y1 = t[1] * s4.y;
    float y2 = t[2] * s4.z;
    float y3 = t[3] * s4.w;
    epi_extra4(y0, y1, y2, y3, ex, xrow, n, N);
    const u32x2 d = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
    const uint32_t row = (uint32_t)m * (uint32_t)N + (uint32_t)n;
    __builtin_amdgcn_raw_buffer_store_b64(d, rs_o, m < M ? row * 2u : kBufferOutside, 0, 0);
#endif  // __HIP_DEVICE_COMPILE__
}

template <int ACT, int LOG_G, int CH>
void launch_ch(const uint16_t* x, int64_t ldx, const int8_t* wq, const float* sw, bool dec, int M, int N, int K,
               float cg, uint16_t* y, hipStream_t st, EpiExtra ex)
{
    const int n_rows = (N + 255) / 256 * 256;
    if (dec)
        hipLaunchKernelGGL((gemm_dec_fused_kernel<ACT, LOG_G, CH, true>), dim3(N / 16), dim3(NT), 0, st, x, ldx, wq,
                           sw, M, N, K, n_rows, cg, static_cast<void*>(y), ex);
    else
        hipLaunchKernelGGL((gemm_dec_fused_kernel<ACT, LOG_G, CH, false>), dim3(N / 16), dim3(NT), 0, st, x, ldx, wq,
                           sw, M, N, K, n_rows, cg, static_cast<void*>(y), ex);
}

template <int ACT, int LOG_G>
hipError_t launch_g(int ch, const uint16_t* x, int64_t ldx, const int8_t* wq, const float* sw, bool dec, int M,
                    int N, int K, float cg, uint16_t* y, hipStream_t st, EpiExtra ex)
{
    if (ch == 1)
        launch_ch<ACT, LOG_G, 1>(x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
    else if (ch == 2)
        launch_ch<ACT, LOG_G, 2>(x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
    else if constexpr (ACT == 1) {
        if (ch == 3)
            launch_ch<ACT, LOG_G, 3>(x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
        else if (ch == 4)
            launch_ch<ACT, LOG_G, 4>(x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
        else
            return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int ACT, int LOG_G, int CH>
void launch_w8_ch(const uint16_t* x, int64_t ldx, const int8_t* wq, const float* sw, int M, int N, int K,
                  float cg, uint16_t* y, hipStream_t st, EpiExtra ex)
{
    const int n_rows = (N + 255) / 256 * 256;
    hipLaunchKernelGGL((gemm_w8a16_fused_kernel<ACT, LOG_G, CH>), dim3(N / 16), dim3(NT), 0, st, x, ldx, wq, sw, M,
                       N, K, n_rows, cg, static_cast<void*>(y), ex);
}

template <int ACT, int LOG_G>
hipError_t launch_w8_g(int ch, const uint16_t* x, int64_t ldx, const int8_t* wq, const float* sw, int M, int N,
                       int K, float cg, uint16_t* y, hipStream_t st, EpiExtra ex)
{
    if (ch == 1)
        launch_w8_ch<ACT, LOG_G, 1>(x, ldx, wq, sw, M, N, K, cg, y, st, ex);
    else if (ch == 2)
        launch_w8_ch<ACT, LOG_G, 2>(x, ldx, wq, sw, M, N, K, cg, y, st, ex);
    else if constexpr (ACT == 1) {
        if (ch == 3)
            launch_w8_ch<ACT, LOG_G, 3>(x, ldx, wq, sw, M, N, K, cg, y, st, ex);
        else if (ch == 4)
            launch_w8_ch<ACT, LOG_G, 4>(x, ldx, wq, sw, M, N, K, cg, y, st, ex);
        else
            return hipErrorInvalidValue;
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fused

bool use_fused_decode(int act, int64_t m, int64_t k, int g)
{
    if (g != 64 && g != 128 && g != 256) return false;
    if (act == 0) return m <= fused::FusedCfg<0>::MAXR && k <= 8 * fused::NT * 2;
    return m <= fused::FusedCfg<1>::MAXR && k <= 8 * fused::NT * 4;
}

hipError_t launch_gemm_dec_fused(int act, const uint16_t* x, int64_t ldx, int64_t m, int64_t k, int g,
                                 const int8_t* wq, const float* sw, bool dec, int64_t n, uint16_t* y, hipStream_t st,
                                 EpiExtra ex)
{
    if (!use_fused_decode(act, m, k, g)) return hipErrorInvalidValue;
    const int K = (int)k;
    const int ch = (K / 8 + fused::NT - 1) / fused::NT;
    const float cg = (float)(1.0 / sqrt((double)g));
    const int M = (int)m, N = (int)n;
    if (act == 0) {
        if (g == 64) return fused::launch_g<0, 6>(ch, x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
        if (g == 128) return fused::launch_g<0, 7>(ch, x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
        return fused::launch_g<0, 8>(ch, x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
    }
    if (g == 64) return fused::launch_g<1, 6>(ch, x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
    if (g == 128) return fused::launch_g<1, 7>(ch, x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
    return fused::launch_g<1, 8>(ch, x, ldx, wq, sw, dec, M, N, K, cg, y, st, ex);
}

}  // namespace ck

namespace ck {

hipError_t launch_gemm_w8a16_fused(int act, const uint16_t* x, int64_t ldx, int64_t m, int64_t k, int g,
                                   const int8_t* wq, const float* sw, int64_t n, uint16_t* y, hipStream_t st,
                                   EpiExtra ex)
{
    if (!use_fused_decode(act, m, k, g)) return hipErrorInvalidValue;
    const int K = (int)k;
    const int ch = (K / 8 + fused::NT - 1) / fused::NT;
    const float cg = (float)(1.0 / sqrt((double)g));
    const int M = (int)m, N = (int)n;
    if (act == 0) {
        if (g == 64) return fused::launch_w8_g<0, 6>(ch, x, ldx, wq, sw, M, N, K, cg, y, st, ex);
        if (g == 128) return fused::launch_w8_g<0, 7>(ch, x, ldx, wq, sw, M, N, K, cg, y, st, ex);
        return fused::launch_w8_g<0, 8>(ch, x, ldx, wq, sw, M, N, K, cg, y, st, ex);
    }
    if (g == 64) return fused::launch_w8_g<1, 6>(ch, x, ldx, wq, sw, M, N, K, cg, y, st, ex);
    if (g == 128) return fused::launch_w8_g<1, 7>(ch, x, ldx, wq, sw, M, N, K, cg, y, st, ex);
    return fused::launch_w8_g<1, 8>(ch, x, ldx, wq, sw, M, N, K, cg, y, st, ex);
}

}  // namespace ck
