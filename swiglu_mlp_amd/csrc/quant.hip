// quant.hip -- fused (SwiGLU) + blockwise Hadamard rotation + per-row INT8
// quantizer for gfx950, used for activations (per token) and, with FP32 input,
// for weight preparation (per output row).
//
// Sources: comfy-kitchen PR #277, "The key observation" (x_rot = x H online,
// W_rot = W H^T stored, INT8 on one grid); sglang PR #44196, "Motivation" and
// "Accuracy Tests" (input_act="swiglu", silu(gate) * up kept in FP32);
// sglang PR #35994 report, key source excerpts (per-output-channel INT8 weight
// with an F32 [out, 1] scale).
//
// Work decomposition: a row is owned by a team of T lanes (T a power of two,
// 8 <= T <= 256, T a multiple of group/8).  Lane t of the team holds chunks
// c = j*T + t (j < CH) of 8 consecutive elements, so each load instruction
// reads consecutive 16-byte pieces across the team (coalesced) and the 16 lanes
// of one 128-element group are adjacent (the cross-lane butterflies stay in a
// swizzle group).  The whole rotated row stays in registers until the row's
// absmax is known; codes are then written once.  A workgroup holds 256/T rows.
// The kernel is bound by HBM and by VALU issue; every per-element step is a
// single VALU op except the SwiGLU's exp/reciprocal.
#include <algorithm>

#include "ck_device.hpp"
#include "ck_internal.hpp"

namespace ck {

enum InKind { IN_BF16 = 0, IN_BF16_SWIGLU = 1, IN_F32 = 2 };

// Byte offset of codes (row, 8c .. 8c+7) in the blocked layout: block
// (row / 32, k / 32) of 1 KB, inside it the 16-byte half (k % 32) / 16, then the
// row within the block, then k % 16.
__device__ __forceinline__ int64_t blocked_offset(int row, int c, int kb)
{
    return ((int64_t)(row >> 5) * kb + (c >> 2)) * 1024 + ((c >> 1) & 1) * 512 + (row & 31) * 16 +
           (c & 1) * 8;
}

// Byte offset of BF16 values (row, 8c .. 8c+7) in the BF16 blocked layout
// (include/ck.h): 2 KB per (row / 32, k / 32), inside it the MFMA step
// (k % 16) / 8, then the half (k % 32) / 16, the row within the block, k % 8.
__device__ __forceinline__ int64_t blocked_bf16_offset(int row, int c, int kb)
{
    return ((int64_t)(row >> 5) * kb + (c >> 2)) * 2048 + (c & 1) * 1024 + ((c >> 1) & 1) * 512 +
           (row & 31) * 16;
}

// What the kernel writes: INT8 codes and row scales, the unnormalised rotated
// row in FP32 (a diagnostic), or the normalised rotated row in BF16.
enum OutKind { OUT_CODES = 0, OUT_ROT_F32 = 1, OUT_ROT_BF16 = 2 };

// Staged blocked output: the LDS image of one 8-row group's codes.  In the
// blocked layout the 8 rows' 16-byte pieces of one (k / 32 block, k half)
// form one 128-byte line; the image keeps them in that order, 256 bytes per
// k-block plus 16 bytes of padding (so the code writes of lanes 4 apart,
// which are one k-block apart, fall in different banks).
constexpr int kStageKbBytes = 272;
// Largest k staged by quant_rows_kernel (its LDS image: 34,816 bytes) and by
// the SwiGLU table kernel (121,856 bytes beside the 37,128-byte table).
constexpr int kStageMaxK = 4096;
constexpr int kTabStageMaxK = 14336;

__device__ __forceinline__ int stage_offset(int r8, int c)
{
    return (c >> 2) * kStageKbBytes + ((c >> 1) & 1) * 128 + r8 * 16 + (c & 1) * 8;
}

// BS: threads per workgroup (256, or T for the wide teams of few-row calls).
// STAGE (blocked codes, 8 rows per workgroup, i.e. BS = 8 T, k <= kStageMaxK):
// the workgroup assembles its rows' codes in LDS and writes them as whole
// 128-byte lines, 16 bytes per lane; without it each
// lane writes 8 bytes into a line that seven other rows complete, and every
// store instruction touches 32 lines.  NT: those line writes are
// non-temporal.
template <int KIND, int LOG_G, int CH, int OUT, bool BLOCKED, int BS, bool STAGE = false, bool NT = false>
__global__ __launch_bounds__(BS) void quant_rows_kernel(
    const void* __restrict__ src, int64_t ld, int m, int k, int log_t, float cg,
    int8_t* __restrict__ q, float* __restrict__ s, void* __restrict__ u_out)
{
    static_assert(!STAGE || (BLOCKED && OUT == OUT_CODES), "staging is for blocked codes");
    constexpr int G = 1 << LOG_G;
    const int T = 1 << log_t;
    const int t = threadIdx.x & (T - 1);
    const int team = threadIdx.x >> log_t;
    const int rows_per_wg = blockDim.x >> log_t;
    int wg = blockIdx.x;
    if constexpr (BLOCKED) {
        // In the blocked layout a 128-byte line holds 16 code bytes of each of
        // 8 consecutive rows.  Workgroups are dispatched to the 8 XCDs round
        // robin (blockIdx % 8), each with its own L2, so the S workgroups
        // covering one 8-row set are taken from one XCD: the line then fills
        // in a single L2 instead of being written back piecewise from
        // several.  The grid is a multiple of 8 S, which makes this a
        // permutation of the workgroups.
        const int S = rows_per_wg >= 8 ? 1 : 8 / rows_per_wg;
        const int u = wg >> 3;
        wg = (u / S) * (8 * S) + (wg & 7) * S + (u % S);
    }
    if (wg * rows_per_wg >= m) return;      // a padding workgroup: no rows (uniform exit)
    int row = wg * rows_per_wg + team;
    const bool row_ok = row < m;
    if (!row_ok) row = m - 1;               // compute on a valid row, store nothing
    const int k8 = k >> 3;

    float v[CH][8];

    // ---- load + activation -------------------------------------------------
    if constexpr (KIND == IN_F32) {
        const float* rp = static_cast<const float*>(src) + (int64_t)row * ld;
        float4 raw[CH][2];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = j * T + t;
            if (c < k8) {
                raw[j][0] = *reinterpret_cast<const float4*>(rp + c * 8);
                raw[j][1] = *reinterpret_cast<const float4*>(rp + c * 8 + 4);
            } else {
                raw[j][0] = make_float4(0.f, 0.f, 0.f, 0.f);
                raw[j][1] = raw[j][0];
            }
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            v[j][0] = raw[j][0].x; v[j][1] = raw[j][0].y; v[j][2] = raw[j][0].z; v[j][3] = raw[j][0].w;
            v[j][4] = raw[j][1].x; v[j][5] = raw[j][1].y; v[j][6] = raw[j][1].z; v[j][7] = raw[j][1].w;
        }
    } else {
        const uint16_t* rp = static_cast<const uint16_t*>(src) + (int64_t)row * ld;
        uint4 rg[CH];
        uint4 ru[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = j * T + t;
            if (c < k8) {
                rg[j] = *reinterpret_cast<const uint4*>(rp + c * 8);
                if constexpr (KIND == IN_BF16_SWIGLU)
                    ru[j] = *reinterpret_cast<const uint4*>(rp + k + c * 8);
            } else {
                rg[j] = make_uint4(0u, 0u, 0u, 0u);
                ru[j] = rg[j];
            }
        }
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const uint32_t w[4] = {rg[j].x, rg[j].y, rg[j].z, rg[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[j][2 * e] = bf16_lo(w[e]);
                v[j][2 * e + 1] = bf16_hi(w[e]);
            }
            if constexpr (KIND == IN_BF16_SWIGLU) {
                const uint32_t wu[4] = {ru[j].x, ru[j].y, ru[j].z, ru[j].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[j][2 * e] = silu_f32(w[e] << 16) * bf16_lo(wu[e]);
                    v[j][2 * e + 1] = silu_f32(w[e] & 0xffff0000u) * bf16_hi(wu[e]);
                }
            }
        }
    }

    // ---- rotation (unnormalised blockwise FWHT) + absmax --------------------
    // From G = 32 the exchanges with the lanes 1, 2 (and, from G = 128, 8)
    // apart are fused into the butterfly and the values come out as sigma * u
    // (fwht_cross_lane_signed; sigma = +-1, fixed per lane): |.| gives the
    // absmax, and what the values are multiplied by below takes sigma.
    float amax = 0.0f, sigma = 1.0f;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        fwht_in_lane<G>(v[j]);
        if constexpr (G >= 32) sigma = fwht_cross_lane_signed<G>(v[j], t);
        else fwht_cross_lane<G>(v[j], t);
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
    }

    if constexpr (OUT == OUT_ROT_BF16) {
        // x_rot = bf16(fl(u * c_g) + 0): the rotation with the orthonormal H
        // (fl(sigma u * sigma c_g) = fl(u * c_g) up to the sign of a zero)
        char* ob = static_cast<char*>(u_out);
        const float cs = cg * sigma;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = j * T + t;
            const uint4 w = make_uint4(rot_bf16x2(v[j][0], v[j][1], cs), rot_bf16x2(v[j][2], v[j][3], cs),
                                       rot_bf16x2(v[j][4], v[j][5], cs), rot_bf16x2(v[j][6], v[j][7], cs));
            if (row_ok && c < k8) {
                const int64_t off = BLOCKED ? blocked_bf16_offset(row, c, k >> 5) : ((int64_t)row * k + c * 8) * 2;
                *reinterpret_cast<uint4*>(ob + off) = w;
            }
        }
        return;
    }
    if constexpr (OUT == OUT_ROT_F32) {
        float* up = static_cast<float*>(u_out) + (int64_t)row * k;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = j * T + t;
            if (row_ok && c < k8) {
                // + 0: an exact zero as +0, whatever sign the butterflies left it
                *reinterpret_cast<float4*>(up + c * 8) = make_float4(
                    v[j][0] * sigma + 0.0f, v[j][1] * sigma + 0.0f, v[j][2] * sigma + 0.0f, v[j][3] * sigma + 0.0f);
                *reinterpret_cast<float4*>(up + c * 8 + 4) = make_float4(
                    v[j][4] * sigma + 0.0f, v[j][5] * sigma + 0.0f, v[j][6] * sigma + 0.0f, v[j][7] * sigma + 0.0f);
            }
        }
        return;
    }

    // ---- team reduction of the absmax (exact; order does not matter) -------
    __shared__ float red[BS / 64];
    if (T >= 2) amax = fmaxf(amax, swizzle_xor<1>(amax));
    if (T >= 4) amax = fmaxf(amax, swizzle_xor<2>(amax));
    if (T >= 8) amax = fmaxf(amax, swizzle_xor<4>(amax));
    if (T >= 16) amax = fmaxf(amax, swizzle_xor<8>(amax));
    if (T >= 32) amax = fmaxf(amax, swizzle_xor<16>(amax));
    if (T >= 64) amax = fmaxf(amax, __shfl_xor(amax, 32));
    if (T > 64) {
        // one team spans T/64 waves of this workgroup
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) red[wave] = amax;
        __syncthreads();
        const int w0 = (team * T) >> 6;
        for (int w = 0; w < (T >> 6); ++w) amax = fmaxf(amax, red[w0 + w]);
    }

    // ---- scale and codes ----------------------------------------------------
    // s = fl(fl(A * c_g) / 127); r = fl(127 / A), or 0 for an all-zero row
    // (every code is then round(u * 0) = 0 and the scale is 0).
    const float scale = (amax * cg) / 127.0f;
    const float r = (amax > 0.0f ? 127.0f / amax : 0.0f) * sigma;
    int8_t* qp = q + (int64_t)row * k;
    __shared__ __align__(16) char stage[STAGE ? kStageMaxK / 32 * kStageKbBytes : 16];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int c = j * T + t;
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) b[i] = code_bits(v[j][i], r);
        const uint2 codes = make_uint2(pack4(b[0], b[1], b[2], b[3]), pack4(b[4], b[5], b[6], b[7]));
        if constexpr (STAGE) {
            if (c < k8) *reinterpret_cast<uint2*>(stage + stage_offset(team, c)) = codes;
        } else if (row_ok && c < k8) {
            if constexpr (BLOCKED)
                *reinterpret_cast<uint2*>(q + blocked_offset(row, c, k >> 5)) = codes;
            else
                *reinterpret_cast<uint2*>(qp + c * 8) = codes;
        }
    }
    if (row_ok && t == 0) s[row] = scale;
    if constexpr (STAGE) {
        // 16-byte unit u of the group: k-block u / 16, half (u / 8) % 2, row
        // u % 8; a wave writes 64 consecutive units, i.e. 8 whole lines
        __syncthreads();
        const int row0 = wg * 8;              // rows_per_wg == 8: one aligned 8-row group
        const int kb = k >> 5;
        int8_t* gq = q + ((int64_t)(row0 >> 5) * kb) * 1024 + ((row0 >> 3) & 3) * 128;
        typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
        for (int u = threadIdx.x; u < kb * 16; u += BS) {
            const int r8 = u & 7;
            if (row0 + r8 < m) {
                const u4_t w = *reinterpret_cast<const u4_t*>(stage + (u >> 4) * kStageKbBytes + (u & 15) * 16);
                u4_t* dst = reinterpret_cast<u4_t*>(gq + (int64_t)(u >> 4) * 1024 + ((u >> 3) & 1) * 512 + r8 * 16);
                if constexpr (NT) __builtin_nontemporal_store(w, dst);
                else *dst = w;
            }
        }
    }
}

// Blocked codes of many BF16 rows (g = 64, 128 or 256): a workgroup owns one
// aligned group of 8 rows, and its waves share the rows' Hadamard groups
// (wave w takes groups w, w + NW, ...).  In a wave, lane bits 2, 4 and 5 pick
// the row (r8) and lane bits 0, 1 and 3 the 8-element chunk j of a 64-element
// segment; a group is G / 64 such segments, one 16-byte load each.  So
//  - a load instruction reads 128 contiguous bytes of each of the 8 rows;
//  - the butterflies of element strides 8, 16 and 32 pair lanes 1, 2 and 8
//    apart, all three fused into DPP FMAs as in fwht_cross_lane_signed (the
//    values come out as sigma * u with the same sigma), and strides 64 and
//    128 pair the lane's own loads, after them (the order stays ascending);
//  - a store instruction's 8-byte codes per lane are 4 whole 128-byte lines of
//    the blocked layout (8 rows x 16 codes), with no staging through LDS.
// The code stores are non-temporal: measured after a MALL flush at
// 4096 x 3072 (kernel trace) the kernel takes 8.9 us with them and 10.2 us
// without; the per-row kernel 11.4 us, its staged form 10.1 us.  Outputs are
// those of quant_rows_kernel<IN_BF16, ..., OUT_CODES, true> bit for bit.
// (A SwiGLU form with the silu table of quant_swiglu_tab_kernel built per
// workgroup was slower than the per-row kernel at 2048 x 3072, 12.0 against
// 11.3 us: building the table costs each workgroup more than its 8 rows save.)
constexpr int kLinesMaxLoads = 8;          // 16-byte loads per lane (64 FP32 values)

template <int LOG_G, int GPW>
__global__ __launch_bounds__(1024) void quant_lines_kernel(const uint16_t* __restrict__ src, int64_t ld, int m,
                                                           int k, float cg, int8_t* __restrict__ q,
                                                           float* __restrict__ s)
{
    static_assert(LOG_G >= 6 && LOG_G <= 8, "groups of 64, 128 or 256");
    constexpr int G = 1 << LOG_G;
    constexpr int NLG = G / 64;              // the lane's loads per group
    static_assert(GPW * NLG <= kLinesMaxLoads, "load cap");
    typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
    const int nw = blockDim.x >> 6;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int j = (lane & 3) | ((lane >> 1) & 4);
    const int r8 = ((lane >> 2) & 1) | ((lane >> 3) & 6);
    int row = blockIdx.x * 8 + r8;
    const bool row_ok = row < m;
    if (!row_ok) row = m - 1;                // compute on a valid row, store nothing
    const int ngroups = k >> LOG_G;
    const uint16_t* rp = src + (int64_t)row * ld + 8 * j;

    uint4 raw[GPW][NLG];
#pragma unroll
    for (int p = 0; p < GPW; ++p) {
        const int gi = w + p * nw;
#pragma unroll
        for (int n = 0; n < NLG; ++n)
            raw[p][n] = gi < ngroups ? *reinterpret_cast<const uint4*>(rp + gi * G + n * 64)
                                     : make_uint4(0u, 0u, 0u, 0u);
    }

    const float t0 = (lane & 1) ? -1.0f : 1.0f;
    const float t1 = (lane & 2) ? -1.0f : 1.0f;
    const float t3 = (lane & 8) ? -1.0f : 1.0f;
    float v[GPW][NLG][8];
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < GPW; ++p) {
#pragma unroll
        for (int n = 0; n < NLG; ++n) {
            const uint32_t wd[4] = {raw[p][n].x, raw[p][n].y, raw[p][n].z, raw[p][n].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[p][n][2 * e] = bf16_lo(wd[e]);
                v[p][n][2 * e + 1] = bf16_hi(wd[e]);
            }
            fwht_in_lane<G>(v[p][n]);                // strides 1, 2, 4
            fmac_dpp8<0xB1>(v[p][n], t0);            // stride 8: lane ^ 1
            fmac_dpp8<0x4E>(v[p][n], t1);            // stride 16: lane ^ 2
            fmac_dpp8<0x128>(v[p][n], t3);           // stride 32: lane ^ 8
        }
#pragma unroll
        for (int h = 1; h < NLG; h <<= 1)            // strides 64, 128
#pragma unroll
            for (int n = 0; n < NLG; ++n)
                if ((n & h) == 0)
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float a = v[p][n][i], b = v[p][n + h][i];
                        v[p][n][i] = a + b;
                        v[p][n + h][i] = a - b;
                    }
#pragma unroll
        for (int n = 0; n < NLG; ++n)
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[p][n][i]));
    }
    const float sigma = t0 * t1 * t3;

    // row absmax: the row's 8 lanes of each wave (lane bits 0, 1, 3), then the waves
    __shared__ float red[16][8];
    amax = fmaxf(amax, dpp_xor<1>(amax));
    amax = fmaxf(amax, dpp_xor<2>(amax));
    amax = fmaxf(amax, swizzle_xor<8>(amax));
    if (j == 0) red[w][r8] = amax;
    __syncthreads();
    for (int i = 0; i < nw; ++i) amax = fmaxf(amax, red[i][r8]);

    // s = fl(fl(A * c_g) / 127); r = fl(127 / A), or 0 for an all-zero row
    const float scale = (amax * cg) / 127.0f;
    const float r = (amax > 0.0f ? 127.0f / amax : 0.0f) * sigma;
    const int kb = k >> 5;
#pragma unroll
    for (int p = 0; p < GPW; ++p) {
        const int gi = w + p * nw;
#pragma unroll
        for (int n = 0; n < NLG; ++n) {
            uint32_t b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) b[i] = code_bits(v[p][n][i], r);
            const u2_t codes = {pack4(b[0], b[1], b[2], b[3]), pack4(b[4], b[5], b[6], b[7])};
            if (row_ok && gi < ngroups) {
                const int c = ((gi * G + n * 64) >> 3) + j;
                __builtin_nontemporal_store(codes, reinterpret_cast<u2_t*>(q + blocked_offset(row, c, kb)));
            }
        }
    }
    if (row_ok && w == 0 && j == 0) s[row] = scale;
}

// The SwiGLU quantizer for large calls: persistent, one 1024-thread workgroup
// per CU (16 waves).  silu here is a lookup in a table of silu_sigma (ck_device.hpp,
// identical bits to silu_f32), which the workgroup builds in its LDS while the
// loads of its first rows are in flight; it then walks its rows, a team of T
// lanes per row as in quant_rows_kernel, with the next rows' loads issued
// before the current rows are rotated and quantized (two register buffers).
// The per-element work drops from ~43 to ~24 VALU instructions (measured on
// c5's shape, the table's construction included).  Outputs are those of
// quant_rows_kernel<IN_BF16_SWIGLU, ..., OUT_CODES> bit for bit.
//
// STAGE (blocked codes, k <= kTabStageMaxK): rows are taken in aligned groups
// of 8, last group first (group i of the workgroup is the (blockIdx + i *
// gridDim)-th from the end), each in 8 / rpw passes of rpw = 1024 / T rows; a
// group's codes are assembled in LDS (laid out as in quant_rows_kernel) and
// written as whole 128-byte lines after its last pass.  Last rows first: in
// the MLP the gate_up GEMM writes its rows in ascending bands just before, so
// the rows it wrote last are the likeliest still to sit in the MALL (c5's
// block, back to back, paired rounds on two boxes: 1.9 us per step faster in
// 9 of 10 on one, 0.4 us in 11 of 22 (one tie) on the other).
//
// Otherwise pass p of the workgroup takes rpw rows of row slot p * gridDim +
// (an XCD-grouped index of blockIdx): in each pass the
// workgroups together read one contiguous band of rows, and the workgroups
// of one XCD take consecutive slots, so the 8 rows that share a 128-byte line
// of unstaged blocked codes are written from one L2 (the grid is a multiple
// of 8, rpw divides 8, and an XCD's run of slots, gridDim / 8 * rpw rows, is
// a multiple of 8).  Measured on c5's shape (4096 x 12288, after a MALL
// flush): staged 56.4 us, the unstaged slot order 60.0 us, the group order
// without staging 78.5 us; with row-major codes the slot order is 1.4 us
// faster than the group order.
constexpr int kTabThreads = 1024;

template <int LOG_G, int CH, bool BLOCKED, bool STAGE>
__global__ __launch_bounds__(kTabThreads) void quant_swiglu_tab_kernel(
    const uint16_t* __restrict__ src, int64_t ld, int m, int k, int log_t, float cg, int8_t* __restrict__ q,
    float* __restrict__ s)
{
    static_assert(!STAGE || BLOCKED, "staging is for blocked codes");
    constexpr int G = 1 << LOG_G;
    __shared__ float tab[kSiluTabEntries];
    __shared__ float red[2][kTabThreads / 64];
    __shared__ __align__(16) char stage[STAGE ? kTabStageMaxK / 32 * kStageKbBytes : 16];
    const int T = 1 << log_t;
    const int t = threadIdx.x & (T - 1);
    const int team = threadIdx.x >> log_t;
    const int rpw = kTabThreads >> log_t;      // rows per workgroup pass: 1, 2, 4 or 8
    const int lppg = log_t - 7;                // log2 of the passes per 8-row group
    const int nwg = gridDim.x;
    const int k8 = k >> 3;
    const char* tb = reinterpret_cast<const char*>(tab) - kSiluTabBias;   // see silu_tab_offset
    // STAGE: first row of the 8-row group of pass p (uniform; past m when the
    // workgroup has no group left); the pass ends the group when its index
    // within the group is the last one
    const int ng8 = (m + 7) >> 3;
    auto group_row = [&](int p) {
        const int gi = blockIdx.x + (p >> lppg) * nwg;
        return gi < ng8 ? (ng8 - 1 - gi) * 8 : m + 8;
    };
    const int slot0 = ((blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3)) * rpw;
    // first row of pass p (uniform), and whether pass p has rows to do
    auto pass_row = [&](int p) {
        return STAGE ? group_row(p) + (p & ((1 << lppg) - 1)) * rpw : slot0 + p * nwg * rpw;
    };
    auto pass_live = [&](int p) { return (STAGE ? group_row(p) : pass_row(p)) < m; };
    if (!pass_live(0)) return;                 // uniform exit (no barrier reached)

    // Loads and stores go through buffer resources (the launcher keeps every
    // extent below 2^31 bytes): a lane with nothing to load or store uses an
    // offset past the end, which reads zeros or drops the store, so the code
    // has no branches and the compiler can count the loads in flight exactly.
    const __amdgpu_buffer_rsrc_t rs_x =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), (short)0, (int)((int64_t)m * ld * 2), 0x00020000);
    const int64_t qbytes = BLOCKED ? (int64_t)((m + 255) / 256 * 256) * k : (int64_t)m * k;
    const __amdgpu_buffer_rsrc_t rs_q = __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)qbytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_s = __builtin_amdgcn_make_buffer_rsrc(s, (short)0, m * 4, 0x00020000);
    typedef int v4i_t __attribute__((ext_vector_type(4)));
    typedef int v2i_t __attribute__((ext_vector_type(2)));

    // Gate / up chunks in two register buffers: pass p reads buffer p % 2
    // and, once its silu * up is formed, loads pass p + 2 into the same
    // buffer, so two passes of loads are always in flight.  Chunks past k8
    // and rows past m (also every row of a pass after the last) read as zeros
    // without a memory access, and nothing is stored for them.  The loads are
    // unconditional: under a branch the compiler copied every loaded register
    // once per pass.
    v4i_t gb[2][CH], ub[2][CH];
    auto load = [&](int h, int first) {
        const int row = first + team;
        const uint32_t rb = row < m ? (uint32_t)((int64_t)row * ld * 2) : kBufferOutside;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = j * T + t;
            const uint32_t og = c < k8 ? rb + (uint32_t)c * 16u : kBufferOutside;
            const uint32_t ou = c < k8 ? og + (uint32_t)k * 2u : kBufferOutside;
            gb[h][j] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, og, 0, 0);
            ub[h][j] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, ou, 0, 0);
        }
    };
    load(0, pass_row(0));
    load(1, pass_row(1));
    for (int i = threadIdx.x; i < kSiluTabEntries; i += kTabThreads) tab[i] = silu_tab_entry(i);
    __syncthreads();

    for (int p0 = 0;; p0 += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int pass = p0 + h;
            if (!pass_live(pass)) return;         // uniform; every started group has been written
            const int rp0 = pass_row(pass);       // this pass's first row (uniform)
            float v[CH][8];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const uint32_t wg[4] = {(uint32_t)gb[h][j][0], (uint32_t)gb[h][j][1], (uint32_t)gb[h][j][2],
                                        (uint32_t)gb[h][j][3]};
                const uint32_t wu[4] = {(uint32_t)ub[h][j][0], (uint32_t)ub[h][j][1], (uint32_t)ub[h][j][2],
                                        (uint32_t)ub[h][j][3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y0 = *reinterpret_cast<const float*>(tb + silu_tab_offset<false>(wg[e]));
                    const float y1 = *reinterpret_cast<const float*>(tb + silu_tab_offset<true>(wg[e]));
                    const float s0 = gate_clamp(wg[e] << 16) * y0;    // silu_f32, bit for bit
                    const float s1 = gate_clamp(wg[e] & 0xffff0000u) * y1;
                    v[j][2 * e] = s0 * bf16_lo(wu[e]);
                    v[j][2 * e + 1] = s1 * bf16_hi(wu[e]);
                }
            }
            load(h, pass_row(pass + 2));   // past the last pass: no memory access

            // the rotated values come out as sigma * u (fwht_cross_lane_signed),
            // sigma = +-1 fixed per lane: |.| gives the absmax, and the code
            // multiplier takes sigma
            float amax = 0.0f, sigma = 1.0f;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                fwht_in_lane<G>(v[j]);
                sigma = fwht_cross_lane_signed<G>(v[j], t);
#pragma unroll
                for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[j][i]));
            }
            // T >= 128 here (at most 8 rows per 1024-thread workgroup)
            amax = fmaxf(amax, dpp_xor<1>(amax));
            amax = fmaxf(amax, dpp_xor<2>(amax));
            amax = fmaxf(amax, swizzle_xor<4>(amax));
            amax = fmaxf(amax, swizzle_xor<8>(amax));
            amax = fmaxf(amax, swizzle_xor<16>(amax));
            amax = fmaxf(amax, __shfl_xor(amax, 32));
            {
                // the team spans T / 64 waves; red[h] alternates between passes,
                // so a wave writing the next pass's entry never meets a wave
                // still reading this one (every pass has this barrier, which
                // also orders the previous group's staged reads before this
                // pass's staged writes)
                const int wave = threadIdx.x >> 6;
                if ((threadIdx.x & 63) == 0) red[h][wave] = amax;
                __syncthreads();
                const int w0 = (team * T) >> 6;
                for (int w = 0; w < (T >> 6); ++w) amax = fmaxf(amax, red[h][w0 + w]);
            }

            const int row = rp0 + team;
            const bool row_ok = row < m;
            const float scale = (amax * cg) / 127.0f;
            const float r = (amax > 0.0f ? 127.0f / amax : 0.0f) * sigma;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int c = j * T + t;
                uint32_t bq[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) bq[i] = code_bits(v[j][i], r);
                const v2i_t codes = {(int)pack4(bq[0], bq[1], bq[2], bq[3]), (int)pack4(bq[4], bq[5], bq[6], bq[7])};
                if constexpr (STAGE) {
                    if (c < k8) *reinterpret_cast<v2i_t*>(stage + stage_offset(row & 7, c)) = codes;
                } else {
                    const int64_t off = BLOCKED ? blocked_offset(row, c, k >> 5) : (int64_t)row * k + c * 8;
                    const uint32_t oq = (row_ok && c < k8) ? (uint32_t)off : kBufferOutside;
                    __builtin_amdgcn_raw_buffer_store_b64(codes, rs_q, oq, 0, 0);
                }
            }
            const uint32_t os = (row_ok && t == 0) ? (uint32_t)row * 4u : kBufferOutside;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(scale), rs_s, os, 0, 0);

            if constexpr (STAGE) {
                if ((pass & ((1 << lppg) - 1)) == (1 << lppg) - 1) {   // the group's last pass (uniform)
                    // 16-byte unit u of the group: k-block u / 16, half
                    // (u / 8) % 2, row u % 8; a wave writes 8 whole lines
                    __syncthreads();
                    const int row0 = group_row(pass);
                    const int kb = k >> 5;
                    const uint32_t base = (uint32_t)((int64_t)(row0 >> 5) * kb * 1024) + ((row0 >> 3) & 3) * 128;
                    for (int u = threadIdx.x; u < kb * 16; u += kTabThreads) {
                        const int r8 = u & 7;
                        const v4i_t w =
                            *reinterpret_cast<const v4i_t*>(stage + (u >> 4) * kStageKbBytes + (u & 15) * 16);
                        const uint32_t off = row0 + r8 < m
                            ? base + (uint32_t)(u >> 4) * 1024u + (uint32_t)((u >> 3) & 1) * 512u + (uint32_t)r8 * 16u
                            : kBufferOutside;
                        __builtin_amdgcn_raw_buffer_store_b128(w, rs_q, off, 0, 0);
                    }
                }
            }
        }
    }
}

// The rotation to BF16 in the blocked layout, written as whole lines (x
// itself, or SWI: silu(gate) * up of [gate | up] rows, silu from the LDS
// table as in quant_swiglu_tab_kernel when TAB, else silu_f32 itself).  In
// that layout a 128-byte line holds the 16 bytes of one 8-column chunk of 8
// consecutive rows.  The row-wise
// kernels lay a row's chunks across a workgroup, so a line gathers its pieces
// from several workgroups at different times, and those partial lines cost
// more than the reads (the SwiGLU rotation of 4096 x 12288, after a MALL
// flush: 117 us blocked against 53 us row-major).  Here a wave holds
// RW = 64 / (g / 8) consecutive rows of one rotation group, one lane per
// chunk, so a store writes RW * 16 contiguous bytes of each line it touches,
// and the waves holding the other rows of the 8-row block write the rest of
// those lines with the same instruction.  Unit of work: an aligned block of 8
// rows times a slice of CH * SLOTS consecutive groups; workgroup b takes
// units b + i * gridDim, with the loads of two units in flight.
template <int LOG_G, int CH, bool SWI, bool TAB>
__global__ __launch_bounds__(kTabThreads) void rotate_lines_kernel(const uint16_t* __restrict__ src, int64_t ld,
                                                                   int m, int k, int nsl, float cg,
                                                                   uint16_t* __restrict__ out)
{
    constexpr int G = 1 << LOG_G;
    constexpr int LGL = LOG_G - 3;                    // log2 of a group's lanes
    constexpr int RW = 64 >> LGL;                     // rows per wave
    constexpr int WPB = 8 / RW;                       // waves per 8-row block and group slot
    constexpr int SLOTS = kTabThreads / 64 / WPB;     // group slots of a workgroup
    constexpr int NSG = CH * SLOTS;                   // groups per unit
    static_assert(SWI || !TAB, "the table is silu's");
    __shared__ float tab[TAB ? kSiluTabEntries : 1];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int gpos = lane & ((1 << LGL) - 1);         // chunk within the group
    const int r8 = (wave % WPB) * RW + (lane >> LGL); // row within the 8-row block
    const int slot = wave / WPB;
    const int ng = k >> LOG_G;
    const int units = ((m + 7) >> 3) * nsl;
    const int nwg = gridDim.x;
    if ((int)blockIdx.x >= units) return;             // uniform exit (no barrier reached)
    const char* tb = reinterpret_cast<const char*>(tab) - kSiluTabBias;   // see silu_tab_offset

    // buffer resources as in quant_swiglu_tab_kernel: past-the-end offsets
    // read zeros and drop stores (the launcher keeps both extents below 2^31)
    const __amdgpu_buffer_rsrc_t rs_x =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(src), (short)0, (int)((int64_t)m * ld * 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_o = __builtin_amdgcn_make_buffer_rsrc(
        out, (short)0, (int)((int64_t)((m + 255) / 256 * 256) * k * 2), 0x00020000);
    typedef int v4i_t __attribute__((ext_vector_type(4)));

    v4i_t gb[2][CH], ub[2][SWI ? CH : 1];
    auto load = [&](int h, int u) {   // u >= units: no memory access
        const int row = u < units ? (u / nsl) * 8 + r8 : m;
        const int g0 = (u % nsl) * NSG + slot;
        const uint32_t rb = row < m ? (uint32_t)((int64_t)row * ld * 2) : kBufferOutside;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int gi = g0 + j * SLOTS;
            const uint32_t og = gi < ng ? rb + (uint32_t)((gi << LGL) + gpos) * 16u : kBufferOutside;
            gb[h][j] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, og, 0, 0);
            if constexpr (SWI)
                ub[h][j] = __builtin_amdgcn_raw_buffer_load_b128(rs_x, gi < ng ? og + (uint32_t)k * 2u : kBufferOutside,
                                                                 0, 0);
        }
    };
    load(0, blockIdx.x);
    load(1, blockIdx.x + nwg);
    if constexpr (TAB) {
        for (int i = threadIdx.x; i < kSiluTabEntries; i += kTabThreads) tab[i] = silu_tab_entry(i);
        __syncthreads();
    }

    for (int i0 = 0;; i0 += 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int u = blockIdx.x + (i0 + h) * nwg;
            if (u >= units) return;                   // uniform
            const int row = (u / nsl) * 8 + r8;
            const int g0 = (u % nsl) * NSG + slot;
            float v[CH][8];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const uint32_t wg[4] = {(uint32_t)gb[h][j][0], (uint32_t)gb[h][j][1], (uint32_t)gb[h][j][2],
                                        (uint32_t)gb[h][j][3]};
                if constexpr (SWI) {
                    const uint32_t wu[4] = {(uint32_t)ub[h][j][0], (uint32_t)ub[h][j][1], (uint32_t)ub[h][j][2],
                                            (uint32_t)ub[h][j][3]};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float s0, s1;
                        if constexpr (TAB) {
                            const float y0 = *reinterpret_cast<const float*>(tb + silu_tab_offset<false>(wg[e]));
                            const float y1 = *reinterpret_cast<const float*>(tb + silu_tab_offset<true>(wg[e]));
                            s0 = gate_clamp(wg[e] << 16) * y0;    // silu_f32, bit for bit
                            s1 = gate_clamp(wg[e] & 0xffff0000u) * y1;
                        } else {
                            s0 = silu_f32(wg[e] << 16);
                            s1 = silu_f32(wg[e] & 0xffff0000u);
                        }
                        v[j][2 * e] = s0 * bf16_lo(wu[e]);
                        v[j][2 * e + 1] = s1 * bf16_hi(wu[e]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[j][2 * e] = bf16_lo(wg[e]);
                        v[j][2 * e + 1] = bf16_hi(wg[e]);
                    }
                }
            }
            load(h, u + 2 * nwg);

            // x_rot = bf16(fl(sigma u * sigma c_g) + 0) = bf16(fl(u * c_g) + 0)
            float sigma = 1.0f;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                fwht_in_lane<G>(v[j]);
                sigma = fwht_cross_lane_signed<G>(v[j], gpos);
            }
            const float cs = cg * sigma;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const int gi = g0 + j * SLOTS;
                const int c = (gi << LGL) + gpos;
                const v4i_t w = {(int)rot_bf16x2(v[j][0], v[j][1], cs), (int)rot_bf16x2(v[j][2], v[j][3], cs),
                                 (int)rot_bf16x2(v[j][4], v[j][5], cs), (int)rot_bf16x2(v[j][6], v[j][7], cs)};
                const uint32_t oo =
                    (row < m && gi < ng) ? (uint32_t)blocked_bf16_offset(row, c, k >> 5) : kBufferOutside;
                __builtin_amdgcn_raw_buffer_store_b128(w, rs_o, oo, 0, 0);
            }
        }
    }
}

// Row-major [n, k] int8 -> blocked layout with rows padded to n_rows (zeros).
// One thread per 16-byte unit of the output, written in order.
__global__ __launch_bounds__(256) void pack_blocked_kernel(const int8_t* __restrict__ w, int n, int k,
                                                           int64_t units, int8_t* __restrict__ out)
{
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= units) return;
    const int kb = k >> 5;
    const int64_t block = u >> 6;
    const int l = (int)(u & 63);
    const int row = (int)(block / kb) * 32 + (l & 31);
    const int kbyte = (int)(block % kb) * 32 + (l >> 5) * 16;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (row < n) v = *reinterpret_cast<const uint4*>(w + (int64_t)row * k + kbyte);
    *reinterpret_cast<uint4*>(out + u * 16) = v;
}

// Row-major codes + row scales -> decode layout (include/ck.h): one thread
// per 16-byte unit of the output, written in order.  Group b of 16 rows has
// 4 header units (the 16 scales) then k units: unit 4 + v holds
// W[16 b + v % 16][64 (v / 64) + 16 ((v / 16) % 4) .. + 16].
__global__ __launch_bounds__(256) void pack_decode_kernel(const int8_t* __restrict__ w,
                                                          const float* __restrict__ sw, int k,
                                                          int64_t units, uint4* __restrict__ out)
{
    const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (u >= units) return;
    const int64_t per = 4 + (int64_t)k;       // units per 16-row group
    const int64_t b = u / per;
    const int v = (int)(u - b * per);
    uint4 o;
    if (v < 4) {
        o = *reinterpret_cast<const uint4*>(sw + b * 16 + v * 4);
    } else {
        const int t = v - 4;
        const int r = t & 15, q = (t >> 4) & 3, c = t >> 6;
        o = *reinterpret_cast<const uint4*>(w + (b * 16 + r) * (int64_t)k + c * 64 + q * 16);
    }
    out[u] = o;
}

__global__ __launch_bounds__(256) void silu_kernel(const uint16_t* __restrict__ g, int64_t n,
                                                   float* __restrict__ out)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) out[i] = silu_f32((uint32_t)g[i] << 16);
}

// ---------------------------------------------------------------------------
// Host side: team shape and template dispatch
// ---------------------------------------------------------------------------
namespace {

constexpr int kChOptions[] = {1, 2, 3, 4, 6, 8, 12, 16};

// Choose (log2 T, CH) with T*CH >= k/8, T a power of two in [max(8, G/8), 256].
// Prefer no idle chunk slots, then the widest team (more lanes in flight per
// row; measured at k = 3072: T = 128 beats T = 64 and T = 32, and at k = 12288
// T = 256 beats T = 128), then CH near 6.
// Few rows (fewer than the CUs): the row's latency is the call's, so teams go
// up to 1024 lanes (one workgroup per row) and the fewest chunks per lane win,
// then the fewest idle slots.
constexpr int kFewRows = 256;

bool choose_team(int k, int g, bool few, int* log_t, int* ch)
{
    const int k8 = k / 8;
    const int tmin = g / 8 > 8 ? g / 8 : 8;
    long best = -1;
    for (int lt = 3; lt <= (few ? 10 : 8); ++lt) {
        const int T = 1 << lt;
        if (T < tmin) continue;
        for (int c : kChOptions) {
            if ((long)T * c < k8) continue;
            if (T > 256 && c > 4) continue;
            const long waste = (long)T * c - k8;
            const long score = few ? (long)c * 100000000L + waste * 16 + lt
                                   : waste * 1000 + (8 - lt) * 20 + (c > 6 ? c - 6 : 6 - c);
            if (best < 0 || score < best) {
                best = score;
                *log_t = lt;
                *ch = c;
            }
        }
    }
    return best >= 0;
}

template <int KIND, int LOG_G, int OUT, bool BLOCKED>
hipError_t launch_ch(int ch, dim3 grid, hipStream_t st, const void* src, int64_t ld, int m, int k,
                     int log_t, float cg, int8_t* q, float* s, void* u)
{
    const int bs = log_t > 8 ? 1 << log_t : 256;
#define CK_CASE(C, BS_)                                                                           \
    case C:                                                                                       \
        hipLaunchKernelGGL((quant_rows_kernel<KIND, LOG_G, C, OUT, BLOCKED, BS_>), grid, dim3(BS_), 0, \
                           st, src, ld, m, k, log_t, cg, q, s, u);                                \
        break;
    if (bs == 256) {
        switch (ch) {
            CK_CASE(1, 256) CK_CASE(2, 256) CK_CASE(3, 256) CK_CASE(4, 256) CK_CASE(6, 256)
            CK_CASE(8, 256) CK_CASE(12, 256) CK_CASE(16, 256)
            default: return hipErrorInvalidValue;
        }
    } else if (bs == 512) {
        switch (ch) {
            CK_CASE(1, 512) CK_CASE(2, 512) CK_CASE(3, 512) CK_CASE(4, 512)
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (ch) {
            CK_CASE(1, 1024) CK_CASE(2, 1024) CK_CASE(3, 1024) CK_CASE(4, 1024)
            default: return hipErrorInvalidValue;
        }
    }
#undef CK_CASE
    return hipGetLastError();
}

// Staged blocked codes (see quant_rows_kernel): teams of 128 lanes with up to
// 4 chunks each, 8 rows per 1024-thread workgroup, g in {64, 128, 256}.
// Measured after a MALL flush against the unstaged kernel: faster from
// m * k = 2^24 (4096 x 4096: 14.3 -> 11.7 us; 16384 x 3072: 36.5 -> 28.3 us),
// slower below it (4096 x 3072: 9.3 -> 9.7 us), and slower with 8 chunks
// per lane (4096 x 8192, whose registers allow 4 waves per SIMD).  The BF16
// kernel's line writes are non-temporal at m * k = 2^24 (4096 x 4096: 12.8
// -> 11.8 us, 8192 x 2048: 13.4 -> 13.0 us, events around single calls) and
// plain above it (8192 x 4096: 21.3 against 22.6 us, 16384 x 3072: 28.7
// against 29.6 us).
bool use_stage(int kind, int64_t m, int64_t k, int g)
{
    return (kind == IN_BF16 || kind == IN_BF16_SWIGLU) && k <= kStageMaxK && m * k >= ((int64_t)1 << 24) &&
           (g == 64 || g == 128 || g == 256);
}

template <int KIND, int LOG_G, bool NT>
hipError_t launch_stage_ch(int ch, dim3 grid, hipStream_t st, const void* src, int64_t ld, int m, int k,
                           float cg, int8_t* q, float* s)
{
#define CK_STAGE(C)                                                                                          \
    case C:                                                                                                  \
        hipLaunchKernelGGL((quant_rows_kernel<KIND, LOG_G, C, OUT_CODES, true, 1024, true, NT>), grid, dim3(1024), \
                           0, st, src, ld, m, k, 7, cg, q, s, nullptr);                                      \
        break;
    switch (ch) {
        CK_STAGE(1) CK_STAGE(2) CK_STAGE(3) CK_STAGE(4)
        default: return hipErrorInvalidValue;
    }
#undef CK_STAGE
    return hipGetLastError();
}

hipError_t launch_stage(int kind, const void* src, int64_t ld, int64_t m, int64_t k, int g, int8_t* q, float* s,
                        hipStream_t st)
{
    const int64_t k8 = k / 8;
    int ch = 0;
    for (int c : {1, 2, 3, 4})
        if (ch == 0 && 128 * c >= k8) ch = c;
    if (ch == 0) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((m + 63) / 64 * 8));   // 8 rows per workgroup, a multiple of 8 workgroups
    const float cg = (float)(1.0 / sqrt((double)g));
    const bool nt = kind == IN_BF16 && m * k <= ((int64_t)1 << 24);
#define CK_STAGE_G(KD, L, GV, NT)                   \
    if (kind == KD && g == GV && nt == NT)          \
        return launch_stage_ch<KD, L, NT>(ch, grid, st, src, ld, (int)m, (int)k, cg, q, s);
    CK_STAGE_G(IN_BF16, 6, 64, false) CK_STAGE_G(IN_BF16, 7, 128, false) CK_STAGE_G(IN_BF16, 8, 256, false)
    CK_STAGE_G(IN_BF16, 6, 64, true) CK_STAGE_G(IN_BF16, 7, 128, true) CK_STAGE_G(IN_BF16, 8, 256, true)
    CK_STAGE_G(IN_BF16_SWIGLU, 6, 64, false) CK_STAGE_G(IN_BF16_SWIGLU, 7, 128, false)
    CK_STAGE_G(IN_BF16_SWIGLU, 8, 256, false)
#undef CK_STAGE_G
    return hipErrorInvalidValue;
}

// quant_lines_kernel's shape for a row of k: the most waves (16, 12, 8, 4)
// that divide the row's groups evenly within the load cap (with idle group
// slots the workgroup waits for its busiest waves: 2560 x 5120 took 16.0 us
// against 12.7 on the per-row kernel).  Measured after a MALL flush (4096
// rows, g 128): k = 3072 with 12 waves 9.8 us, 16 waves 10.1, 8 waves 10.4;
// k = 4096 with 16 waves 12.4, 12 waves 13.6, 8 waves 14.4.
bool lines_plan(int64_t k, int g, int* nw, int* gpw)
{
    const int64_t ng = k / g, nlg = g / 64;
    for (int w : {16, 12, 8, 4})
        if (ng % w == 0 && ng / w * nlg <= kLinesMaxLoads) {
            *nw = w;
            *gpw = (int)(ng / w);
            return true;
        }
    return false;
}

// The line kernel for blocked BF16 codes of at least 8 rows per CU (one
// workgroup per 8 rows: below that it leaves CUs idle, and the per-row kernel
// is faster, e.g. 1024 x 4096: 6.0 against 7.0 us), k >= 1024 (fewer groups
// than waves otherwise), outside the staged kernel's domain (k <= 4096 and
// m * k >= 2^24: there the two are within a few percent, the staged one ahead
// at 4096 x 4096, 11.8 against 12.3 us).  Measured after a MALL flush
// (events around single calls) against the kernels it replaces: 4096 x 3072
// 12.2 -> 10.0 us, 2048 x 3072 7.4 -> 6.9, 4096 x 2048 9.8 -> 7.0, 4096 x
// 1024 5.8 -> 5.2, 4096 x 8192 28.6 -> 25.6.
bool use_lines(int kind, int64_t m, int64_t k, int g)
{
    int nw, gpw;
    const bool staged = k <= kStageMaxK && m * k >= ((int64_t)1 << 24);
    return kind == IN_BF16 && (g == 64 || g == 128 || g == 256) && k % g == 0 && k >= 1024 && !staged &&
           m >= 8 * (int64_t)num_cus() && lines_plan(k, g, &nw, &gpw);
}

hipError_t launch_lines(const void* src, int64_t ld, int64_t m, int64_t k, int g, int8_t* q, float* s,
                        hipStream_t st)
{
    int nw = 0, gpw = 0;
    if (!lines_plan(k, g, &nw, &gpw)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((m + 7) / 8)), block((unsigned)(nw * 64));
    const float cg = (float)(1.0 / sqrt((double)g));
    const uint16_t* x = static_cast<const uint16_t*>(src);
#define CK_LINES(L, P)                                                                                      \
    if (g == (1 << L) && gpw == P) {                                                                        \
        hipLaunchKernelGGL((quant_lines_kernel<L, P>), grid, block, 0, st, x, ld, (int)m, (int)k, cg, q, s); \
        return hipGetLastError();                                                                           \
    }
    CK_LINES(6, 1) CK_LINES(6, 2) CK_LINES(6, 3) CK_LINES(6, 4) CK_LINES(6, 5) CK_LINES(6, 6) CK_LINES(6, 7)
    CK_LINES(6, 8) CK_LINES(7, 1) CK_LINES(7, 2) CK_LINES(7, 3) CK_LINES(7, 4) CK_LINES(8, 1) CK_LINES(8, 2)
#undef CK_LINES
    return hipErrorInvalidValue;
}

template <int KIND, int OUT, bool BLOCKED>
hipError_t launch_g(int log_g, int ch, dim3 grid, hipStream_t st, const void* src, int64_t ld, int m,
                    int k, int log_t, float cg, int8_t* q, float* s, void* u)
{
    switch (log_g) {
#define CK_G(L) \
    case L: return launch_ch<KIND, L, OUT, BLOCKED>(ch, grid, st, src, ld, m, k, log_t, cg, q, s, u);
        CK_G(0) CK_G(1) CK_G(2) CK_G(3) CK_G(4) CK_G(5) CK_G(6) CK_G(7) CK_G(8)
#undef CK_G
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

namespace {

struct Launch {
    dim3 grid;
    int log_t, ch, log_g, m, k;
    float cg;
};

bool plan(int64_t m, int64_t k, int g, bool blocked, Launch* p)
{
    if (!choose_team((int)k, g, m < kFewRows, &p->log_t, &p->ch)) return false;
    const int rows_per_wg = p->log_t > 8 ? 1 : 256 >> p->log_t;
    int64_t wgs = (m + rows_per_wg - 1) / rows_per_wg;
    if (blocked) {
        // a multiple of 8 S workgroups (see the row mapping in the kernel)
        const int64_t mult = 8 * (rows_per_wg >= 8 ? 1 : 8 / rows_per_wg);
        wgs = (wgs + mult - 1) / mult * mult;
    }
    p->grid = dim3((unsigned)wgs);
    p->log_g = 0;
    while ((1 << p->log_g) < g) ++p->log_g;
    p->cg = (float)(1.0 / sqrt((double)g));
    p->m = (int)m;
    p->k = (int)k;
    return true;
}

}  // namespace

namespace {

// The table kernel pays for its table (~9K silu_sigma evaluations per CU)
// once per launch, so it takes calls with enough elements per CU.
// Team of the table kernel: T lanes (a power of two, 128..1024) times CH <= 3
// chunks covering the row's k / 8 chunks with the fewest idle slots, then
// the fewest chunks per lane (16 waves of at most 128 VGPRs each), except
// that a one-row pass (T = 1024, CH = 1) gives way to two rows of two chunks
// per lane: 8 values per lane and pass leave the pass's barrier and absmax
// reduction too little to hide behind (after a MALL flush: 3072 x 8192
// 34.6 -> 30.7 us, 4096 x 8192 38.3 -> 35.7; at k = 4096, T = 512 with one
// chunk stays ahead of T = 256 with two, 19.9 against 20.6 us).
bool tab_team(int64_t k, int* log_t, int* ch)
{
    const int64_t k8 = k / 8;
    int64_t best = -1;
    for (int lt = 7; lt <= 10; ++lt) {
        for (int c = 1; c <= 3; ++c) {
            const int64_t slots = ((int64_t)1 << lt) * c;
            if (slots < k8) continue;
            const int64_t score = (slots - k8) * 4 + c + (lt == 10 && c == 1 ? 2 : 0);
            if (best < 0 || score < best) {
                best = score;
                *log_t = lt;
                *ch = c;
            }
        }
    }
    return best >= 0;
}

// The table kernel from m * k = 2^24 (m >= 512), and from 2^23 with at least 8
// rows per CU: each workgroup builds the 37 KB table once, which its rows must
// repay.  Measured after a MALL flush (events around single calls, one box)
// against the per-row kernel: 4096 x 2048 13.7 -> 13.0 us, 2048 x 4096 13.1 ->
// 12.8, 3072 x 4096 20.4 -> 18.9; at 2048 x 3072 the two are within the
// box-to-box spread (11.0 against 11.3 us on one box, 12.0 against 11.4 on
// another), and with fewer rows per CU the per-row kernel is ahead (1024 x 3072
// 7.8 against 9.4, 512 x 12288 12.5 against 20.3 us).
bool swiglu_tab_pays(int64_t m, int64_t k)
{
    const bool big = m >= 512 && m * k >= ((int64_t)1 << 24);
    const bool many_rows = m >= 8 * (int64_t)num_cus() && m * k >= ((int64_t)1 << 23);
    return k >= 1024 && (big || many_rows);
}

// The table quantizer also needs a team for the row: k <= 24576 (at most
// 1024 lanes of 3 chunks); longer rows take the per-row kernel.
bool use_swiglu_tab(int64_t m, int64_t k, int64_t ld, int g)
{
    const bool gs = g == 64 || g == 128 || g == 256;
    const bool fits = m * ld * 2 < ((int64_t)1 << 31) && (m + 255) / 256 * 256 * k < ((int64_t)1 << 31);
    int log_t = 0, ch = 0;
    return gs && fits && swiglu_tab_pays(m, k) && tab_team(k, &log_t, &ch);
}

template <int LOG_G, bool BLOCKED, bool STAGE>
hipError_t launch_tab_ch(int ch, dim3 grid, hipStream_t st, const uint16_t* src, int64_t ld, int m, int k,
                         int log_t, float cg, int8_t* q, float* s)
{
#define CK_TAB(C)                                                                                               \
    case C:                                                                                                     \
        hipLaunchKernelGGL((quant_swiglu_tab_kernel<LOG_G, C, BLOCKED, STAGE>), grid, dim3(kTabThreads), 0,      \
                           st, src, ld, m, k, log_t, cg, q, s);                                                 \
        break;
    switch (ch) {
        CK_TAB(1) CK_TAB(2) CK_TAB(3)
        default: return hipErrorInvalidValue;
    }
#undef CK_TAB
    return hipGetLastError();
}

hipError_t launch_swiglu_tab(const uint16_t* src, int64_t ld, int64_t m, int64_t k, int g, int8_t* q, float* s,
                             bool blocked, hipStream_t st)
{
    int log_t = 0, ch = 0;
    if (!tab_team(k, &log_t, &ch)) return hipErrorInvalidValue;
    const bool stage = blocked && k <= kTabStageMaxK;
    const int rpw = kTabThreads >> log_t;
    // staged: aligned groups of 8 rows; otherwise row slots of rpw rows, and
    // a multiple of 8 workgroups (see the slot order in the kernel)
    int64_t wgs = std::min<int64_t>(stage ? (m + 7) / 8 : (m + rpw - 1) / rpw, num_cus());
    if (!stage) wgs = (wgs + 7) / 8 * 8;
    const dim3 grid((unsigned)wgs);
    const float cg = (float)(1.0 / sqrt((double)g));
    const int lg = g == 64 ? 6 : g == 128 ? 7 : 8;
#define CK_TAB_ARGS ch, grid, st, src, ld, (int)m, (int)k, log_t, cg, q, s
#define CK_TAB_G(L)                                                                            \
    if (lg == L) {                                                                             \
        return stage     ? launch_tab_ch<L, true, true>(CK_TAB_ARGS)                           \
               : blocked ? launch_tab_ch<L, true, false>(CK_TAB_ARGS)                          \
                         : launch_tab_ch<L, false, false>(CK_TAB_ARGS);                        \
    }
    CK_TAB_G(6) CK_TAB_G(7) CK_TAB_G(8)
#undef CK_TAB_G
#undef CK_TAB_ARGS
    return hipErrorInvalidValue;
}

// Which line rotation (blocked BF16 output) a call takes: 0 none, 1 x, 2
// SwiGLU with the silu table, 3 SwiGLU with silu_f32 itself.  x from m * k =
// 2^20 with at least 512 rows; SwiGLU with the table at the sizes where the
// table kernel takes the codes (the table must be repaid as there), else from
// m * k = 2^22 with at least 1024 rows.  Measured after a MALL flush against the row-wise
// kernel: x 4096 x 3072 16.6 -> 12.7 us, 2048 x 4096 11.2 -> 8.3, 1024 x 1024
// 4.8 -> 4.6; SwiGLU 4096 x 12288 94.0 -> 56.0 (the table's 56.2 against 59.3
// without it), 2048 x 8192 31.4 -> 21.6; without the table 2048 x 3072
// 11.4 -> 10.8, 1024 x 12288 21.2 -> 18.9.  With fewer rows the units are too
// few for the CUs (x 256 x 4096: 5.8 against 4.6 us; SwiGLU 1024 x 3072: 8.4
// against 8.0).
int rotate_lines_mode(int kind, int64_t m, int64_t k, int64_t ld, int g)
{
    const bool gs = g == 64 || g == 128 || g == 256;
    const bool fits = m * ld * 2 < ((int64_t)1 << 31) && (m + 255) / 256 * 256 * k * 2 < ((int64_t)1 << 31);
    if (!gs || !fits) return 0;
    if (kind == IN_BF16) return m >= 512 && m * k >= ((int64_t)1 << 20) ? 1 : 0;
    if (kind != IN_BF16_SWIGLU) return 0;
    if (swiglu_tab_pays(m, k)) return 2;
    return m >= 1024 && m * k >= ((int64_t)1 << 22) ? 3 : 0;
}

// Groups per lane and unit: the fewest idle group slots over a row's slices,
// then the most groups per unit (at most 3 with SwiGLU, whose two inputs
// double the registers in flight, else 4).
// mode as rotate_lines_mode (1, 2 or 3)
hipError_t launch_rotate_lines(int mode, const uint16_t* src, int64_t ld, int64_t m, int64_t k, int g,
                               uint16_t* out, hipStream_t st)
{
    const bool swi = mode >= 2;
    const int lg = g == 64 ? 6 : g == 128 ? 7 : 8;
    const int slots = 16 / (8 / (64 >> (lg - 3)));
    const int64_t ng = k / g;
    int ch = 0;
    int64_t nsl = 0, best = -1;
    for (int c = swi ? 3 : 4; c >= 1; --c) {
        const int64_t n = (ng + (int64_t)c * slots - 1) / ((int64_t)c * slots);
        const int64_t idle = n * c * slots - ng;
        if (best < 0 || idle < best) {
            best = idle;
            ch = c;
            nsl = n;
        }
    }
    const int64_t units = (m + 7) / 8 * nsl;
    const dim3 grid((unsigned)std::min<int64_t>(units, num_cus()));
    const float cg = (float)(1.0 / sqrt((double)g));
#define CK_RL(L, C, MODE)                                                                                \
    if (lg == L && ch == C && mode == MODE) {                                                            \
        hipLaunchKernelGGL((rotate_lines_kernel<L, C, (MODE >= 2), (MODE == 2)>), grid, dim3(kTabThreads), 0, st, \
                           src, ld, (int)m, (int)k, (int)nsl, cg, out);                                  \
        return hipGetLastError();                                                                        \
    }
#define CK_RL_G(L) CK_RL(L, 1, 1) CK_RL(L, 2, 1) CK_RL(L, 3, 1) CK_RL(L, 4, 1) \
    CK_RL(L, 1, 2) CK_RL(L, 2, 2) CK_RL(L, 3, 2) CK_RL(L, 1, 3) CK_RL(L, 2, 3) CK_RL(L, 3, 3)
    CK_RL_G(6) CK_RL_G(7) CK_RL_G(8)
#undef CK_RL_G
#undef CK_RL
    return hipErrorInvalidValue;
}

}  // namespace

// kind: 0 = BF16, 1 = BF16 [gate | up] with SwiGLU, 2 = FP32 (weights).
hipError_t launch_quant_rows(int kind, const void* src, int64_t ld, int64_t m, int64_t k, int g,
                             int8_t* q, float* s, float* u_out, bool blocked, hipStream_t st)
{
    if (m == 0) return hipSuccess;
    Launch p;
    if (!plan(m, k, g, blocked && u_out == nullptr, &p)) return hipErrorInvalidValue;
#define CK_ARGS p.log_g, p.ch, p.grid, st, src, ld, p.m, p.k, p.log_t, p.cg
    if (u_out != nullptr) {
        if (kind == IN_BF16) return launch_g<IN_BF16, OUT_ROT_F32, false>(CK_ARGS, q, s, u_out);
        if (kind == IN_BF16_SWIGLU) return launch_g<IN_BF16_SWIGLU, OUT_ROT_F32, false>(CK_ARGS, q, s, u_out);
        return hipErrorInvalidValue;
    }
    if (kind == IN_BF16_SWIGLU && use_swiglu_tab(m, k, ld, g))
        return launch_swiglu_tab(static_cast<const uint16_t*>(src), ld, m, k, g, q, s, blocked, st);
    if (blocked && use_lines(kind, m, k, g)) return launch_lines(src, ld, m, k, g, q, s, st);
    if (blocked && use_stage(kind, m, k, g)) return launch_stage(kind, src, ld, m, k, g, q, s, st);
    switch (kind * 2 + (blocked ? 1 : 0)) {
        case 0: return launch_g<IN_BF16, OUT_CODES, false>(CK_ARGS, q, s, nullptr);
        case 1: return launch_g<IN_BF16, OUT_CODES, true>(CK_ARGS, q, s, nullptr);
        case 2: return launch_g<IN_BF16_SWIGLU, OUT_CODES, false>(CK_ARGS, q, s, nullptr);
        case 3: return launch_g<IN_BF16_SWIGLU, OUT_CODES, true>(CK_ARGS, q, s, nullptr);
        case 4: return launch_g<IN_F32, OUT_CODES, false>(CK_ARGS, q, s, nullptr);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_rotate_bf16(int kind, const void* src, int64_t ld, int64_t m, int64_t k, int g,
                              uint16_t* out, bool blocked, hipStream_t st)
{
    if (m == 0) return hipSuccess;
    Launch p;
    if (!plan(m, k, g, blocked, &p)) return hipErrorInvalidValue;
    // row-major output: the row-wise kernel writes whole rows (the table
    // kernel's rows took as long: 4096 x 12288 SwiGLU 51.9 against 49.8 us)
    const int lines = blocked ? rotate_lines_mode(kind, m, k, ld, g) : 0;
    if (lines) return launch_rotate_lines(lines, static_cast<const uint16_t*>(src), ld, m, k, g, out, st);
    switch (kind * 2 + (blocked ? 1 : 0)) {
        case 0: return launch_g<IN_BF16, OUT_ROT_BF16, false>(CK_ARGS, nullptr, nullptr, out);
        case 1: return launch_g<IN_BF16, OUT_ROT_BF16, true>(CK_ARGS, nullptr, nullptr, out);
        case 2: return launch_g<IN_BF16_SWIGLU, OUT_ROT_BF16, false>(CK_ARGS, nullptr, nullptr, out);
        case 3: return launch_g<IN_BF16_SWIGLU, OUT_ROT_BF16, true>(CK_ARGS, nullptr, nullptr, out);
        default: return hipErrorInvalidValue;
    }
#undef CK_ARGS
}

hipError_t launch_pack_blocked(const int8_t* w, int64_t n, int64_t k, int8_t* out, hipStream_t st)
{
    const int64_t n_rows = (n + 255) / 256 * 256;
    const int64_t units = n_rows * k / 16;
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_blocked_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, w,
                       (int)n, (int)k, units, out);
    return hipGetLastError();
}

hipError_t launch_pack_decode(const int8_t* w, const float* sw, int64_t n, int64_t k, void* out,
                              hipStream_t st)
{
    const int64_t units = (n / 16) * (4 + k);
    if (units == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_decode_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st, w, sw,
                       (int)k, units, static_cast<uint4*>(out));
    return hipGetLastError();
}

hipError_t launch_silu(const uint16_t* g, int64_t n, float* out, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(silu_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, g, n, out);
    return hipGetLastError();
}

}  // namespace ck
