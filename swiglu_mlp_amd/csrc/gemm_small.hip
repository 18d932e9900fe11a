// gemm_small.hip -- INT8 GEMM + dequant epilogue for few token rows (M <= 64)
// on operands in the blocked layout (include/ck.h, CK_LAYOUT_BLOCKED).
//
// Sources: comfy-kitchen PR #277, "The key observation" (y = x_rot W_rot^T with
// int32 accumulation); comfy-kitchen PR #248 "Performance improvements for qwen
// 3.x (Part 2)", "Description" (at small M the layer is bound by streaming the
// weights, so they are laid out to be read linearly).
//
// At M <= 64 the weight matrix (N x K bytes) is read once and the arithmetic is
// negligible, so the kernel is bound by HBM.  One workgroup owns 16 weight
// rows (or 32, see NG) and all of K: N / 16 workgroups, each streaming 16 x K
// contiguous bytes in 256-byte runs (16 rows of a 1 KB block half).  Its 8 waves take
// interleaved 64-byte k-chunks so the workgroup reads a contiguous front, and
// each wave keeps two batches of U chunks in flight.  The few activation rows
// (16 per MFMA fragment) come from L2.  Products use v_mfma_i32_16x16x64_i8
// with W as the A operand (16 output columns n) and x as B (16 rows m);
// partial accumulators of the 8 waves are summed through LDS, then one wave
// per 16-row fragment applies y = bf16(fl(fl(f32(acc) * sx[m]) * sw[n])).
//
// W8A16 (A16): the activation is the BF16 rotated x in the BF16 blocked layout;
// each 16-byte INT8 weight piece is widened in registers to two BF16 operands
// of v_mfma_f32_16x16x32_bf16 (lane k-bytes 0..7, then 8..15), matched by two
// 16-byte BF16 activation pieces; FP32 accumulators, summed over the waves in a
// fixed order; y = bf16(fl(acc * sw[n])).
#include "ck_device.hpp"
#include "ck_internal.hpp"

#include <type_traits>

namespace ck {
namespace small {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVES = 8;

template <int MT, bool A16, int NG>
struct SmallCfg {
    // chunks per batch per wave (W8A16 holds twice the activation registers;
    // two weight groups per workgroup hold twice the weight registers)
    static constexpr int U1 = A16 ? (MT == 1 ? 6 : (MT == 2 ? 3 : (MT == 4 ? 2 : 1)))
                                  : (MT == 1 ? 8 : (MT == 2 ? 4 : (MT == 4 ? 3 : 2)));
    static constexpr int U = NG == 1 ? U1 : NG == 2 ? (U1 > 4 ? 4 : (U1 > 1 ? U1 - 1 : 1)) : (U1 > 4 ? 2 : 1);
    static constexpr int XP = A16 ? 2 : 1;   // activation pieces per chunk and fragment
};

// DEC: W in the decode layout (include/ck.h): each 16-row group one linear
// stream, its row scales in the group's 64-byte header.
// A16: xq points to BF16 x_rot (see above); OUT_I32 then writes FP32 sums.
// NG: 16-row weight groups per workgroup (1, 2 or 4).  With NG groups, each
// activation fragment loaded serves NG times the weight bytes: at 16 or more
// rows the activation reads, not the weights, fill a CU's vector-memory path.
template <int MT, bool OUT_I32, bool DEC, bool A16, int NG>
__global__ __launch_bounds__(WAVES * 64) void gemm_small_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, const int8_t* __restrict__ wq,
    const float* __restrict__ sw, int M, int N, int K, int m_rows, int n_rows, void* __restrict__ out,
    EpiExtra ex)
{
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int U = SmallCfg<MT, A16, NG>::U;
    constexpr int XP = SmallCfg<MT, A16, NG>::XP;
    constexpr int NF = NG * MT;                     // output fragments (16 x 16 each)
    constexpr int PASS = NF < WAVES ? NF : WAVES;   // fragments summed per pass, one per wave
    __shared__ v4i red[WAVES][PASS][64];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb0 = blockIdx.x * NG;  // first 16-row group of W (output columns 16 nb0 ..)
    const int KB = K >> 5;           // 1 KB blocks per 32-row block
    const int KC = K >> 6;           // 64-byte k-chunks

    const uint32_t grp_bytes = 64u + 16u * (uint32_t)K;     // DEC: one 16-row group
    const __amdgpu_buffer_rsrc_t rs_w = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wq, (short)0, DEC ? (int)((uint32_t)(N / 16) * grp_bytes) : n_rows * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_x =
        __builtin_amdgcn_make_buffer_rsrc((void*)xq, (short)0, m_rows * K * XP, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_o =
        __builtin_amdgcn_make_buffer_rsrc(out, (short)0, M * N * (OUT_I32 ? 4 : 2), 0x00020000);

    // A 16-row operand fragment of k-chunk j (64 bytes of k): lane l holds row
    // l % 16 and the 16 k-bytes of quarter c = l / 16, which sit in 1 KB block
    // 2 j + c / 2, half c % 2, at row offset 16 r (the 16-row half h of the
    // 32-row block adds 256 bytes).  A and B use the same k assignment, so the
    // order of k inside the chunk does not matter for the dot products.
    const int r = lane & 15;
    const int c = lane >> 4;
    const uint32_t lane_off = (uint32_t)((c >> 1) * 1024 + (c & 1) * 512 + r * 16);
    // DEC: chunk j of group nb is the 1 KB at nb * grp_bytes + 64 + 1024 j,
    // lane l's 16 bytes at 16 l (quarter l / 16, row l % 16)
    uint32_t w_base[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const int nb = nb0 + g;
        w_base[g] = DEC ? (uint32_t)nb * grp_bytes + 64u + (uint32_t)lane * 16u
                        : (uint32_t)((nb >> 1) * KB) * 1024u + (uint32_t)(nb & 1) * 256u + lane_off;
    }
    const uint32_t w_step = DEC ? 1024u : 2048u;   // bytes per 64-byte k-chunk
    // activation piece of fragment f (rows 16 f ..), chunk 0: INT8 codes in the
    // blocked layout, or (A16) BF16 in the BF16 blocked layout, where lane l's
    // 8 values of chunk j, piece s (k = 64 j + 16 c + 8 s ..) sit in the 2 KB
    // k-slice 2 j + c / 2 of row block row / 32, at s * 1024 + (c % 2) * 512 + 16 (row % 32)
    uint32_t x_base[MT];
#pragma unroll
    for (int f = 0; f < MT; ++f) {
        if constexpr (A16) {
            const int row = 16 * f + r;
            x_base[f] = (uint32_t)((row >> 5) * KB + (c >> 1)) * 2048u + (uint32_t)(c & 1) * 512u +
                        (uint32_t)(row & 31) * 16u;
        } else {
            x_base[f] = (uint32_t)((f >> 1) * KB) * 1024u + (uint32_t)(f & 1) * 256u + lane_off;
        }
    }
    const uint32_t x_step = A16 ? 4096u : 2048u;   // activation bytes per 64-k chunk and row block
    // rows past M (padding of the last fragment) load zeros without touching
    // memory: at M < 16 they would be most of the activation reads
    bool x_ok[MT];
#pragma unroll
    for (int f = 0; f < MT; ++f) x_ok[f] = 16 * f + r < M;

    using AccT = std::conditional_t<A16, v4f, v4i>;
    AccT acc[NG][MT];
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int f = 0; f < MT; ++f) acc[g][f] = AccT{0, 0, 0, 0};

    // batch b covers chunks j = wave + WAVES * (U b + u), u < U; chunks past
    // the end load zeros (offset outside the buffers) and add nothing
    auto load = [&](int b, v4i (&w)[U][NG], v4i (&x)[U][MT][XP]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = wave + WAVES * (U * b + u);
            const bool ok = j < KC;
            const uint32_t ko = (uint32_t)j * x_step;
#pragma unroll
            for (int g = 0; g < NG; ++g)
                w[u][g] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs_w, ok ? w_base[g] + (uint32_t)j * w_step : kBufferOutside, 0, 0);
#pragma unroll
            for (int f = 0; f < MT; ++f)
#pragma unroll
                for (int s = 0; s < XP; ++s)
                    x[u][f][s] = __builtin_amdgcn_raw_buffer_load_b128(
                        rs_x, ok && x_ok[f] ? x_base[f] + ko + (uint32_t)s * 1024u : kBufferOutside, 0, 0);
        }
    };
    auto compute = [&](const v4i (&w)[U][NG], const v4i (&x)[U][MT][XP]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                if constexpr (A16) {
                    const v8bf w0 = widen8(w[u][g][0], w[u][g][1]), w1 = widen8(w[u][g][2], w[u][g][3]);
#pragma unroll
                    for (int f = 0; f < MT; ++f) {
                        acc[g][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            w0, __builtin_bit_cast(v8bf, x[u][f][0]), acc[g][f], 0, 0, 0);
                        acc[g][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            w1, __builtin_bit_cast(v8bf, x[u][f][XP - 1]), acc[g][f], 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int f = 0; f < MT; ++f)
                        acc[g][f] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u][g], x[u][f][0], acc[g][f], 0, 0, 0);
                }
            }
        }
    };

    const int batches = (KC + WAVES * U - 1) / (WAVES * U);
    v4i wa[U][NG], xa[U][MT][XP], wb[U][NG], xb[U][MT][XP];
    load(0, wa, xa);
    for (int b = 0; b < batches; b += 2) {
        if (b + 1 < batches) load(b + 1, wb, xb);
        compute(wa, xa);
        if (b + 1 >= batches) break;
        if (b + 2 < batches) load(b + 2, wa, xa);
        compute(wb, xb);
    }

    // ---- epilogue: lane l holds D[n = 4 (l / 16) + i][m = l % 16], i < 4, of
    // fragment f of weight group g ----
    auto epilogue = [&](int g, int f, AccT t) {
        const int nb = nb0 + g;
        const int m = f * 16 + r;
        const int n = nb * 16 + 4 * c;
        const uint32_t row = (uint32_t)m * (uint32_t)N + (uint32_t)n;
        if constexpr (OUT_I32) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, t), rs_o, m < M ? row * 4u : kBufferOutside,
                                                   0, 0);
        } else {
            const float4 s4 = DEC ? *reinterpret_cast<const float4*>(wq + (size_t)nb * grp_bytes + 16 * c)
                                  : *reinterpret_cast<const float4*>(sw + n);
            float y0, y1, y2, y3;
            if constexpr (A16) {
                y0 = t[0] * s4.x;
                y1 = t[1] * s4.y;
                y2 = t[2] * s4.z;
                y3 = t[3] * s4.w;
            } else {
                const float sxm = sx[min(m, M - 1)];
                y0 = ((float)t[0] * sxm) * s4.x;
                y1 = ((float)t[1] * sxm) * s4.y;
                y2 = ((float)t[2] * sxm) * s4.z;
                y3 = ((float)t[3] * sxm) * s4.w;
            }
            epi_extra4(y0, y1, y2, y3, ex, min(m, M - 1), n, N);
            const u32x2 d = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
            __builtin_amdgcn_raw_buffer_store_b64(d, rs_o, m < M ? row * 2u : kBufferOutside, 0, 0);
        }
    };

    // ---- sum the waves' partial accumulators (in wave order), PASS fragments
    // at a time, wave q taking fragment p0 + q ----
#pragma unroll
    for (int p0 = 0; p0 < NF; p0 += PASS) {
        if (p0 > 0) __syncthreads();   // the previous pass has read its sums
#pragma unroll
        for (int q = 0; q < PASS; ++q)
            red[wave][q][lane] = __builtin_bit_cast(v4i, acc[(p0 + q) / MT][(p0 + q) % MT]);
        __syncthreads();
        if (wave < PASS) {
            AccT t = __builtin_bit_cast(AccT, red[0][wave][lane]);
#pragma unroll
            for (int w = 1; w < WAVES; ++w) t += __builtin_bit_cast(AccT, red[w][wave][lane]);
            epilogue((p0 + wave) / MT, (p0 + wave) % MT, t);
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

// Weight groups per workgroup: the most that still leave a workgroup per CU,
// and more than one only where the fragments' activation reads are a load: at
// 16 rows and more (below, the padding rows load nothing).  Measured at
// N = 8192..28672: two groups with one workgroup per CU beat one group with two
// per CU; four beat two at 17..32 rows, and for W8A16 (twice the activation
// bytes) at 16; INT8 at 16 rows gains nothing from four.  (W8A16 at 33..64
// rows on N this wide runs on tiles.)
int groups_per_wg(int M, int N, int MT, bool a16)
{
    if (MT > 4 || M < 16) return 1;
    if ((MT == 2 || (MT == 4 && !a16) || (MT == 1 && a16)) && N % 64 == 0 && N / 64 >= num_cus()) return 4;
    if (N % 32 == 0 && N / 32 >= num_cus()) return 2;
    return 1;
}

template <int MT, bool I32, bool DEC, bool A16 = false>
hipError_t launch(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, int M, int N,
                  int K, void* out, hipStream_t st, EpiExtra ex)
{
    const int m_rows = (M + 255) / 256 * 256;
    const int n_rows = (N + 255) / 256 * 256;
    if constexpr (MT <= 4) {
        const int ng = groups_per_wg(M, N, MT, A16);
        if constexpr (MT == 2 || (MT == 4 && !A16) || (MT == 1 && A16)) {
            if (ng == 4) {
                hipLaunchKernelGGL((gemm_small_kernel<MT, I32, DEC, A16, 4>), dim3(N / 64), dim3(WAVES * 64), 0,
                                   st, xq, sx, wq, sw, M, N, K, m_rows, n_rows, out, ex);
                return hipGetLastError();
            }
        }
        if (ng == 2) {
            hipLaunchKernelGGL((gemm_small_kernel<MT, I32, DEC, A16, 2>), dim3(N / 32), dim3(WAVES * 64), 0, st,
                               xq, sx, wq, sw, M, N, K, m_rows, n_rows, out, ex);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_small_kernel<MT, I32, DEC, A16, 1>), dim3(N / 16), dim3(WAVES * 64), 0, st, xq, sx,
                       wq, sw, M, N, K, m_rows, n_rows, out, ex);
    return hipGetLastError();
}

}  // namespace small

// m <= kSmallMaxM, n % 16 == 0, k % 64 == 0 (checked by the caller).
hipError_t launch_gemm_small(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                             int64_t m, int64_t n, int64_t k, void* out, bool out_i32, hipStream_t st,
                             EpiExtra ex, bool decode)
{
    const int M = (int)m, N = (int)n, K = (int)k;
#define CK_SMALL(MT_)                                                                                   \
    return decode ? (out_i32 ? small::launch<MT_, true, true>(xq, sx, wq, sw, M, N, K, out, st, ex)      \
                             : small::launch<MT_, false, true>(xq, sx, wq, sw, M, N, K, out, st, ex))    \
                  : (out_i32 ? small::launch<MT_, true, false>(xq, sx, wq, sw, M, N, K, out, st, ex)     \
                             : small::launch<MT_, false, false>(xq, sx, wq, sw, M, N, K, out, st, ex))
    if (m <= 16) CK_SMALL(1);
    if (m <= 32) CK_SMALL(2);
    if (m <= 64) CK_SMALL(4);
    CK_SMALL(8);
#undef CK_SMALL
}

// W8A16, m <= 64: x_rot BF16 in the BF16 blocked layout, W blocked.
hipError_t launch_gemm_small_w8a16(const uint16_t* x_rot, const int8_t* wq, const float* sw, int64_t m,
                                   int64_t n, int64_t k, void* out, bool out_f32, hipStream_t st, EpiExtra ex)
{
    const int M = (int)m, N = (int)n, K = (int)k;
    const int8_t* xr = reinterpret_cast<const int8_t*>(x_rot);
#define CK_SMALL(MT_)                                                                                      \
    return out_f32 ? small::launch<MT_, true, false, true>(xr, nullptr, wq, sw, M, N, K, out, st, ex)       \
                   : small::launch<MT_, false, false, true>(xr, nullptr, wq, sw, M, N, K, out, st, ex)
    if (m <= 16) CK_SMALL(1);
    if (m <= 32) CK_SMALL(2);
    if (m <= 64) CK_SMALL(4);
    CK_SMALL(8);
#undef CK_SMALL
}

}  // namespace ck
