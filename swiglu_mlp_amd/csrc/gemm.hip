// gemm.hip -- INT8 x INT8 -> int32 GEMM on the gfx950 matrix cores with the
// ConvRot dequant epilogue: y[m, n] = bf16(fl(fl(f32(acc) * sx[m]) * sw[n])).
//
// Sources: comfy-kitchen PR #277, "The key observation" (the GEMM runs in the
// rotated basis: y = x_rot W_rot^T with no inverse rotation of y) and
// "Measured results" (int32 accumulation); sglang PR #35994 report, key source
// excerpts (F32 per-output-row weight scale).
//
// Both operands are K-contiguous ("NT"): x_q [M, K] and w_q [N, K].  The MFMA
// computes the transposed tile D[n][m] = sum_k W[n][k] X[m][k] with
// v_mfma_i32_32x32x32_i8, W as the A operand and X as the B operand; a lane
// supplies 16 consecutive k of one row to both operands, so whatever order
// the matrix core uses inside the 32-wide k-slice is the same for both and the
// int32 sum is exact.  With D transposed, each lane ends up holding 4
// consecutive output columns n of one output row m, i.e. 8 bytes of BF16 to
// store at once.
//
// Workgroup tile BM x BN (m x n) with BK k per stage; tiles are staged in LDS,
// double-buffered, as 16-byte chunks whose position inside a row is XOR-
// swizzled with the row index so that the 32 lanes reading 32 different rows
// hit distinct banks.  Workgroups are renumbered so that the tiles handled by
// one XCD (workgroups are dealt round-robin over the 8 XCDs) are contiguous,
// and walked in groups of `group_m` tile-rows so that neighbouring workgroups
// share operand panels in that XCD's L2.
#include "ck_device.hpp"
#include "ck_internal.hpp"

#include <atomic>

namespace ck {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

template <int BK>
__device__ __forceinline__ int swz(int row, int chunk)
{
    if constexpr (BK == 128) return chunk ^ (row & 7);
    else return chunk ^ ((row >> 1) & 3);
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool OUT_I32>
__global__ __launch_bounds__(WAVES_M * WAVES_N * 64) void gemm_i8_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, const int8_t* __restrict__ wq,
    const float* __restrict__ sw, int M, int N, int K, void* __restrict__ out, int tiles_m,
    int tiles_n, int group_m, EpiExtra ex)
{
    constexpr int NT = WAVES_M * WAVES_N * 64;
    constexpr int WM = BM / WAVES_M;     // wave tile, m extent
    constexpr int WN = BN / WAVES_N;     // wave tile, n extent
    constexpr int FM = WM / 32;
    constexpr int FN = WN / 32;
    constexpr int CPR = BK / 16;         // 16-byte chunks per tile row
    constexpr int A_CH = BN * CPR;       // W tile chunks
    constexpr int B_CH = BM * CPR;       // X tile chunks
    constexpr int LA = A_CH / NT;
    constexpr int LB = B_CH / NT;
    constexpr int STAGE = A_CH + B_CH;   // chunks per stage
    static_assert(A_CH % NT == 0 && B_CH % NT == 0, "tile/thread mismatch");
    static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile must be a multiple of 32");

    __shared__ uint4 smem[2 * STAGE];

    // ---- tile coordinates (XCD-contiguous, grouped) -------------------------
    const int nwg = gridDim.x;
    int b = blockIdx.x;
    if ((nwg & 7) == 0) b = (b & 7) * (nwg >> 3) + (b >> 3);
    const int width = group_m * tiles_n;
    const int grp = b / width;
    const int first_m = grp * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int tm = first_m + (b % width) % gm;
    const int tn = (b % width) / gm;
    const int m0 = tm * BM;
    const int n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave % WAVES_M) * WM;
    const int wn0 = (wave / WAVES_M) * WN;

    // ---- global -> register staging ------------------------------------------
    // Thread tid moves chunks ci = i*NT + tid of each tile: tile row
    // i*RPI + r0 and chunk column c0 (the same column for every i).  RPI is a
    // multiple of 8, so the row's swizzle term depends on r0 alone.  Rows past
    // the matrix edge are clamped to the last row (their results are dropped).
    constexpr int RPI = NT / CPR;
    static_assert(RPI % 8 == 0, "rows per staging pass must keep the swizzle phase");
    const int r0 = tid / CPR;
    const int c0 = tid % CPR;
    const int dst0 = r0 * CPR + swz<BK>(r0, c0);

    uint4 ra[LA], rb[LB];
    v16i acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = v16i{};

    const int lr = lane & 31;       // operand row within a 32-row fragment
    const int lh = lane >> 5;       // which 16-byte half of the 32-wide k-slice
    const int KT = K / BK;

#define CK_LOAD_GLOBAL(k0)                                                                  \
    do {                                                                                    \
        _Pragma("unroll") for (int i = 0; i < LA; ++i) {                                    \
            const int gr = min(n0 + i * RPI + r0, N - 1);                                   \
            ra[i] = *reinterpret_cast<const uint4*>(wq + (int64_t)gr * K + (k0) + c0 * 16); \
        }                                                                                   \
        _Pragma("unroll") for (int i = 0; i < LB; ++i) {                                    \
            const int gr = min(m0 + i * RPI + r0, M - 1);                                   \
            rb[i] = *reinterpret_cast<const uint4*>(xq + (int64_t)gr * K + (k0) + c0 * 16); \
        }                                                                                   \
    } while (0)
#define CK_STORE_LDS(stage)                                                        \
    do {                                                                           \
        uint4* s_ = smem + (stage) * STAGE;                                        \
        _Pragma("unroll") for (int i = 0; i < LA; ++i) s_[i * NT + dst0] = ra[i];          \
        _Pragma("unroll") for (int i = 0; i < LB; ++i) s_[A_CH + i * NT + dst0] = rb[i];   \
    } while (0)
#define CK_COMPUTE(stage)                                                                       \
    do {                                                                                        \
        const uint4* s_ = smem + (stage) * STAGE;                                               \
        _Pragma("unroll") for (int ks = 0; ks < BK / 32; ++ks) {                                \
            const int ch = 2 * ks + lh;                                                         \
            v4i af[FN], bf[FM];                                                                 \
            _Pragma("unroll") for (int i = 0; i < FN; ++i) {                                    \
                const int r = wn0 + 32 * i + lr;                                                \
                const uint4 v = s_[r * CPR + swz<BK>(r, ch)];                                   \
                af[i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};                            \
            }                                                                                   \
            _Pragma("unroll") for (int j = 0; j < FM; ++j) {                                    \
                const int r = wm0 + 32 * j + lr;                                                \
                const uint4 v = s_[A_CH + r * CPR + swz<BK>(r, ch)];                            \
                bf[j] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};                            \
            }                                                                                   \
            _Pragma("unroll") for (int i = 0; i < FN; ++i)                                      \
                _Pragma("unroll") for (int j = 0; j < FM; ++j)                                  \
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j],  \
                                                                      0, 0, 0);                 \
        }                                                                                       \
    } while (0)

    // Software pipeline: the loads of stage kt+1 are in flight while stage kt
    // is multiplied; the last stage is peeled so no load is conditional.
    CK_LOAD_GLOBAL(0);
    CK_STORE_LDS(0);
    __syncthreads();
    for (int kt = 0; kt + 1 < KT; ++kt) {
        CK_LOAD_GLOBAL((kt + 1) * BK);
        CK_COMPUTE(kt & 1);
        CK_STORE_LDS((kt + 1) & 1);
        __syncthreads();
    }
    CK_COMPUTE((KT - 1) & 1);
#undef CK_LOAD_GLOBAL
#undef CK_STORE_LDS
#undef CK_COMPUTE

    // ---- epilogue -------------------------------------------------------------
    // D fragment layout (32x32): lane l holds column j = l % 32 (output row m)
    // and, in registers 4q..4q+3, rows i = 8q + 4(l/32) + 0..3 (output cols n).
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int m = m0 + wm0 + 32 * j + lr;
        if (m >= M) continue;
        float sxm = 0.0f;
        if constexpr (!OUT_I32) sxm = sx[m];
#pragma unroll
        for (int i = 0; i < FN; ++i) {
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int n = n0 + wn0 + 32 * i + 8 * qd + 4 * lh;
                if (n >= N) continue;
                const int a0 = acc[i][j][4 * qd + 0], a1 = acc[i][j][4 * qd + 1];
                const int a2 = acc[i][j][4 * qd + 2], a3 = acc[i][j][4 * qd + 3];
                if constexpr (OUT_I32) {
                    *reinterpret_cast<int4*>(static_cast<int32_t*>(out) + (int64_t)m * N + n) =
                        make_int4(a0, a1, a2, a3);
                } else {
                    const float4 s4 = *reinterpret_cast<const float4*>(sw + n);
                    float y0 = ((float)a0 * sxm) * s4.x;
                    float y1 = ((float)a1 * sxm) * s4.y;
                    float y2 = ((float)a2 * sxm) * s4.z;
                    float y3 = ((float)a3 * sxm) * s4.w;
                    epi_extra4(y0, y1, y2, y3, ex, m, n, N);
                    const uint32_t p0 = f32_to_bf16_bits(y0) | (f32_to_bf16_bits(y1) << 16);
                    const uint32_t p1 = f32_to_bf16_bits(y2) | (f32_to_bf16_bits(y3) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + (int64_t)m * N + n) =
                        make_uint2(p0, p1);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side: tile-shape choice and launch
// ---------------------------------------------------------------------------
namespace {

// Candidate shapes: the two persistent large-tile kernels (gemm_big.hip) and
// the three generic tiles above.  `eff` is the relative per-CU MFMA
// efficiency of the shape; the choice minimises rounds * tile area / eff,
// where a round is one tile per CU.
struct TileCfg {
    int bm, bn;
    bool big;
    double eff;
};
constexpr TileCfg kCfgs[] = {
    {256, 256, true, 1.00},
    {256, 192, true, 0.97},
    {128, 128, false, 0.60},
    {64, 128, false, 0.35},
};

}  // namespace

// Measured on MI355X: the weight-streaming kernel carries 1 + m / 16 activation
// fragments per weight fragment through each CU's vector-memory path.  Up to
// m = 32 that is cheap and it wins or ties everywhere; beyond, it wins while it
// runs at most one workgroup per CU (n <= 16 * CUs: n = 4096, k = 12288 takes
// 21 us at m = 65..128 against 32 us on 128 x 128 tiles) and loses when each
// CU streams several workgroups (n = 24576, k = 3072: 21 us at m = 64 and 34 us
// at m = 128, against 17 us on tiles).
bool use_small_kernel(int64_t m, int64_t n)
{
    if (m <= 32) return true;
    if (m > kSmallMaxM) return false;
    return n / 16 <= num_cus();
}

int num_cus()
{
    // per-device cache; threads may race to fill an entry, all with the same value
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

namespace {

int pick_cfg(int64_t m, int64_t n, int ncu)
{
    int best = 0;
    double best_t = 0;
    for (int c = 0; c < 4; ++c) {
        const int64_t tiles = ((m + kCfgs[c].bm - 1) / kCfgs[c].bm) * ((n + kCfgs[c].bn - 1) / kCfgs[c].bn);
        const int64_t rounds = (tiles + ncu - 1) / ncu;
        const double t = (double)rounds * kCfgs[c].bm * kCfgs[c].bn / kCfgs[c].eff;
        if (c == 0 || t < best_t) {
            best = c;
            best_t = t;
        }
    }
    return best;
}

template <int BM, int BN, int BK, int WM_, int WN_, bool I32>
hipError_t launch_one(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, int M,
                      int N, int K, void* out, hipStream_t st, EpiExtra ex)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int group_m = tiles_m < 8 ? tiles_m : 8;
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM_, WN_, I32>), dim3(tiles_m * tiles_n),
                       dim3(WM_ * WN_ * 64), 0, st, xq, sx, wq, sw, M, N, K, out, tiles_m, tiles_n,
                       group_m, ex);
    return hipGetLastError();
}

template <bool I32>
hipError_t launch_gemm_t(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                         int64_t m, int64_t n, int64_t k, void* out, hipStream_t st,
                         EpiExtra ex = EpiExtra{})
{
    const int ncu = num_cus();
    const int cfg = pick_cfg(m, n, ncu);
    if (kCfgs[cfg].big)
        return launch_gemm_big(xq, sx, wq, sw, m, n, k, out, I32, kCfgs[cfg].bn, ncu, st, ex);
    const bool bk128 = (k % 128) == 0;
    const int M = (int)m, N = (int)n, K = (int)k;
    switch ((cfg - 2) * 2 + (bk128 ? 1 : 0)) {
        case 0: return launch_one<128, 128, 64, 2, 2, I32>(xq, sx, wq, sw, M, N, K, out, st, ex);
        case 1: return launch_one<128, 128, 128, 2, 2, I32>(xq, sx, wq, sw, M, N, K, out, st, ex);
        case 2: return launch_one<64, 128, 64, 2, 2, I32>(xq, sx, wq, sw, M, N, K, out, st, ex);
        default: return launch_one<64, 128, 128, 2, 2, I32>(xq, sx, wq, sw, M, N, K, out, st, ex);
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                            int64_t m, int64_t n, int64_t k, uint16_t* y, int layout, hipStream_t st,
                            EpiExtra ex, void* ws, size_t ws_bytes)
{
    if (m == 0 || n == 0) return hipSuccess;
    if (layout == 2) return launch_gemm_small(xq, sx, wq, sw, m, n, k, y, false, st, ex, true);
    const bool blocked = layout == 1;
    hipError_t err = hipSuccess;
    if (blocked && launch_gemm_blk_splitk(xq, sx, wq, sw, m, n, k, y, st, ex, ws, ws_bytes, &err)) return err;
    if (blocked && use_small_kernel(m, n)) return launch_gemm_small(xq, sx, wq, sw, m, n, k, y, false, st, ex);
    if (blocked) return launch_gemm_blk(xq, sx, wq, sw, m, n, k, y, false, num_cus(), st, ex);
    return launch_gemm_t<false>(xq, sx, wq, sw, m, n, k, y, st, ex);
}

hipError_t launch_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t m, int64_t n, int64_t k,
                           int32_t* acc, int layout, hipStream_t st)
{
    if (m == 0 || n == 0) return hipSuccess;
    if (layout == 2) return launch_gemm_small(xq, nullptr, wq, nullptr, m, n, k, acc, true, st, EpiExtra{}, true);
    const bool blocked = layout == 1;
    if (blocked && use_small_kernel(m, n)) return launch_gemm_small(xq, nullptr, wq, nullptr, m, n, k, acc, true, st);
    if (blocked) return launch_gemm_blk(xq, nullptr, wq, nullptr, m, n, k, acc, true, num_cus(), st);
    return launch_gemm_t<true>(xq, nullptr, wq, nullptr, m, n, k, acc, st);
}

}  // namespace ck
