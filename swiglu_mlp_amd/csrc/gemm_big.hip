// gemm_big.hip -- the large-problem INT8 GEMM for gfx950: persistent
// workgroups, 256 x BN output tiles (BN = 256 or 192), direct-to-LDS operand
// loads into a 4-deep ring with 3 stages in flight, v_mfma_i32_32x32x32_i8, and
// the ConvRot dequant epilogue y = bf16(fl(fl(f32(acc) * sx[m]) * sw[n])).
//
// Sources: comfy-kitchen PR #277, "The key observation" (the GEMM runs in the
// rotated basis, y = x_rot W_rot^T) and "Measured results" (int32
// accumulation); sglang PR #35994 report, key source excerpts (F32
// per-output-row weight scale).
//
// Design (MI355X: 256 CUs in 8 XCDs, 160 KB LDS per CU, one wave per SIMD):
//  * A workgroup of 4 waves owns a 256 (m) x BN (n) tile; each wave computes a
//    128 x BN/2 sub-tile as (BN/64) x 4 fragments of 32 x 32 (accumulators in
//    AGPRs).  The MFMA computes D[n][m] = sum_k W[n][k] X[m][k], W as the A
//    operand, X as B, so a lane ends up with 4 consecutive n of one row m.
//  * K advances 64 bytes per stage.  A stage of the tile is (256 + BN) rows of
//    64 bytes, moved by buffer_load_dwordx4 ... lds: one wave instruction
//    fills a 1 KB slab (16 rows) of LDS, lane i writing bytes [16 i, 16 i + 16).
//    The 16-byte chunks of a row are XOR-swizzled (chunk ^ ((row >> 1) & 3)) by
//    choosing which global chunk each lane fetches, so the 32 rows read by one
//    ds_read_b128 fall in distinct banks.  Each lane's byte offset into the
//    operand is fixed for the kernel except for the tile's row offset; rows
//    past the matrix fall outside the buffer's range and read as zero.
//  * Stages live in a ring of 4 LDS buffers; loads run 3 stages ahead of the
//    MFMAs.  The stage sequence runs across the workgroup's tiles, so the next
//    tile's first loads are in flight during the current tile's tail and
//    epilogue.
//  * Workgroups are persistent (one per CU); in each round the 32 workgroups
//    of one XCD take 32 consecutive tiles of a grouped order, so they share
//    operand panels in that XCD's L2.
#include "ck_device.hpp"
#include "ck_internal.hpp"

#include <type_traits>

namespace ck {
namespace big {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt that waits for vmcnt <= N only (gfx9 encoding: vmcnt[3:0] and
// [15:14], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_barrier without a memory fence; the empty asm statements stop the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void workgroup_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int BN>
struct Big {
    static constexpr int BM = 256;
    static constexpr int BK = 64;
    static constexpr int NBUF = 4;          // LDS ring
    static constexpr int P = 3;             // stages in flight ahead of compute
    static constexpr int WN = BN / 2;       // wave sub-tile, n extent
    static constexpr int FM = 4;            // 128 / 32
    static constexpr int FN = WN / 32;
    static constexpr int A_SLABS = BN / 16; // W rows, 16 rows per 1 KB slab
    static constexpr int B_SLABS = BM / 16; // X rows
    static constexpr int SLABS = A_SLABS + B_SLABS;
    static constexpr int L = SLABS / 4;     // slab loads per lane per stage
    static constexpr int STAGE = SLABS * 1024;
    static_assert(SLABS % 4 == 0, "slabs must split evenly over 4 waves");
    static_assert(WN % 32 == 0, "wave tile");
};

__device__ __forceinline__ int swz64(int row, int chunk) { return chunk ^ ((row >> 1) & 3); }

// Tile j of the grouped order -> (tm, tn): columns of `group_m` tile-rows.
__device__ __forceinline__ void tile_coords(int j, int tiles_m, int tiles_n, int group_m, int& tm,
                                            int& tn)
{
    const int width = group_m * tiles_n;
    const int grp = j / width;
    const int first_m = grp * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    tm = first_m + (j % width) % gm;
    tn = (j % width) / gm;
}

template <int BN, bool OUT_I32, bool EXTRA>
__global__ __launch_bounds__(256, 1) void gemm_big_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, const int8_t* __restrict__ wq,
    const float* __restrict__ sw, int M, int N, int K, void* __restrict__ out, int tiles_m,
    int tiles_n, int group_m, EpiExtra ex)
{
    // The body uses AMDGPU-only types (buffer resources); the host pass only
    // needs this function's launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    using C = Big<BN>;
    __shared__ __attribute__((aligned(1024))) char smem[C::NBUF * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int tiles = tiles_m * tiles_n;
    const int KT = K / C::BK;

    // tiles of this workgroup: j = q*G + b (q = 0, 1, ...), renumbered within a
    // full round so that the workgroups of one XCD (b % 8) take consecutive
    // tiles.
    const int my_tiles = (tiles - b + G - 1) / G;
    auto tile_of = [&](int q) {
        int j = q * G + b;
        if ((G & 7) == 0 && (q + 1) * G <= tiles) j = q * G + (b & 7) * (G >> 3) + (b >> 3);
        return j;
    };

    // Per-lane byte offsets of this lane's chunk in each of its slabs, relative
    // to the tile's first row (fixed for the kernel).
    const int lrow = lane >> 2;            // row within a 16-row slab
    const int lchunk = lane & 3;           // physical 16-byte chunk within the row
    uint32_t off[C::L];
#pragma unroll
    for (int i = 0; i < C::L; ++i) {
        const int slab = wave + 4 * i;
        const int r = (slab < C::A_SLABS ? slab : slab - C::A_SLABS) * 16 + lrow;
        off[i] = (uint32_t)r * (uint32_t)K + 16u * (uint32_t)swz64(r, lchunk);
    }
    const __amdgpu_buffer_rsrc_t rs_w =
        __builtin_amdgcn_make_buffer_rsrc((void*)wq, (short)0, N * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_x =
        __builtin_amdgcn_make_buffer_rsrc((void*)xq, (short)0, M * K, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs_o =
        __builtin_amdgcn_make_buffer_rsrc(out, (short)0, M * N * (OUT_I32 ? 4 : 2), 0x00020000);

    // issue the loads of global stage s (tile q = s / KT, k-step s % KT)
    auto issue = [&](int s) {
        const int q = s / KT;
        const int kt = s - q * KT;
        int tm, tn;
        tile_coords(tile_of(q), tiles_m, tiles_n, group_m, tm, tn);
        const uint32_t w_row0 = (uint32_t)(tn * BN) * (uint32_t)K;
        const uint32_t x_row0 = (uint32_t)(tm * C::BM) * (uint32_t)K;
        const uint32_t k0 = (uint32_t)(kt * C::BK);
        char* dst_stage = smem + (s % C::NBUF) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::L; ++i) {
            const int slab = wave + 4 * i;           // wave-uniform
            lds_void_t* dst = (lds_void_t*)(dst_stage + slab * 1024);
            if (slab < C::A_SLABS)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_w, dst, 16, w_row0 + off[i], k0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs_x, dst, 16, x_row0 + off[i], k0, 0, 0);
        }
    };

    const int total = my_tiles * KT;
    if (total == 0) return;

    v16i acc[C::FN][C::FM];

    const int lr = lane & 31;
    const int lh = lane >> 5;
    const int wm0 = (wave & 1) * 128;
    const int wn0 = (wave >> 1) * C::WN;

    // One stage of MFMAs out of LDS buffer `buf`; on a tile's first k-step
    // (`first`) the MFMAs take an inline-zero accumulator input.
    auto compute = [&](int buf, auto first) {
        const char* sA = smem + buf * C::STAGE;
        const char* sB = sA + C::A_SLABS * 1024;
#pragma unroll
        for (int ks = 0; ks < C::BK / 32; ++ks) {
            const int ch = 2 * ks + lh;
            v4i af[C::FN], bf[C::FM];
#pragma unroll
            for (int i = 0; i < C::FN; ++i) {
                const int r = wn0 + 32 * i + lr;
                af[i] = *reinterpret_cast<const v4i*>(sA + (r * 4 + swz64(r, ch)) * 16);
            }
#pragma unroll
            for (int j = 0; j < C::FM; ++j) {
                const int r = wm0 + 32 * j + lr;
                bf[j] = *reinterpret_cast<const v4i*>(sB + (r * 4 + swz64(r, ch)) * 16);
            }
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                        af[i], bf[j], (decltype(first)::value && ks == 0) ? v16i{} : acc[i][j], 0, 0, 0);
        }
    };

#pragma unroll
    for (int s = 0; s < C::P; ++s)
        if (s < total) issue(s);

    for (int s = 0; s < total; ++s) {
        // stages issued after s and still possibly in flight
        const int after = min(total - 1, s + C::P - 1) - s;
        if (after >= 2) wait_vmcnt<2 * C::L>();
        else if (after == 1) wait_vmcnt<C::L>();
        else wait_vmcnt<0>();
        // Stage s is in LDS for every wave (each waited for its own loads) and
        // every wave has consumed stage s-1 (its MFMAs read those registers),
        // so a bare barrier suffices; a fenced __syncthreads would also wait
        // for the loads still in flight for stages s+1 .. s+P-1.
        workgroup_barrier();
        if (s + C::P < total) issue(s + C::P);

        const int kt = s % KT;
        if (kt == 0) compute(s % C::NBUF, std::true_type{});
        else compute(s % C::NBUF, std::false_type{});

        if (kt == KT - 1) {
            // ---- epilogue of tile q = s / KT ----
            // D fragment layout (32 x 32): lane l holds column l % 32 (output
            // row m) and, in registers 4 qd .. 4 qd + 3, rows 8 qd + 4 (l / 32)
            // + 0..3 (four consecutive output columns n).  Stores go through a
            // buffer resource: 32-bit offsets, and rows past M fall outside it.
            int tm, tn;
            tile_coords(tile_of(s / KT), tiles_m, tiles_n, group_m, tm, tn);
            const int m_base = tm * C::BM + wm0 + lr;
            const int n_base = tn * BN + wn0 + 4 * lh;
            float sxm[C::FM];
#pragma unroll
            for (int j = 0; j < C::FM; ++j) {
                const int m = min(m_base + 32 * j, M - 1);
                sxm[j] = 0.0f;
                if constexpr (!OUT_I32) sxm[j] = sx[m];
            }
#pragma unroll
            for (int i = 0; i < C::FN; ++i) {
                float4 s4[4];
                bool n_ok[4];
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int n = n_base + 32 * i + 8 * qd;
                    n_ok[qd] = n < N;
                    s4[qd] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if constexpr (!OUT_I32) s4[qd] = *reinterpret_cast<const float4*>(sw + min(n, N - 4));
                }
#pragma unroll
                for (int j = 0; j < C::FM; ++j) {
                    // copy one fragment out of the accumulators here (and not
                    // all of them up front)
                    v16i f = acc[i][j];
                    asm volatile("" : "+v"(f));
                    const uint32_t row = (uint32_t)(m_base + 32 * j) * (uint32_t)N;
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        if (!n_ok[qd]) continue;
                        const uint32_t o = row + (uint32_t)(n_base + 32 * i + 8 * qd);
                        if constexpr (OUT_I32) {
                            const v4i d = {f[4 * qd], f[4 * qd + 1], f[4 * qd + 2], f[4 * qd + 3]};
                            __builtin_amdgcn_raw_buffer_store_b128(d, rs_o, o * 4u, 0, 0);
                        } else {
                            float y0 = ((float)f[4 * qd + 0] * sxm[j]) * s4[qd].x;
                            float y1 = ((float)f[4 * qd + 1] * sxm[j]) * s4[qd].y;
                            float y2 = ((float)f[4 * qd + 2] * sxm[j]) * s4[qd].z;
                            float y3 = ((float)f[4 * qd + 3] * sxm[j]) * s4[qd].w;
                            if constexpr (EXTRA)
                                epi_extra4(y0, y1, y2, y3, ex, min(m_base + 32 * j, M - 1),
                                           n_base + 32 * i + 8 * qd, N);
                            const u32x2 d = {pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
                            __builtin_amdgcn_raw_buffer_store_b64(d, rs_o, o * 2u, 0, 0);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int BN, bool I32, bool EXTRA>
hipError_t launch_big(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, int M,
                      int N, int K, void* out, int num_cu, hipStream_t st, EpiExtra ex)
{
    const int tiles_m = (M + 255) / 256;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n;
    const int grid = tiles < num_cu ? tiles : num_cu;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    hipLaunchKernelGGL((gemm_big_kernel<BN, I32, EXTRA>), dim3(grid), dim3(256), 0, st, xq, sx, wq, sw, M,
                       N, K, out, tiles_m, tiles_n, group_m, ex);
    return hipGetLastError();
}

}  // namespace big

// Large-tile path; returns hipErrorNotSupported when the shape does not suit it
// (the caller then uses the generic kernel).
hipError_t launch_gemm_big(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                           int64_t m, int64_t n, int64_t k, void* out, bool out_i32, int bn,
                           int num_cu, hipStream_t st, EpiExtra ex)
{
    const int M = (int)m, N = (int)n, K = (int)k;
    const bool extra = ex.bias || ex.res;
    if (bn == 256)
        return out_i32 ? big::launch_big<256, true, false>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex)
               : extra ? big::launch_big<256, false, true>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex)
                       : big::launch_big<256, false, false>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex);
    if (bn == 192)
        return out_i32 ? big::launch_big<192, true, false>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex)
               : extra ? big::launch_big<192, false, true>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex)
                       : big::launch_big<192, false, false>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex);
    return hipErrorNotSupported;
}

}  // namespace ck
