// gemm_blk.hip -- INT8 GEMM for gfx950 on operands stored in the blocked
// layout (include/ck.h, CK_LAYOUT_BLOCKED), with the ConvRot dequant
// epilogue y = bf16(fl(fl(f32(acc) * sx[m]) * sw[n])).
//
// Sources: comfy-kitchen PR #277, "The key observation" (the GEMM runs in the
// rotated basis, y = x_rot W_rot^T) and "Measured results" (int32
// accumulation); sglang PR #35994 report, key source excerpts (F32
// per-output-row weight scale); comfy-kitchen PR #248 "Performance
// improvements for qwen 3.x (Part 2)", "Description" (weights relaid out once
// so the GEMM reads them linearly).
//
// Why the blocked layout: on MI355X the L2 -> LDS stream rate depends on how
// many cache lines one load instruction touches.  Measured with
// buffer_load_dwordx4 ... lds over all 256 CUs: 1 KB contiguous per
// instruction streams at ~27 TB/s, 8 rows x 128 B at ~15 TB/s, 16 rows x 64 B
// at ~12.7 TB/s.  A 256 x 256 tile needs ~66 GB/s per CU (~17 TB/s) at full
// MFMA rate.  In the blocked layout each 1 KB block is one 32-row x 32-byte
// MFMA operand fragment in lane order, so
//   * one load instruction moves one contiguous KB into LDS, and
//   * every ds_read_b128 of a fragment reads 1 KB linearly (no bank conflicts).
//
// Kernel structure (4 waves in a 2 x 2 grid; one workgroup per CU for the
// 256-wide tiles and the two-slice stages, two for the other 128-wide ones):
//   * Workgroup tile BM x BN (m x n), wave sub-tile BM/2 x BN/2 built from
//     32 x 32 fragments of v_mfma_i32_32x32x32_i8 with accumulators in AGPRs.
//     The MFMA computes D[n][m] = sum_k W[n][k] X[m][k] (W is the A operand),
//     so a lane ends with 4 consecutive n of one output row m.  A wave's LDS
//     reads per k-slice are FN + FM fragments for FN * FM MFMAs, which is why
//     the 4 x 4-fragment waves of the 256 x 256 tile are the fastest shape: the
//     2 x 2-fragment waves of the 128 x 128 tile read as many LDS bytes per
//     MFMA as the LDS delivers.
//   * K advances 2 KSL 32-byte k-slices per stage (64 bytes, or 128 or 256
//     for the few-tile GEMMs that use KSL = 2 or 4).  Stages live in a ring of (at most) 4
//     LDS buffers; loads run 3 stages ahead.  Each stage is split in two halves
//     around one barrier: the first half multiplies the first KSL k-slices,
//     reads the last KSL k-slices' fragments and issues the loads of stage
//     s+3; the second multiplies the last KSL k-slices and reads the next
//     stage's first-half fragments, so MFMAs never wait on LDS.  The order
//     inside each half is fixed in source order with sched_barrier.
//   * The loads are LDS DMA (buffer_load_dwordx4 ... lds) issued from inline
//     assembly, with the waits counted by hand (see lds_dma_b128).
//   * Workgroups are persistent; the stage sequence runs across a workgroup's
//     tiles so the next tile's loads overlap the current tile's epilogue.  In
//     each round the workgroups of one XCD take consecutive tiles of a grouped
//     order, so they share operand panels in that XCD's L2.
//   * Split K (few-tile GEMMs with a workspace): a work unit is a tile and one
//     of ksplit equal k ranges; the int32 variant then writes unit (tile,
//     split s) to partial s of [ksplit][M][N], and splitk_reduce_kernel adds
//     the partials (exact in int32) and applies the same epilogue.
#include "ck_device.hpp"
#include "ck_internal.hpp"

#include <type_traits>

namespace ck {
namespace blk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt encodings (gfx9: vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8])
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_barrier without a memory fence (a fenced __syncthreads would also wait for
// the loads still in flight for later stages); the empty asm statements stop
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void workgroup_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A16: the X operand is BF16 (2 bytes per k) in the BF16 blocked layout and
// the INT8 W fragments are widened to BF16 in registers (W8A16); the stage
// then holds twice the X bytes.
// KSL: k-slices (32 bytes of k each) per half stage.  A stage covers 2 KSL
// k-slices; KSL = 2 halves the stages, and with them the per-stage fixed cost
// (barrier, waits, read latency), for small tiles that run one workgroup per
// CU.
// The ring has as many slots as fit the LDS share of a workgroup (160 KB per
// CU over the workgroups meant to share it: one for tiles of 256 x 192 and
// larger and for KSL > 1, two otherwise; 6 KB of it go to scale buffers), at
// most NMAX; P = NBUF - 1 stages are in flight.
template <int BM_, int BN_, bool A16, int KSL_ = 1>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, KSL = KSL_;
    static constexpr int XS = A16 ? 2 : 1;         // X bytes per k
    static constexpr int FM = BM / 64;             // fragments per wave along m
    static constexpr int FN = BN / 64;             // fragments per wave along n
    static constexpr int A_BLK = (BN / 32) * 2 * KSL;      // W blocks per stage
    static constexpr int B_BLK = (BM / 32) * 2 * KSL * XS; // X blocks per stage
    static constexpr int BLK = A_BLK + B_BLK;
    static constexpr int L = BLK / 4;              // block loads per lane per stage
    static constexpr int STAGE = BLK * 1024;
    static constexpr int PER_CU = (BM * BN >= 256 * 192 || KSL > 1) ? 1 : 2;
    static constexpr int NMAX = 4;
    static constexpr int FIT = (160 * 1024 / PER_CU - 6144) / STAGE;
    static constexpr int NBUF = FIT < NMAX ? FIT : NMAX;   // LDS ring slots
    static constexpr int P = NBUF - 1;             // stages in flight
    static_assert(NBUF >= 3, "the ring needs at least 3 slots");
    static_assert(BLK % 4 == 0, "blocks must split evenly over 4 waves");
};

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

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes at buffer
// offset voff + soff land at LDS byte address lds + 16 l.  Written as inline
// assembly so the compiler does not track this LDS write itself: it would
// otherwise wait for every such load in flight before any later LDS read,
// which empties the prefetch ring.  The caller orders the loads and the reads
// with explicit s_waitcnt vmcnt and barriers.  M0 must be set one instruction
// before the load uses it.
__device__ __forceinline__ void lds_dma_b128(v4i rsrc, uint32_t voff, uint32_t soff, uint32_t lds)
{
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
        : "memory", "m0");
}

__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    return v4i{(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// EXTRA: the epilogue adds the optional bias / residual (a separate
// instantiation, so the plain epilogue carries no branches for them).
// A16 (W8A16): xq points to BF16 values, the accumulators are FP32, the
// epilogue is y = bf16(fl(acc * sw[n])) (sx unused), and OUT_I32 writes the
// raw FP32 accumulators.
template <int BM, int BN, bool OUT_I32, bool EXTRA, bool A16, int KSL>
__global__ __launch_bounds__(256) void gemm_blk_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ sx, const int8_t* __restrict__ wq,
    const float* __restrict__ sw, int M, int N, int K, int m_rows, int n_rows, void* __restrict__ out,
    int tiles_m, int tiles_n, int group_m, EpiExtra ex, int ksplit)
{
    // The body uses AMDGPU-only types (buffer resources); the host pass only
    // needs this function's launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
    using C = Cfg<BM, BN, A16, KSL>;
    using AccT = std::conditional_t<A16, v16f, v16i>;
    // LDS: the NBUF-slot operand ring, then two scale buffers (tile q uses
    // buffer q % 2), each 1 KB of row scales sx, 1 KB of column scales sw
    // and, with EXTRA, 1 KB of bias.
    constexpr int SCALES = EXTRA ? 3072 : 2048;
    __shared__ __attribute__((aligned(1024))) char smem[C::NBUF * C::STAGE + 2 * SCALES];
    constexpr int AW = C::A_BLK / 4;   // W blocks each wave loads per stage
    constexpr int XW = C::B_BLK / 4;   // X blocks each wave loads per stage
    constexpr int NMF = C::FN * C::FM; // fragment pairs (MFMA steps) per wave per k-slice
    constexpr int NDS = C::FN + C::FM * C::XS; // fragment reads per wave per k-slice
    constexpr int KS2 = 2 * KSL;       // k-slices per stage
    // steps of the two halves of a stage (small tiles have fewer MFMAs than
    // reads or loads)
    // BF16 stores per wave in one epilogue (two 16-byte stores per fragment).
    // The int32 variant issues more than the vmcnt field can express and is
    // waited for in full.
    constexpr int NST = OUT_I32 ? 0 : 2 * NMF;
    static_assert((C::P - 1) * C::L + 1 + NST < 64, "vmcnt range");
    constexpr int STEPS1 = KSL * (NMF > NDS ? NMF : NDS);
    constexpr int STEPS0 = STEPS1 > AW + XW ? STEPS1 : AW + XW;
    // The large INT8 tiles spread a stage's loads over both halves, one every
    // few MFMAs: issued in a burst, the 32 loads of a stage fill the texture
    // unit's command queue and stall the MFMA stream behind them.
    constexpr bool SPREAD = !A16 && KSL == 1 && BM * BN >= 256 * 192;
    constexpr int NL = AW + XW;                  // loads per wave per stage
    constexpr int HL = SPREAD ? NL / 2 : NL;     // ... issued in the first half
    // loads issued after a stage's last load and before the mid-stage wait two
    // stages later: the next stage's (L) and the first-half loads of the stage
    // after that, or (P - 1) L when every load goes out in the first half
    constexpr int OUTS = SPREAD ? (C::P - 2) * C::L + HL : (C::P - 1) * C::L;
    static_assert(OUTS + 1 + NST < 64, "vmcnt range");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int tiles = tiles_m * tiles_n;
    const int units = tiles * ksplit;   // work units: (split, tile), split-major
    const int KU = K / ksplit;          // k of one unit
    const int KT = KU / (64 * KSL);     // stages per unit
    const int KB = K / 32;              // k-slices per 32-row block (W: 1 KB, X: XS KB each)
    const int my_tiles = (units - b + G - 1) / G;
    const int total = my_tiles * KT;
    if (total == 0) return;

    // Within a full round the workgroups of one XCD (b % 8) take consecutive
    // units; the last, partial round keeps the plain order.
    const bool xcd_order = (G & 7) == 0;
    const int b_xcd = (b & 7) * (G >> 3) + (b >> 3);
    auto tile_of = [&](int q) {   // the unit index of this workgroup's q-th unit
        const bool full = xcd_order & ((q + 1) * G <= units);
        return q * G + (full ? b_xcd : b);
    };
    // Operand buffers span the padded row counts m_rows, n_rows (multiples of
    // 256), so every block a tile touches is inside the buffer.
    const v4i rs_w = make_rsrc(wq, (uint32_t)(n_rows * K));
    const v4i rs_x = make_rsrc(xq, (uint32_t)(m_rows * K * C::XS));
    // scale vectors (absent, so every lane out of range, for the int32
    // variant; no activation scale in W8A16)
    const v4i rs_sx = make_rsrc(sx, (OUT_I32 || A16) ? 0u : (uint32_t)M * 4u);
    const v4i rs_sw = make_rsrc(sw, OUT_I32 ? 0u : (uint32_t)N * 4u);
    const v4i rs_b = make_rsrc(ex.bias, (EXTRA && ex.bias) ? (uint32_t)N * 4u : 0u);
    const __amdgpu_buffer_rsrc_t rs_o =
        __builtin_amdgcn_make_buffer_rsrc(out, (short)0, M * N * (OUT_I32 ? 4 * ksplit : 2), 0x00020000);
    const uint32_t smem_addr = (uint32_t)(uintptr_t)(lds_void_t*)smem;
    const uint32_t lane16 = (uint32_t)lane * 16u;

    // Load cursor: the stage whose loads are issued next (it stops at the last
    // stage, so the final P issues reload that stage into slots nobody reads
    // again; this keeps the number of loads per stage, and the wait counts,
    // constant).  la / lx: byte offset of the cursor tile's first W / X row
    // block at the unit's first k.
    int ls = 0, lq = 0, lkt = 0;
    uint32_t la = 0, lx = 0;
    auto set_tile = [&](int q) {
        int tm, tn;
        const int u = tile_of(q);
        const int k0 = (u / tiles) * (KU / 32);   // the unit's first k-slice
        tile_coords(u % tiles, tiles_m, tiles_n, group_m, tm, tn);
        la = (uint32_t)(tn * (BN / 32) * KB + k0) * 1024u;
        lx = (uint32_t)(tm * (BM / 32) * KB + k0) * (1024u * C::XS);
    };
    auto advance = [&]() {
        if (ls + 1 < total) {
            ++ls;
            if (++lkt == KT) {
                lkt = 0;
                set_tile(++lq);
            }
        }
    };
    // Block a of this wave's share: W block ai = wave * AW + a covers row
    // block ai / KS2, k-slice ai % KS2 of the stage.  X blocks follow the W
    // blocks in the LDS stage: X block bj covers row block bj / (KS2 XS) and
    // the bj % (KS2 XS)-th KB of the stage's KS2 XS KB of that row block.
    auto issue_one = [&](int a, uint32_t slot_addr) {
        if (a < AW) {
            const int ai = wave * AW + a;
            const uint32_t off = la + (uint32_t)lkt * (1024u * KS2) +
                                 (uint32_t)((ai / (unsigned)KS2) * KB + (ai % (unsigned)KS2)) * 1024u;
            lds_dma_b128(rs_w, lane16, off, slot_addr + (uint32_t)ai * 1024u);
        } else {
            constexpr int XR = KS2 * C::XS;   // X blocks per row block per stage
            const int bj = wave * XW + (a - AW);
            const uint32_t off = lx + (uint32_t)lkt * (1024u * XR) +
                                 (uint32_t)((bj / XR) * KB * C::XS + (bj % XR)) * 1024u;
            lds_dma_b128(rs_x, lane16, off, slot_addr + (uint32_t)(C::A_BLK + bj) * 1024u);
        }
    };

    AccT acc[C::FN][C::FM];
    const int lr = lane & 31;
    const int lh = lane >> 5;
    const int wm0 = (wave & 1) * (BM / 2);
    const int wn0 = (wave >> 1) * (BN / 2);
    // This wave's fragments of a stage: W fragment i, k-slice ks at block
    // (wn0 / 32 + i) * KS2 + ks; X fragment j, k-slice ks, part h (the XS KB
    // of one k-slice) at block A_BLK + ((wm0 / 32 + j) * KS2 + ks) * XS + h.
    auto frag_a = [&](int buf, int i, int ks) {
        const int blk = ((wn0 >> 5) + i) * KS2 + ks;
        return *reinterpret_cast<const v4i*>(smem + buf * C::STAGE + blk * 1024 + lane * 16);
    };
    auto frag_b = [&](int buf, int j, int ks, int h) {
        const int blk = C::A_BLK + (((wm0 >> 5) + j) * KS2 + ks) * C::XS + h;
        return *reinterpret_cast<const v4i*>(smem + buf * C::STAGE + blk * 1024 + lane * 16);
    };

    set_tile(0);
#pragma unroll
    for (int p = 0; p < C::P; ++p) {
#pragma unroll
        for (int a = 0; a < AW + XW; ++a) issue_one(a, smem_addr + (uint32_t)(p * C::STAGE));
        advance();
    }
    wait_vmcnt<(C::P - 1) * C::L>();
    workgroup_barrier();
    v4i fa[KSL][C::FN], fb[KSL][C::FM][C::XS];
#pragma unroll
    for (int ks = 0; ks < KSL; ++ks) {
#pragma unroll
        for (int i = 0; i < C::FN; ++i) fa[ks][i] = frag_a(0, i, ks);
#pragma unroll
        for (int j = 0; j < C::FM; ++j)
#pragma unroll
            for (int h = 0; h < C::XS; ++h) fb[ks][j][h] = frag_b(0, j, ks, h);
    }

    // One stage s (ring slot s % NBUF).  The instruction order inside each half
    // is fixed in source order (sched_barrier): MFMA k, then fragment read k,
    // then load k, so reads and loads issue in the shadow of the MFMAs.
    // The compiler sees no global loads at all: the tile's scale vectors come
    // into LDS by the same DMA, one load per wave at the tile's first stage
    // (even waves sx, odd waves sw), so the epilogue never makes the compiler
    // wait for the prefetch loads in flight.
    //
    // vmcnt bookkeeping at the mid-stage wait of stage s: the loads of stage
    // s + 1 must have landed.  Issued after them are the loads of s + 2 ..
    // s + P ((P - 1) L; with SPREAD the loads of a stage go out over the two
    // halves of the stage P earlier, so (P - 2) L + HL), plus, on a tile's
    // stages kt <= P - 2, that tile's scale load (1) and, from the second tile
    // on, the previous epilogue's NST stores.
    // A smaller wait count than the number issued after is always safe.
    // W8A16: the W fragments of a k-slice widened to BF16 (two MFMA operands
    // each); fragment i + 1 is widened in the shadow of fragment i's MFMAs.
    v8bf cw[A16 ? C::FN : 1][2];
    auto widen = [&](const v4i (&w)[C::FN], int i) {
        if constexpr (A16) {
            cw[i][0] = widen8(w[i][0], w[i][1]);
            cw[i][1] = widen8(w[i][2], w[i][3]);
        }
    };
    // MFMA step k of a half: k-slice ks = k / NMF of the half, fragment pair
    // (i, j) = ((k % NMF) / FM, k % FM).  One INT8 MFMA, or in W8A16 two BF16
    // MFMAs over the two 8-byte halves of the W fragment (lane k-bytes 0..7,
    // then 8..15), matched by the two X parts.
    auto mfma_step = [&](int k, const v4i (&w)[KSL][C::FN], const v4i (&x)[KSL][C::FM][C::XS], bool zero) {
        const int ks = k / NMF, kk = k % NMF;
        const int i = kk / C::FM, j = kk % C::FM;
        const AccT c = (zero && ks == 0) ? AccT{} : acc[i][j];
        if constexpr (A16) {
            if (kk == 0) widen(w[ks], 0);
            const AccT t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cw[i][0], __builtin_bit_cast(v8bf, x[ks][j][0]),
                                                                   c, 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cw[i][1], __builtin_bit_cast(v8bf, x[ks][j][1]), t,
                                                                0, 0, 0);
            if (j == 0 && i + 1 < C::FN) widen(w[ks], i + 1);
        } else {
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(w[ks][i], x[ks][j][0], c, 0, 0, 0);
        }
    };
    // Fragment read r of a half: k-slice ks0 + r / NDS; within it W fragment
    // rr < FN, else X fragment (rr - FN) / XS, part (rr - FN) % XS.
    auto read_step = [&](int r, int buf, int ks0, v4i (&w)[KSL][C::FN], v4i (&x)[KSL][C::FM][C::XS]) {
        if (r >= KSL * NDS) return;
        const int ks = r / NDS, rr = r % NDS;
        if (rr < C::FN) w[ks][rr] = frag_a(buf, rr, ks0 + ks);
        else x[ks][(rr - C::FN) / C::XS][(rr - C::FN) % C::XS] =
            frag_b(buf, (rr - C::FN) / C::XS, ks0 + ks, (rr - C::FN) % C::XS);
    };

    auto stage = [&](int s, int kt, auto first, bool after_epilogue, int tm, int tn, int q) {
        const int buf = (int)((unsigned)s % C::NBUF);
        const int nbuf = (int)((unsigned)(s + 1) % C::NBUF);
        const uint32_t lslot = smem_addr + (uint32_t)(((unsigned)(s + C::P) % C::NBUF) * C::STAGE);
        v4i ga[KSL][C::FN], gb[KSL][C::FM][C::XS];
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(first)::value) {
            const uint32_t sbase = smem_addr + (uint32_t)(C::NBUF * C::STAGE + (q & 1) * SCALES);
            if constexpr (!EXTRA) {
                const bool odd = wave & 1;
                lds_dma_b128(odd ? rs_sw : rs_sx, lane16, (uint32_t)((odd ? tn * BN : tm * BM) * 4),
                             sbase + (odd ? 1024u : 0u));
            } else {
                // wave 0: sx, waves 1 and 3: sw, wave 2: the bias (zeros when absent)
                // (uniform branches: selecting among three resources made the
                // compiler keep the accumulators in scratch)
                if (wave == 0)
                    lds_dma_b128(rs_sx, lane16, (uint32_t)(tm * BM * 4), sbase);
                else if (wave == 2)
                    lds_dma_b128(rs_b, lane16, (uint32_t)(tn * BN * 4), sbase + 2048u);
                else
                    lds_dma_b128(rs_sw, lane16, (uint32_t)(tn * BN * 4), sbase + 1024u);
            }
        }
#pragma unroll
        for (int k = 0; k < (SPREAD ? STEPS1 : STEPS0); ++k) {
            if (k < KSL * NMF) mfma_step(k, fa, fb, decltype(first)::value);
            read_step(k, buf, KSL, ga, gb);
            if constexpr (SPREAD) {
                constexpr int SP = STEPS1 / HL;
                if (k % SP == SP / 2 && k / SP < HL) issue_one(k / SP, lslot);
            } else {
                if (k < NL) issue_one(k, lslot);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (!SPREAD) advance();

        wait_lgkmcnt0();              // this wave's second-half fragments are in registers
        if (kt <= C::P - 2) {
            if (after_epilogue) wait_vmcnt<OUTS + 1 + NST>();
            else wait_vmcnt<OUTS + 1>();
        } else {
            wait_vmcnt<OUTS>();
        }
        workgroup_barrier();          // ... for every wave; slot s % NBUF is no longer read

        // slot (s + P) % NBUF was last read in stage s - 1, before that
        // stage's barrier, so the second-half loads may go into it too
#pragma unroll
        for (int k = 0; k < STEPS1; ++k) {
            if (k < KSL * NMF) mfma_step(k, ga, gb, false);
            read_step(k, nbuf, 0, fa, fb);
            if constexpr (SPREAD) {
                constexpr int SP = STEPS1 / (NL - HL);
                if (k % SP == SP / 2 && k / SP < NL - HL) issue_one(HL + k / SP, lslot);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (SPREAD) advance();
    };

    auto epilogue = [&](int q, int tm, int tn, int sp) {
        // D fragment (32 x 32): lane l holds column l % 32 (output row m)
        // and, in registers 4 qd .. 4 qd + 3, rows 8 qd + 4 (l / 32) + 0..3
        // (four consecutive output columns n).  Stores go through a buffer
        // resource: rows past M fall outside it, and masked columns are given
        // an offset past its end, so both are dropped while every lane still
        // issues the same number of stores.  The int32 variant writes split
        // sp's partial (rows past M are given the past-the-end offset too: in
        // a partial they would land in the next one).
        const int m_base = tm * BM + wm0 + lr;
        const int n_base = tn * BN + wn0 + 4 * lh;
        const char* sc = smem + C::NBUF * C::STAGE + (q & 1) * SCALES;
        // EXTRA: all of this lane's residual words, loaded together up front
        uint2 rall[EXTRA ? C::FN : 1][EXTRA ? C::FM : 1][4];
        const bool has_b = EXTRA && ex.bias != nullptr;
        const bool has_r = EXTRA && ex.res != nullptr;
        if constexpr (EXTRA) {
#pragma unroll
            for (int i = 0; i < C::FN; ++i)
#pragma unroll
                for (int j = 0; j < C::FM; ++j)
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) rall[i][j][qd] = make_uint2(0u, 0u);
            if (has_r) {
#pragma unroll
                for (int i = 0; i < C::FN; ++i)
#pragma unroll
                    for (int j = 0; j < C::FM; ++j)
#pragma unroll
                        for (int qd = 0; qd < 4; ++qd) {
                            const int mm = min(m_base + 32 * j, M - 1);
                            const int nn = min(n_base + 32 * i + 8 * qd, N - 4);
                            rall[i][j][qd] = *reinterpret_cast<const uint2*>(ex.res + (int64_t)mm * N + nn);
                        }
            }
        }
        float sxm[C::FM];
#pragma unroll
        for (int j = 0; j < C::FM; ++j) {
            sxm[j] = 0.0f;
            if constexpr (!OUT_I32 && !A16) sxm[j] = *reinterpret_cast<const float*>(sc + (wm0 + lr + 32 * j) * 4);
        }
        // Fragments go out one row block at a time (j outer), so the two
        // fragments that share each row's 128-byte line are stored back to
        // back and the line is whole in L2 before it can be evicted (with i
        // outer, half-written lines were written back twice: 23% more HBM
        // writes for c5's gate_up).
#pragma unroll
        for (int j = 0; j < C::FM; ++j) {
#pragma unroll
            for (int i = 0; i < C::FN; ++i) {
                float4 s4[4], b4[4];
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    if constexpr (EXTRA)
                        b4[qd] = *reinterpret_cast<const float4*>(sc + 2048 + (wn0 + 4 * lh + 32 * i + 8 * qd) * 4);
                    s4[qd] = make_float4(0.f, 0.f, 0.f, 0.f);
                    if constexpr (!OUT_I32)
                        s4[qd] = *reinterpret_cast<const float4*>(sc + 1024 + (wn0 + 4 * lh + 32 * i + 8 * qd) * 4);
                }
                // copy one fragment out of the accumulators here, not all of
                // them up front (the empty asm statements pin the copy between
                // the previous fragment's stores and this fragment's math)
                asm volatile("" : "+a"(acc[i][j]));
                AccT f = acc[i][j];
                asm volatile("" : "+v"(f));
                const uint32_t row = (uint32_t)(m_base + 32 * j) * (uint32_t)N;
                if constexpr (OUT_I32) {
                    const uint32_t prow = row + (uint32_t)sp * (uint32_t)M * (uint32_t)N;
                    const bool mok = m_base + 32 * j < M;
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        const int n = n_base + 32 * i + 8 * qd;
                        const uint32_t ob = (mok && n < N) ? (prow + (uint32_t)n) * 4u : kBufferOutside;
                        const v4i d = __builtin_bit_cast(
                            v4i, (std::conditional_t<A16, float4, int4>){f[4 * qd], f[4 * qd + 1], f[4 * qd + 2],
                                                                         f[4 * qd + 3]});
                        __builtin_amdgcn_raw_buffer_store_b128(d, rs_o, ob, 0, 0);
                    }
                } else {
                    uint32_t w[4][2];
#pragma unroll
                    for (int qd = 0; qd < 4; ++qd) {
                        float y0, y1, y2, y3;
                        if constexpr (A16) {
                            y0 = f[4 * qd + 0] * s4[qd].x;
                            y1 = f[4 * qd + 1] * s4[qd].y;
                            y2 = f[4 * qd + 2] * s4[qd].z;
                            y3 = f[4 * qd + 3] * s4[qd].w;
                        } else {
                            y0 = ((float)f[4 * qd + 0] * sxm[j]) * s4[qd].x;
                            y1 = ((float)f[4 * qd + 1] * sxm[j]) * s4[qd].y;
                            y2 = ((float)f[4 * qd + 2] * sxm[j]) * s4[qd].z;
                            y3 = ((float)f[4 * qd + 3] * sxm[j]) * s4[qd].w;
                        }
                        if constexpr (EXTRA) {
                            // selects, not branches (an absent term must not
                            // turn -0 into +0)
                            y0 = has_b ? y0 + b4[qd].x : y0;
                            y1 = has_b ? y1 + b4[qd].y : y1;
                            y2 = has_b ? y2 + b4[qd].z : y2;
                            y3 = has_b ? y3 + b4[qd].w : y3;
                            const uint2 r = rall[i][j][qd];
                            y0 = has_r ? y0 + bf16_lo(r.x) : y0;
                            y1 = has_r ? y1 + bf16_hi(r.x) : y1;
                            y2 = has_r ? y2 + bf16_lo(r.y) : y2;
                            y3 = has_r ? y3 + bf16_hi(r.y) : y3;
                        }
                        w[qd][0] = pack_bf16x2(y0, y1);
                        w[qd][1] = pack_bf16x2(y2, y3);
                    }
                    // Columns 8p + 4 lh + 0..3 (p = qd) -> swap the upper lanes'
                    // even-p words with the lower lanes' odd-p words, so lane l
                    // holds 8 consecutive columns 16 h + 8 lh + 0..7 (h = 0, 1)
                    // and stores them with one 16-byte write each.
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        uint32_t x0 = w[2 * h][0], x1 = w[2 * h][1];
                        uint32_t y0 = w[2 * h + 1][0], y1 = w[2 * h + 1][1];
                        const auto r0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
                        const auto r1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
                        const int n = tn * BN + wn0 + 32 * i + 16 * h + 8 * lh;
                        const uint32_t ob = n < N ? (row + (uint32_t)n) * 2u : kBufferOutside;
                        const v4i d = {(int)r0[0], (int)r1[0], (int)r0[1], (int)r1[1]};
                        __builtin_amdgcn_raw_buffer_store_b128(d, rs_o, ob, 0, 0);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    int s = 0;
    for (int q = 0; q < my_tiles; ++q) {
        int tm, tn;
        const int u = tile_of(q);
        tile_coords(u % tiles, tiles_m, tiles_n, group_m, tm, tn);
        stage(s++, 0, std::true_type{}, q > 0, tm, tn, q);
        for (int kt = 1; kt < KT; ++kt) stage(s++, kt, std::false_type{}, q > 0, tm, tn, q);
        if (KT < C::P) {
            // the scale load is otherwise covered by the waits of stages 2+
            wait_vmcnt<0>();
            workgroup_barrier();
        }
        epilogue(q, tm, tn, u / tiles);
    }
    wait_vmcnt<0>();   // no LDS load may land after the workgroup retires
#endif  // __HIP_DEVICE_COMPILE__
}

// Sum of the ksplit int32 partials [ksplit][M][N] and the dequant epilogue of
// gemm_blk_kernel, bit for bit: y = bf16(fl(fl(f32(acc) * sx[m]) * sw[n])),
// then + bias[n] and + residual[m, n] in that order when present.  One thread
// per 8 consecutive outputs of a row (N % 16 == 0).
template <bool EXTRA>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const int32_t* __restrict__ part, int ksplit, int M,
                                                            int N, const float* __restrict__ sx,
                                                            const float* __restrict__ sw, EpiExtra ex,
                                                            uint16_t* __restrict__ y)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int n8 = N >> 3;
    if (i >= (int64_t)M * n8) return;
    const int m = (int)(i / n8), n0 = (int)(i % n8) * 8;
    int a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int s = 0; s < ksplit; ++s) {
        const int4* p = reinterpret_cast<const int4*>(part + ((int64_t)s * M + m) * N + n0);
        const int4 u = p[0], v = p[1];
        a[0] += u.x; a[1] += u.y; a[2] += u.z; a[3] += u.w;
        a[4] += v.x; a[5] += v.y; a[6] += v.z; a[7] += v.w;
    }
    const float xs = sx[m];
    const float4 w0 = *reinterpret_cast<const float4*>(sw + n0), w1 = *reinterpret_cast<const float4*>(sw + n0 + 4);
    const float ws[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = ((float)a[e] * xs) * ws[e];
    if constexpr (EXTRA) {
        if (ex.bias != nullptr) {
            const float4 b0 = *reinterpret_cast<const float4*>(ex.bias + n0);
            const float4 b1 = *reinterpret_cast<const float4*>(ex.bias + n0 + 4);
            const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = v[e] + bb[e];
        }
        if (ex.res != nullptr) {
            const uint2* rp = reinterpret_cast<const uint2*>(ex.res + (int64_t)m * N + n0);
            const uint2 r0 = rp[0], r1 = rp[1];
            const uint32_t rw[4] = {r0.x, r0.y, r1.x, r1.y};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[2 * e] = v[2 * e] + bf16_lo(rw[e]);
                v[2 * e + 1] = v[2 * e + 1] + bf16_hi(rw[e]);
            }
        }
    }
    *reinterpret_cast<uint4*>(y + (int64_t)m * N + n0) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

template <int BM, int BN, bool I32, bool EXTRA, bool A16, int KSL = 1>
hipError_t launch(const void* xq, const float* sx, const int8_t* wq, const float* sw, int M, int N,
                  int K, void* out, int num_cu, hipStream_t st, EpiExtra ex, int ksplit = 1)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles = tiles_m * tiles_n * ksplit;   // work units
    // LDS per workgroup: the stage ring and two scale buffers; 160 KB per CU.
    using C = Cfg<BM, BN, A16, KSL>;
    const int lds = C::NBUF * C::STAGE + (EXTRA ? 6144 : 4096);
    const int per_cu = (160 * 1024) / lds >= 2 ? 2 : 1;
    const int slots = num_cu * per_cu;
    const int grid = tiles < slots ? tiles : slots;
    const int group_m = tiles_m < 4 ? tiles_m : 4;
    const int m_rows = (M + 255) / 256 * 256;
    const int n_rows = (N + 255) / 256 * 256;
    hipLaunchKernelGGL((gemm_blk_kernel<BM, BN, I32, EXTRA, A16, KSL>), dim3(grid), dim3(256), 0, st,
                       static_cast<const int8_t*>(xq), sx, wq, sw, M, N, K, m_rows, n_rows, out, tiles_m,
                       tiles_n, group_m, ex, ksplit);
    return hipGetLastError();
}

// Split-K GEMM: the int32 partials into `part` ([ksplit][M][N]), then the
// reduction with the epilogue into y.
template <int BM, int BN, int KSL>
hipError_t launch_splitk(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, int M, int N, int K,
                         uint16_t* y, int num_cu, hipStream_t st, EpiExtra ex, int ksplit, int32_t* part)
{
    hipError_t e = launch<BM, BN, true, false, false, KSL>(xq, nullptr, wq, nullptr, M, N, K, part, num_cu, st,
                                                           EpiExtra{}, ksplit);
    if (e != hipSuccess) return e;
    const int64_t threads = (int64_t)M * (N / 8);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (ex.bias || ex.res)
        hipLaunchKernelGGL(splitk_reduce_kernel<true>, grid, dim3(256), 0, st, part, ksplit, M, N, sx, sw, ex, y);
    else
        hipLaunchKernelGGL(splitk_reduce_kernel<false>, grid, dim3(256), 0, st, part, ksplit, M, N, sx, sw, ex, y);
    return hipGetLastError();
}

}  // namespace blk

// Tile shapes for the blocked-layout GEMM.  `eff` is the relative per-CU MFMA
// efficiency of the shape; the choice minimises rounds * tile area * per_cu /
// eff, where a round is one tile per workgroup slot and per_cu workgroups
// share a CU.  The efficiencies are measured (MI355X, random INT8 data):
// 4096^3 takes 62 us with 256 x 256 tiles, 69 us with 128 x 128, 90 us with
// 64 x 128.  128 x 256 and 256 x 128 tiles (two workgroups per CU, 3-slot
// rings) measured no faster than these (c5 gate_up 295-311 us vs 300 us for
// 256 x 256; c5 down 152 us vs 128 us for 256 x 192).  The W8A16 variant uses
// the same table.
namespace {

int choose_shape(int64_t m, int64_t n, int num_cu)
{
    struct Shape {
        int bm, bn, per_cu;
        double eff;
    };
    static constexpr Shape shapes[] = {
        {128, 128, 2, 0.90}, {64, 128, 2, 0.70}, {256, 256, 1, 1.00}, {256, 192, 1, 0.97},
    };
    int best = 0;
    double best_t = 0;
    for (int c = 0; c < 4; ++c) {
        const int64_t tiles = ((m + shapes[c].bm - 1) / shapes[c].bm) * ((n + shapes[c].bn - 1) / shapes[c].bn);
        const int64_t slots = (int64_t)num_cu * shapes[c].per_cu;
        const int64_t rounds = (tiles + slots - 1) / slots;
        const double t = (double)rounds * shapes[c].bm * shapes[c].bn * shapes[c].per_cu / shapes[c].eff;
        if (best_t == 0 || t < best_t) {
            best = c;
            best_t = t;
        }
    }
    return best;
}

// Few tiles: a GEMM whose tiles number at most one per CU runs as a single
// round, and its time is the per-stage fixed cost (barrier, waits, LDS read
// latency) times the stage count.  Such GEMMs take more k-slices per half
// stage (KSL), which cuts the count, and the smallest tile that still keeps
// to one per CU, which spreads the work over more CUs:
//   * 64 x 64 tiles at most one per CU: KSL = 4 (k % 256 == 0), else 2;
//   * else 64 x 128 tiles at most one per CU: KSL = 2;
//   * else 128 x 128 tiles at most one per CU: KSL = 2.
// Measured (MI355X, random operands, warm caches), INT8: 2048 x 1024 x 3072
// 12.3 -> 10.8 us (64 x 128, KSL 2); 1024 x 4096 x 4096, where 512 tiles of
// 64 x 128 would share CUs two by two, 23.8 us on those, 20.7 us on 128 x 128
// tiles with KSL = 2; 256 x 3072 x 12288 32.2 us on 64 x 128 tiles, 26.1 us
// with KSL = 2, 19.4 us on 64 x 64 tiles with KSL = 4 (20.4 with KSL = 2);
// 1024 x 1024 x 12288 33.5 -> 27.0 -> 20.9 us the same way.  64 x 64 tiles
// lose once they outnumber the CUs (512 x 3072 x 12288: 35.6 us against
// 28.4 us on 64 x 128).  W8A16: 27.4 -> 24.8 us and 50.4 -> 43.6 us on the
// first two shapes (64 x 128 and 128 x 128, KSL 2), 256 x 3072 x 12288
// 76.9 -> 48.5 us and 1024 x 1024 x 12288 77.2 -> 48.8 us going from 64 x 128
// to 64 x 64 tiles.  Deeper rings (5 or 6 slots) and KSL = 4 on 64 x 128
// measured slower.
struct FewTiles {
    int shape;   // index as in choose_shape, 4 for 64 x 64; -1: not a few-tile GEMM
    int ksl;
};

FewTiles few_tile_shape(int64_t m, int64_t n, int64_t k, int num_cu)
{
    if (k % 128 != 0) return {-1, 1};
    const int64_t tm64 = (m + 63) / 64, tm128 = (m + 127) / 128;
    const int64_t tn64 = (n + 63) / 64, tn128 = (n + 127) / 128;
    if (tm64 * tn64 <= num_cu) return {4, k % 256 == 0 ? 4 : 2};
    if (tm64 * tn128 <= num_cu) return {1, 2};
    if (tm128 * tn128 <= num_cu) return {0, 2};
    return {-1, 1};
}

// Split K for few-tile GEMMs (INT8, with a workspace for the int32 partials).
// Few tiles leave each CU streaming (BM + BN) K operand bytes for one tile; k
// split s ways over s times the units cuts that to (BM + BN) K / s per CU at
// the price of the partials (s M N int32, written and read once more).  The
// estimate per plan: the unit's operand bytes at ~100 GB/s (one CU's L2 -> LDS
// stream) plus 2 s M N 4 bytes at ~5 TB/s; a plan is taken when it beats the
// unsplit tiles by 5%, or, for 48..128 rows at k >= 8192, instead of the
// weight-streaming kernel.  Measured on whole ck_int8_linear calls (quantizer
// included; single calls after a MALL flush, one box), unsplit -> split:
// 64 x 12288 -> 4096 25.0 -> 21.5 us, 128 x 12288 -> 4096 33.2 -> 26.4 us,
// 64 x 12288 -> 8192 38.7 -> 29.2 us, 48 x 12288 -> 3072 21.6 -> 20.2 us,
// 256 x 12288 -> 3072 37.2 -> 32.5 us, 1024 x 12288 -> 1024 42.1 -> 38.8 us,
// 128 x 8192 -> 4096 24.2 -> 21.4 us; at 33 rows even (21.4 / 21.6 us), and
// at k = 4096 every split was slower.
constexpr int64_t kSplitMinM = 48;
constexpr int64_t kSplitMinK = 8192;
constexpr int64_t kSplitMinKU = 1536;   // smallest k per unit

struct SplitPlan {
    int shape, ksl, s;   // shape as in choose_shape (4 = 64 x 64); s == 1: no split
};

SplitPlan splitk_plan(int64_t m, int64_t n, int64_t k, int num_cu)
{
    SplitPlan none{-1, 1, 1};
    if (m < kSplitMinM || k < kSplitMinK || n % 16 != 0) return none;
    struct Opt {
        int shape, bm, bn, ksl;
    };
    static constexpr Opt opts[] = {{4, 64, 64, 4}, {1, 64, 128, 2}, {0, 128, 128, 2}};
    auto tiles_of = [&](int bm, int bn) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
    SplitPlan best = none;
    double best_c = 0;
    for (const Opt& o : opts) {
        for (int sp = 2; sp <= 16; sp *= 2) {
            const int64_t ku = k / sp;
            if (k % sp || ku % (64 * o.ksl) || ku < kSplitMinKU || tiles_of(o.bm, o.bn) * sp > num_cu) continue;
            const double c = (double)(o.bm + o.bn) * ku / 1e5 + 2.0 * sp * m * n * 4 / 5e6;
            if (best.s == 1 || c < best_c) {
                best = {o.shape, o.ksl, sp};
                best_c = c;
            }
        }
    }
    if (best.s == 1) return none;
    if (use_small_kernel(m, n)) return best;   // 33..128 rows: the split tiles beat the weight stream
    const FewTiles few = few_tile_shape(m, n, k, num_cu);
    if (few.shape < 0) return none;            // enough tiles for every CU
    const int bm = few.shape == 0 ? 128 : 64, bn = few.shape == 4 ? 64 : 128;
    return best_c < 0.95 * (double)(bm + bn) * k / 1e5 ? best : none;
}

template <bool A16>
hipError_t launch_shape(const void* xq, const float* sx, const int8_t* wq, const float* sw, int64_t m,
                        int64_t n, int64_t k, void* out, bool out_raw, int num_cu, hipStream_t st,
                        EpiExtra ex)
{
    const int M = (int)m, N = (int)n, K = (int)k;
    const FewTiles few = few_tile_shape(m, n, k, num_cu);
    const int ksl = few.ksl;
    const int shape = few.shape >= 0 ? few.shape : choose_shape(m, n, num_cu);
#define CK_BLK(BM_, BN_, KSL_)                                                                         \
    return out_raw                                                                                      \
               ? blk::launch<BM_, BN_, true, false, A16, KSL_>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex) \
           : (ex.bias || ex.res)                                                                        \
               ? blk::launch<BM_, BN_, false, true, A16, KSL_>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex) \
               : blk::launch<BM_, BN_, false, false, A16, KSL_>(xq, sx, wq, sw, M, N, K, out, num_cu, st, ex)
    switch (shape) {
        case 0:
            if (ksl == 2) CK_BLK(128, 128, 2);
            CK_BLK(128, 128, 1);
        case 1:
            if (ksl == 2) CK_BLK(64, 128, 2);
            CK_BLK(64, 128, 1);
        case 4:
            if (ksl == 4) CK_BLK(64, 64, 4);
            CK_BLK(64, 64, 2);
        case 2: CK_BLK(256, 256, 1);
        default: CK_BLK(256, 192, 1);
    }
#undef CK_BLK
}

}  // namespace

hipError_t launch_gemm_blk(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                           int64_t m, int64_t n, int64_t k, void* out, bool out_i32, int num_cu,
                           hipStream_t st, EpiExtra ex)
{
    return launch_shape<false>(xq, sx, wq, sw, m, n, k, out, out_i32, num_cu, st, ex);
}

size_t gemm_splitk_bytes(int64_t m, int64_t n, int64_t k)
{
    const SplitPlan p = splitk_plan(m, n, k, num_cus());
    return p.s > 1 ? (size_t)p.s * (size_t)m * (size_t)n * 4 : 0;
}

bool launch_gemm_blk_splitk(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, int64_t m,
                            int64_t n, int64_t k, uint16_t* y, hipStream_t st, EpiExtra ex, void* ws,
                            size_t ws_bytes, hipError_t* err)
{
    const int num_cu = num_cus();
    const SplitPlan p = splitk_plan(m, n, k, num_cu);
    if (p.s == 1 || ws == nullptr || ws_bytes < (size_t)p.s * (size_t)m * (size_t)n * 4) return false;
    int32_t* part = static_cast<int32_t*>(ws);
    const int M = (int)m, N = (int)n, K = (int)k;
    switch (p.shape) {
        case 4: *err = blk::launch_splitk<64, 64, 4>(xq, sx, wq, sw, M, N, K, y, num_cu, st, ex, p.s, part); break;
        case 1: *err = blk::launch_splitk<64, 128, 2>(xq, sx, wq, sw, M, N, K, y, num_cu, st, ex, p.s, part); break;
        default: *err = blk::launch_splitk<128, 128, 2>(xq, sx, wq, sw, M, N, K, y, num_cu, st, ex, p.s, part); break;
    }
    return true;
}

hipError_t launch_gemm_w8a16(const uint16_t* x_rot, const int8_t* wq, const float* sw, int64_t m,
                             int64_t n, int64_t k, void* out, bool out_f32, hipStream_t st, EpiExtra ex)
{
    if (use_small_kernel(m, n)) return launch_gemm_small_w8a16(x_rot, wq, sw, m, n, k, out, out_f32, st, ex);
    return launch_shape<true>(x_rot, nullptr, wq, sw, m, n, k, out, out_f32, num_cus(), st, ex);
}

}  // namespace ck
