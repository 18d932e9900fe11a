// ck_device.hpp -- device-side building blocks of the ConvRot quantizer for
// gfx950: BF16 unpacking, the FP32 silu, the blockwise Hadamard butterflies and
// the INT8 code packing.  Every floating-point step is one IEEE binary32
// operation in round-to-nearest-even; the translation units that include this
// file are compiled with -ffp-contract=off, and fused multiply-adds appear only
// where written as __builtin_fmaf.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ck {

// ---------------------------------------------------------------------------
// BF16 <-> FP32 (a BF16 value is the high half of an FP32 bit pattern)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even FP32 -> BF16 for finite values.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Optional terms of a linear layer's epilogue (either pointer may be null):
// bias is F32 [N]; res is a BF16 [M, N] row-major residual, which may be the
// output buffer itself.  comfy-kitchen PR #277, "Changes" (the INT8 linear is
// tested with bias and residual) and PR #248's commit list (residuals fused
// into the kernels); the FP32 order is a reading: one FP32 sum, then one BF16
// rounding, t = fl(fl(t + bias[n]) + f32(res[m, n])).
struct EpiExtra {
    const float* bias;
    const uint16_t* res;
};

// Adds the optional terms to the four consecutive outputs (m, n .. n + 3).
// n % 4 == 0; m must be a valid row (callers clamp padding rows, whose stores
// are dropped).
__device__ __forceinline__ void epi_extra4(float& y0, float& y1, float& y2, float& y3,
                                           const EpiExtra& e, int m, int n, int N)
{
    if (e.bias) {
        const float4 b = *reinterpret_cast<const float4*>(e.bias + n);
        y0 = y0 + b.x;
        y1 = y1 + b.y;
        y2 = y2 + b.z;
        y3 = y3 + b.w;
    }
    if (e.res) {
        const uint2 r = *reinterpret_cast<const uint2*>(e.res + (int64_t)m * N + n);
        y0 = y0 + bf16_lo(r.x);
        y1 = y1 + bf16_hi(r.x);
        y2 = y2 + bf16_lo(r.y);
        y3 = y3 + bf16_hi(r.y);
    }
}

// Buffer-resource offset past the end of every buffer the kernels address: a
// buffer load there returns zeros and a buffer store there is dropped, so
// lanes with nothing to load or store still issue the same instructions.
constexpr uint32_t kBufferOutside = 0x80000000u;

// 8 INT8 weight codes (two dwords) -> 8 BF16 values, exact (|q| <= 127 has 7
// significant bits): one v_cvt_f32_i32 (byte select, sign-extended) per value
// and one v_cvt_pk_bf16_f32 per pair.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8_t widen8(int lo, int hi)
{
    bf16x8_t r;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int w = e < 4 ? lo : hi;
        r[e] = (__bf16)(float)(int)(signed char)(w >> (8 * (e & 3)));
    }
    return r;
}

// Two FP32 values -> packed BF16 pair (lo = a, hi = b), round-to-nearest-even:
// one v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// A rotated pair as BF16: bf16(fl(a * c) + 0), bf16(fl(b * c) + 0).  Adding
// +0 changes no value and writes an exact zero as +0, so the sign of a zero
// does not depend on the butterfly form (the sign-folded butterflies hold a
// cancelled value as +0 where the plain ones hold -0, and the reverse).
__device__ __forceinline__ uint32_t rot_bf16x2(float a, float b, float c)
{
    return pack_bf16x2(a * c + 0.0f, b * c + 0.0f);
}

// ---------------------------------------------------------------------------
// FP32 silu.  sglang PR #44196, "Accuracy Tests": the fused quantizer keeps
// silu(gate) * up in FP32.  The evaluation procedure is fixed so the result is
// reproducible bit for bit:
//   gl = max(gamma, -80), gc = min(gl, 80)
//   e^{-gc}: k = rint(fl(-gc * log2e)); r = fma(k, -ln2_hi, -gc);
//            r = fma(k, -ln2_lo, r); p = Taylor series of e^r to degree 7
//            (Horner, fma); e = p * 2^k  (Cody-Waite range reduction)
//   1/d, d = 1 + e: seed from the bit pattern (magic - bits(d)), then three
//            Newton steps  t = fma(-d, y, 1); y = fma(y, t, y)
//   silu = gl * y
// Constants: log2e = fl(log2 e); ln2_hi = ln 2 rounded to 16 significant bits
// (so k * ln2_hi is exact for |k| <= 116); ln2_lo = fl(ln 2 - ln2_hi);
// Taylor coefficients fl(1/n!); the seed constant minimises the seed's maximum
// relative error (5.05%) over a binade.
// ---------------------------------------------------------------------------
// y = 1 / (1 + e^{-gc}) by the procedure above, for the clamped gate gc.
__device__ __forceinline__ float silu_sigma(float gc)
{
    constexpr float kNegLog2e = -0x1.715476p+0f;
    constexpr float kLn2Hi = 0x1.62e4p-1f;
    constexpr float kLn2Lo = 0x1.7f7d1cp-20f;
    constexpr uint32_t kRcpMagic = 0x7ef311c2u;
    const float kf = __builtin_rintf(gc * kNegLog2e);
    float r = __builtin_fmaf(kf, -kLn2Hi, -gc);
    r = __builtin_fmaf(kf, -kLn2Lo, r);
    float p = 0x1.a01a02p-13f;                    // 1/7!
    p = __builtin_fmaf(p, r, 0x1.6c16c2p-10f);    // 1/6!
    p = __builtin_fmaf(p, r, 0x1.111112p-7f);     // 1/5!
    p = __builtin_fmaf(p, r, 0x1.555556p-5f);     // 1/4!
    p = __builtin_fmaf(p, r, 0x1.555556p-3f);     // 1/3!
    p = __builtin_fmaf(p, r, 0x1p-1f);            // 1/2!
    p = __builtin_fmaf(p, r, 1.0f);               // 1/1!
    p = __builtin_fmaf(p, r, 1.0f);               // 1/0!
    const float e = __builtin_amdgcn_ldexpf(p, (int)kf);
    const float d = 1.0f + e;
    float y = __uint_as_float(kRcpMagic - __float_as_uint(d));
#pragma unroll
    for (int it = 0; it < 3; ++it) {
        const float t = __builtin_fmaf(-d, y, 1.0f);
        y = __builtin_fmaf(y, t, y);
    }
    return y;
}

// max(gamma, -80) of a gate given as its FP32 bit pattern.  As unsigned
// integers the patterns of all values at or above -80 (the non-negative ones,
// sign bit clear, and the negatives down to -80 = 0xC2A00000) lie below those
// of the values under -80, so an unsigned min with -80's pattern is the clamp,
// bit for bit, for every gate that is not a NaN.  (fmaxf on a float that the
// compiler got from a reinterpreted word is one canonicalizing max(x, x) more.)
__device__ __forceinline__ float gate_clamp(uint32_t bits)
{
    return __uint_as_float(min(bits, 0xC2A00000u));
}

// silu_f32 of the gate with FP32 bit pattern `bits`: gl = max(gamma, -80) as
// gate_clamp, gc = min(gl, 80) as a signed integer min (FP32 patterns of
// non-negative values order as signed integers, and every negative pattern is
// a negative integer, below 80's), then gl * silu_sigma(gc).
__device__ __forceinline__ float silu_f32(uint32_t bits)
{
    const uint32_t gl = min(bits, 0xC2A00000u);
    const int gc = min((int)gl, 0x42A00000);
    return __uint_as_float(gl) * silu_sigma(__int_as_float(gc));
}

// ---------------------------------------------------------------------------
// silu of BF16 gates through a table of silu_sigma.  A gate is a BF16 value,
// and silu_sigma depends only on gc = min(max(gamma, -80), 80): it is exactly 1
// for every gamma >= 17 (1 + e^{-gamma} rounds to 1 and the reciprocal of 1 is
// 1), and constant below -80.  It is also one constant for every |gamma| <=
// 2^-25: there kf = 0 and r = -gc, the polynomial's last two steps round
// 1 + r/2 and 1 + r to exactly 1 (|r| is at most half an ulp of 1), so e = 1,
// d = 2, and the Newton steps see the same operands for every such gate.  So
// the BF16 patterns of magnitude from that of 2^-30 (0x3080, well inside the
// constant range) to that of 80.0 (0x42A0), with either sign, cover every
// value, and
//   silu(gamma) = fl(max(gamma, -80) * T[2 (med3(|bits|, 0x3080, 0x42A0) - 0x3080) + sign])
// is silu_f32(gamma) bit for bit (the same two clamps and the same product).
// T has 2 * (0x42A0 - 0x3080 + 1) FP32 entries (37,128 bytes), and a lookup
// costs a few integer ops instead of the ~20 FP32 ops of silu_sigma.
// ---------------------------------------------------------------------------
constexpr int kSiluTabMag = 0x42A0;                      // bits of 80.0f >> 16
constexpr int kSiluTabLow = 0x3080;                      // bits of 2^-30 >> 16
constexpr int kSiluTabEntries = 2 * (kSiluTabMag - kSiluTabLow + 1);

// Entry i of the table: silu_sigma of the BF16 gate with magnitude bits
// kSiluTabLow + i / 2 and sign i % 2, clamped as silu_f32 clamps it.
__device__ __forceinline__ float silu_tab_entry(int i)
{
    const uint32_t bits = ((uint32_t)(i & 1) << 31) | ((uint32_t)(kSiluTabLow + (i >> 1)) << 16);
    const float gamma = __uint_as_float(bits);
    return silu_sigma(fminf(fmaxf(gamma, -80.0f), 80.0f));
}

// Byte offset of the entry for the 16-bit gate pattern held in bits 0..15
// (HI = false) or 16..31 (HI = true) of w, biased by kSiluTabBias: it is added
// to the table's address minus kSiluTabBias (the bias has zero low bits, so
// ((mag - low) << 3) | sign = ((mag << 3) | sign) - bias).  (mag << 3) | (sign
// << 2) is one alignbit of the clamped magnitude over the gate's FP32 pattern
// (whose bit 31, the sign, lands on bit 2; the two bits below it are masked
// off), the pattern the caller also clamps: four ops per gate with the med3.
constexpr uint32_t kSiluTabBias = (uint32_t)kSiluTabLow << 3;

template <bool HI>
__device__ __forceinline__ uint32_t silu_tab_offset(uint32_t w)
{
    const uint32_t f = HI ? (w & 0xffff0000u) : (w << 16);          // the gate's FP32 pattern
    const uint32_t b = HI ? (w >> 16) & 0x7fffu : w & 0x7fffu;      // its magnitude bits
    const uint32_t mag = min(max(b, (uint32_t)kSiluTabLow), (uint32_t)kSiluTabMag);
    return __builtin_amdgcn_alignbit(mag, f, 29) & 0x3fffcu;
}

// ---------------------------------------------------------------------------
// Blockwise Hadamard rotation.  comfy-kitchen PR #277, "The key observation":
// the activation is rotated online, x_rot = x H.  The transform is applied
// unnormalised as a fast Walsh-Hadamard transform with strides 1, 2, 4, ...
// in ascending order; a butterfly maps (p, q) at (i, i+h) to (p+q, p-q).
//
// Register layout: a lane holds 8 consecutive elements of a row (one 16-byte
// BF16 load), so strides 1, 2 and 4 stay inside the lane; stride 8*d pairs the
// lane with lane ^ d.  The partner's value comes through ds_swizzle (the LDS
// crossbar, no VALU slot) and the butterfly is one fma per element:
//   lower lane: v + partner = fma(v, +1, partner)
//   upper lane: partner - v = fma(v, -1, partner)
// both exact equivalents of the IEEE add/subtract.
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ void fwht_in_lane(float (&v)[8])
{
#pragma unroll
    for (int h = 1; h < 8 && h < G; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & h) == 0) {
                const float p = v[i], q = v[i + h];
                v[i] = p + q;
                v[i + h] = p - q;
            }
        }
    }
}

// ds_swizzle in bit-mask mode: lane l reads lane ((l & 0x1f) ^ D) within its
// group of 32 lanes.
template <int D>
__device__ __forceinline__ float swizzle_xor(float v)
{
    static_assert(D >= 1 && D <= 16, "swizzle xor distance");
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (D << 10) | 0x1f));
}

// The same exchange for D = 1 or 2 through a DPP quad permutation (a VALU
// move within each group of 4 lanes): no LDS traffic, one more VALU op.  Used
// for reductions (the butterflies fuse the move, fwht_cross_lane_signed).
template <int D>
__device__ __forceinline__ float dpp_xor(float v)
{
    static_assert(D == 1 || D == 2, "quad permutation distance");
    constexpr int ctrl = D == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), ctrl, 0xf, 0xf, false));
}

// Cross-lane strides 8 .. G/2.  `lane` is the lane's position in its row team
// (teams are aligned to the group size).
template <int G>
__device__ __forceinline__ void fwht_cross_lane(float (&v)[8], int lane)
{
    if constexpr (G >= 16) {
        const float s = (lane & 1) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], s, swizzle_xor<1>(v[i]));
    }
    if constexpr (G >= 32) {
        const float s = (lane & 2) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], s, swizzle_xor<2>(v[i]));
    }
    if constexpr (G >= 64) {
        const float s = (lane & 4) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], s, swizzle_xor<4>(v[i]));
    }
    if constexpr (G >= 128) {
        const float s = (lane & 8) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], s, swizzle_xor<8>(v[i]));
    }
    if constexpr (G >= 256) {
        const float s = (lane & 16) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], s, swizzle_xor<16>(v[i]));
    }
}

// Cross-lane strides 8 .. G/2 with the exchanges with lanes 1, 2 and 8 apart
// folded into the butterfly: v_fmac_f32 with a DPP lane permutation (quad
// permutations, a rotation by 8 within the 16-lane row) on its first operand
// computes partner * t + own in one VALU op (the move-then-fma form above
// takes two, and the compiler does not fold the move into an FMA).  With the
// partner in the multiplied operand the upper lane gets q - p = -(p - q)
// instead of p - q, so the lane's values come out as sigma * (the true value)
// with sigma = the product of those stages' t = (-1)^(bits 0, 1 and 3 of the
// lane's position), which the function returns: both are exact (t = +-1
// makes the product exact, the
// FMA rounds the sum once, and a negation is exact), and the later
// exchanges pair lanes with equal sigma, where the usual form keeps it.  The
// caller folds sigma into what it multiplies the values by (the code
// multiplier r: u * r = (sigma u) * (sigma r) exactly) and takes |u| for the
// absmax.  `lane`: the lane's position in its row team (aligned to G / 8).
template <int CTRL>
__device__ __forceinline__ void fmac_dpp8(float (&v)[8], float t)
{
    // s_nop 1: two wait states between a VALU write of a register and a DPP
    // read of it; inside the block no op reads a register the op before it
    // wrote.
    if constexpr (CTRL == 0x128) {   // row_ror:8: lane l <- lane l ^ 8 within each row of 16
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %0, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, %1, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, %2, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %3, %3, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %4, %4, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %5, %5, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %6, %6, %8 row_ror:8 row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %7, %7, %8 row_ror:8 row_mask:0xf bank_mask:0xf"
            : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
            : "v"(t));
    } else if constexpr (CTRL == 0xB1) {
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %0, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, %1, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, %2, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %3, %3, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %4, %4, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %5, %5, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %6, %6, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %7, %7, %8 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
            : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
            : "v"(t));
    } else {
        static_assert(CTRL == 0x4E, "quad permutation xor 1 or xor 2, or row rotation xor 8");
        asm("s_nop 1\n\t"
            "v_fmac_f32_dpp %0, %0, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %1, %1, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %2, %2, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %3, %3, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %4, %4, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %5, %5, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %6, %6, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
            "v_fmac_f32_dpp %7, %7, %8 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
            : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]), "+v"(v[7])
            : "v"(t));
    }
}

template <int G>
__device__ __forceinline__ float fwht_cross_lane_signed(float (&v)[8], int lane)
{
    static_assert(G >= 32, "two quad-permutation stages");
    const float t0 = (lane & 1) ? -1.0f : 1.0f;
    const float t1 = (lane & 2) ? -1.0f : 1.0f;
    fmac_dpp8<0xB1>(v, t0);
    fmac_dpp8<0x4E>(v, t1);
    if constexpr (G >= 64) {
        const float s = (lane & 4) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], s, swizzle_xor<4>(v[i]));
    }
    float sigma = t0 * t1;
    if constexpr (G >= 128) {   // lane ^ 8 is a rotation by 8 within the 16-lane row: fused the same way
        const float t3 = (lane & 8) ? -1.0f : 1.0f;
        fmac_dpp8<0x128>(v, t3);
        sigma *= t3;
    }
    if constexpr (G >= 256) {
        const float s = (lane & 16) ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = __builtin_fmaf(v[i], s, swizzle_xor<16>(v[i]));
    }
    return sigma;
}

// ---------------------------------------------------------------------------
// INT8 codes.  code = round-half-even(u * r) of the exact product: fma(u, r,
// 1.5 * 2^23) rounds u*r + 1.5*2^23 once to an integer (|u*r| <= 127 + 2^-16,
// far inside the range where FP32 spacing is 1), and the low byte of its bit
// pattern is the two's-complement code.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t code_bits(float u, float r)
{
    return __float_as_uint(__builtin_fmaf(u, r, 12582912.0f));
}

// Pack the low bytes of four code words into one dword (v_perm_b32).
__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3)
{
    const uint32_t lo = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);
    return lo | hi;
}

}  // namespace ck
