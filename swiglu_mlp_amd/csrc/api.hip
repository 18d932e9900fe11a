// api.hip -- the C ABI declared in include/ck.h: host-side argument checks,
// workspace carving and kernel dispatch.  No function here allocates, frees or
// synchronises; all checks complete before anything is enqueued.
#include "ck.h"
#include "ck_internal.hpp"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool pow2_group(int32_t g) { return g >= 1 && g <= 256 && (g & (g - 1)) == 0; }

// Checks shared by every call that takes an in_features dimension.
ck_status check_k(int64_t k, int32_t group)
{
    if (!pow2_group(group)) return CK_EUNSUPPORTED;
    if (k < 1) return CK_ESHAPE;
    if (k > CK_MAX_K) return CK_EUNSUPPORTED;
    if (k % 64 != 0 || k % group != 0) return CK_ESHAPE;
    return CK_OK;
}

ck_status check_act(int32_t act, int64_t ldx, int64_t k)
{
    if (act != CK_ACT_NONE && act != CK_ACT_SWIGLU) return CK_EINVAL;
    const int64_t need = act == CK_ACT_SWIGLU ? 2 * k : k;
    if (ldx < need || ldx % 8 != 0) return CK_ESHAPE;
    return CK_OK;
}

ck_status from_hip(hipError_t e) { return e == hipSuccess ? CK_OK : CK_EHIP; }

int64_t pad_rows(int64_t r) { return (r + 255) / 256 * 256; }

// Layout of activation codes: row-major or blocked.
ck_status check_layout(int32_t layout)
{
    return (layout == CK_LAYOUT_ROWS || layout == CK_LAYOUT_BLOCKED) ? CK_OK : CK_EINVAL;
}

// Layout of a GEMM's weight (the activation codes are then row-major for
// CK_LAYOUT_ROWS and blocked otherwise).  The decode layout serves m <= 64.
ck_status check_weight_layout(int32_t layout, int64_t m)
{
    if (layout == CK_LAYOUT_ROWS || layout == CK_LAYOUT_BLOCKED) return CK_OK;
    if (layout != CK_LAYOUT_DECODE) return CK_EINVAL;
    return m <= ck::kDecodeMaxM ? CK_OK : CK_EUNSUPPORTED;
}

// Bytes of the decode layout of [n, k] (n % 16 == 0).
int64_t decode_bytes(int64_t n, int64_t k) { return (n / 16) * (64 + 16 * k); }

// Every int8 operand and output of the GEMM kernels is addressed with 32-bit
// byte offsets (buffer resources).
ck_status check_gemm_extent(int64_t m, int64_t n, int64_t k)
{
    if (pad_rows(m) * k > CK_MAX_ELEMS || pad_rows(n) * k > CK_MAX_ELEMS ||
        pad_rows(m) * n * 4 > CK_MAX_ELEMS || decode_bytes(n, k) > CK_MAX_ELEMS)
        return CK_EUNSUPPORTED;
    return CK_OK;
}

#define CK_TRY(expr)                     \
    do {                                 \
        const ck_status st_ = (expr);    \
        if (st_ != CK_OK) return st_;    \
    } while (0)

// Scratch of ck_int8_linear_noalloc: the activation codes and row scales of
// one call, in device memory the library holds itself (each GPU gets its own
// copy when the library's code is loaded on it, kept until the process ends).
// Host code never uses the array's name as an address: on the host it is only
// a stand-in, and a kernel given it would fault.  The device address comes
// from hipGetSymbolAddress, once per device with that device current.
constexpr size_t kNoAllocScratchBytes = CK_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch size");
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

ck_status scratch_of_current_device(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return CK_EHIP;
    if (dev < 0 || dev >= kMaxDevices) return CK_EUNSUPPORTED;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return CK_EHIP;
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return CK_OK;
}

}  // namespace

extern "C" {

const char* ck_version(void) { return "ck-convrot 0.1 (gfx950)"; }

const char* ck_status_str(ck_status s)
{
    switch (s) {
        case CK_OK: return "ok";
        case CK_EINVAL: return "invalid argument (null or misaligned pointer, unknown act)";
        case CK_ESHAPE: return "bad shape (negative size, k % group, k % 64, n % 16, leading dimension)";
        case CK_EUNSUPPORTED: return "unsupported (group not a power of two <= 256, k > CK_MAX_K, a buffer past 2^31 bytes, or the decode layout with m > 64)";
        case CK_EWORKSPACE: return "workspace missing or too small";
        case CK_EHIP: return "HIP runtime error at launch";
    }
    return "unknown status";
}

ck_status ck_weight_prep(const float* w, int64_t n, int64_t k, int32_t group, int8_t* w_q,
                         float* w_scale, void* stream)
{
    CK_TRY(check_k(k, group));
    if (n < 0) return CK_ESHAPE;
    if (n == 0) return CK_OK;
    if (!w || !w_q || !w_scale) return CK_EINVAL;
    if (!aligned16(w) || !aligned16(w_q)) return CK_EINVAL;
    return from_hip(ck::launch_quant_rows(2, w, k, n, k, group, w_q, w_scale, nullptr, false,
                                          (hipStream_t)stream));
}

int64_t ck_blocked_rows(int64_t rows) { return rows <= 0 ? 0 : pad_rows(rows); }

size_t ck_blocked_size(int64_t rows, int64_t k)
{
    if (rows <= 0 || k <= 0) return 0;
    return (size_t)pad_rows(rows) * (size_t)k;
}

ck_status ck_weight_pack(const int8_t* w_q, int64_t n, int64_t k, int8_t* w_blk, void* stream)
{
    if (n < 0 || k < 1 || k % 64 != 0) return CK_ESHAPE;
    if (k > CK_MAX_K || pad_rows(n) * k > CK_MAX_ELEMS) return CK_EUNSUPPORTED;
    if (n == 0) return CK_OK;
    if (!w_q || !w_blk) return CK_EINVAL;
    if (!aligned16(w_q) || !aligned16(w_blk)) return CK_EINVAL;
    return from_hip(ck::launch_pack_blocked(w_q, n, k, w_blk, (hipStream_t)stream));
}

size_t ck_decode_size(int64_t n, int64_t k)
{
    if (n <= 0 || k <= 0) return 0;
    return (size_t)((n + 15) / 16) * (size_t)(64 + 16 * k);
}

ck_status ck_weight_pack_decode(const int8_t* w_q, const float* w_scale, int64_t n, int64_t k,
                                void* w_dec, void* stream)
{
    if (n < 0 || n % 16 != 0 || k < 1 || k % 64 != 0) return CK_ESHAPE;
    if (k > CK_MAX_K || decode_bytes(n, k) > CK_MAX_ELEMS) return CK_EUNSUPPORTED;
    if (n == 0) return CK_OK;
    if (!w_q || !w_scale || !w_dec) return CK_EINVAL;
    if (!aligned16(w_q) || !aligned16(w_scale) || !aligned16(w_dec)) return CK_EINVAL;
    return from_hip(ck::launch_pack_decode(w_q, w_scale, n, k, w_dec, (hipStream_t)stream));
}

ck_status ck_act_quant(const uint16_t* x, int64_t ldx, int64_t m, int64_t k, int32_t act,
                       int32_t group, int32_t layout, int8_t* x_q, float* x_scale, void* stream)
{
    CK_TRY(check_k(k, group));
    CK_TRY(check_act(act, ldx, k));
    CK_TRY(check_layout(layout));
    if (m < 0) return CK_ESHAPE;
    if (layout == CK_LAYOUT_BLOCKED && pad_rows(m) * k > CK_MAX_ELEMS) return CK_EUNSUPPORTED;
    if (m == 0) return CK_OK;
    if (!x || !x_q || !x_scale) return CK_EINVAL;
    if (!aligned16(x) || !aligned16(x_q)) return CK_EINVAL;
    return from_hip(ck::launch_quant_rows(act == CK_ACT_SWIGLU ? 1 : 0, x, ldx, m, k, group, x_q,
                                          x_scale, nullptr, layout == CK_LAYOUT_BLOCKED,
                                          (hipStream_t)stream));
}

// The codes and scales, sized for either layout (the blocked codes are the
// larger): what ck_int8_linear needs at least.
static size_t linear_codes_bytes(int64_t m, int64_t k)
{
    return round_up((size_t)pad_rows(m) * (size_t)k) + round_up((size_t)m * sizeof(float));
}

// The codes and scales, then room for the split-K partials of the GEMM when
// its shape takes them on this device.
size_t ck_int8_linear_workspace_size(int64_t m, int64_t k, int64_t n)
{
    if (m <= 0 || k <= 0 || n <= 0) return 0;
    return linear_codes_bytes(m, k) + round_up(ck::gemm_splitk_bytes(m, n, k));
}

static ck_status check_gemm_args(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                                 const float* w_scale, int32_t layout, int64_t m, int64_t n,
                                 int64_t k, const void* y, bool need_scales)
{
    CK_TRY(check_weight_layout(layout, m));
    if (layout == CK_LAYOUT_DECODE) w_scale = x_scale;   // the decode layout carries its own
    if (k < 1 || k % 64 != 0) return CK_ESHAPE;
    if (k > CK_MAX_K) return CK_EUNSUPPORTED;
    if (m < 0 || n < 0 || n % 16 != 0) return CK_ESHAPE;
    CK_TRY(check_gemm_extent(m, n, k));
    if (m == 0 || n == 0) return CK_OK;
    if (!x_q || !w_q || !y) return CK_EINVAL;
    if (need_scales && (!x_scale || !w_scale)) return CK_EINVAL;
    if (!aligned16(x_q) || !aligned16(w_q) || !aligned16(y)) return CK_EINVAL;
    if (need_scales && !aligned16(w_scale)) return CK_EINVAL;
    return CK_OK;
}

// Optional epilogue terms: bias is read as float4, the residual as 8-byte
// groups of 4 BF16 values.
static ck_status check_extra(const float* bias, const uint16_t* residual)
{
    if (bias && !aligned16(bias)) return CK_EINVAL;
    if (residual && ((uintptr_t)residual % 8) != 0) return CK_EINVAL;
    return CK_OK;
}

ck_status ck_int8_gemm_bf16(const int8_t* x_q, const float* x_scale, const int8_t* w_q,
                            const float* w_scale, const float* bias, const uint16_t* residual,
                            int32_t layout, int64_t m, int64_t n, int64_t k, uint16_t* y,
                            void* stream)
{
    CK_TRY(check_gemm_args(x_q, x_scale, w_q, w_scale, layout, m, n, k, y, true));
    if (m == 0 || n == 0) return CK_OK;
    CK_TRY(check_extra(bias, residual));
    return from_hip(ck::launch_gemm_bf16(x_q, x_scale, w_q, w_scale, m, n, k, y, layout,
                                         (hipStream_t)stream, ck::EpiExtra{bias, residual}));
}

ck_status ck_int8_gemm_i32(const int8_t* x_q, const int8_t* w_q, int32_t layout, int64_t m,
                           int64_t n, int64_t k, int32_t* acc, void* stream)
{
    CK_TRY(check_gemm_args(x_q, nullptr, w_q, nullptr, layout, m, n, k, acc, false));
    if (m == 0 || n == 0) return CK_OK;
    return from_hip(ck::launch_gemm_i32(x_q, w_q, m, n, k, acc, layout, (hipStream_t)stream));
}

// Argument checks of ck_int8_linear and its allocation-free variant (all but
// the workspace).  CK_OK with *noop set for an empty call.
static ck_status check_linear_args(const uint16_t* x, int64_t ldx, int32_t act, const int8_t* w_q,
                                   const float* w_scale, const float* bias, const uint16_t* residual,
                                   int32_t layout, int64_t m, int64_t n, int64_t k, int32_t group,
                                   const uint16_t* y, bool* noop)
{
    *noop = false;
    CK_TRY(check_k(k, group));
    CK_TRY(check_act(act, ldx, k));
    CK_TRY(check_weight_layout(layout, m));
    if (m < 0 || n < 0 || n % 16 != 0) return CK_ESHAPE;
    CK_TRY(check_gemm_extent(m, n, k));
    if (m == 0 || n == 0) {
        *noop = true;
        return CK_OK;
    }
    const bool dec = layout == CK_LAYOUT_DECODE;   // w_scale unused: the layout carries it
    if (!x || !w_q || (!w_scale && !dec) || !y) return CK_EINVAL;
    if (!aligned16(x) || !aligned16(w_q) || (!dec && !aligned16(w_scale)) || !aligned16(y))
        return CK_EINVAL;
    return check_extra(bias, residual);
}

// The linear after its checks: quantizer then GEMM, the codes and scales at
// the start of `workspace` (256-byte aligned, ws_bytes >=
// linear_codes_bytes(m, k)); the GEMM may use the rest for split-K partials.
static ck_status run_int8_linear(const uint16_t* x, int64_t ldx, int32_t act, const int8_t* w_q,
                                 const float* w_scale, const float* bias, const uint16_t* residual,
                                 int32_t layout, int64_t m, int64_t n, int64_t k, int32_t group,
                                 uint16_t* y, void* workspace, size_t ws_bytes, hipStream_t st)
{
    const bool dec = layout == CK_LAYOUT_DECODE;
    const bool blocked = layout != CK_LAYOUT_ROWS;
    int8_t* xq = static_cast<int8_t*>(workspace);
    float* sx = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                         round_up((size_t)pad_rows(m) * (size_t)k));
    const int kind = act == CK_ACT_SWIGLU ? 1 : 0;
    if (blocked && ck::use_fused_decode(kind, m, k, group))   // quantizer inside the GEMM: one launch
        return from_hip(ck::launch_gemm_dec_fused(kind, x, ldx, m, k, group, w_q, w_scale, dec, n, y, st,
                                                  ck::EpiExtra{bias, residual}));
    CK_TRY(from_hip(ck::launch_quant_rows(kind, x, ldx, m, k, group, xq, sx, nullptr, blocked, st)));
    const size_t used = linear_codes_bytes(m, k);
    return from_hip(ck::launch_gemm_bf16(xq, sx, w_q, w_scale, m, n, k, y, layout, st,
                                         ck::EpiExtra{bias, residual}, static_cast<char*>(workspace) + used,
                                         ws_bytes - used));
}

ck_status ck_int8_linear(const uint16_t* x, int64_t ldx, int32_t act, const int8_t* w_q,
                         const float* w_scale, const float* bias, const uint16_t* residual,
                         int32_t layout, int64_t m, int64_t n, int64_t k, int32_t group, uint16_t* y,
                         void* workspace, size_t workspace_bytes, void* stream)
{
    bool noop;
    CK_TRY(check_linear_args(x, ldx, act, w_q, w_scale, bias, residual, layout, m, n, k, group, y, &noop));
    if (noop) return CK_OK;
    if (!workspace || workspace_bytes < linear_codes_bytes(m, k) || ((uintptr_t)workspace % kAlign) != 0)
        return CK_EWORKSPACE;
    return run_int8_linear(x, ldx, act, w_q, w_scale, bias, residual, layout, m, n, k, group, y, workspace,
                           workspace_bytes, (hipStream_t)stream);
}

size_t ck_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

ck_status ck_int8_linear_noalloc(const uint16_t* x, int64_t ldx, int32_t act, const int8_t* w_q,
                                 const float* w_scale, const float* bias, const uint16_t* residual,
                                 int32_t layout, int64_t m, int64_t n, int64_t k, int32_t group,
                                 uint16_t* y, void* stream)
{
    bool noop;
    CK_TRY(check_linear_args(x, ldx, act, w_q, w_scale, bias, residual, layout, m, n, k, group, y, &noop));
    if (noop) return CK_OK;
    if (linear_codes_bytes(m, k) > kNoAllocScratchBytes) return CK_EWORKSPACE;
    void* ws = nullptr;
    CK_TRY(scratch_of_current_device(&ws));
    return run_int8_linear(x, ldx, act, w_q, w_scale, bias, residual, layout, m, n, k, group, y, ws,
                           kNoAllocScratchBytes, (hipStream_t)stream);
}

// Sized for either layout: x codes, x scales, the [m, 2i] BF16 gate|up
// output, its codes and scales (what ck_swiglu_mlp needs at least).
static size_t mlp_base_bytes(int64_t m, int64_t h, int64_t i)
{
    const size_t M = (size_t)m, MP = (size_t)pad_rows(m), H = (size_t)h, I = (size_t)i;
    return round_up(MP * H) + round_up(M * 4) + round_up(M * 2 * I * 2) + round_up(MP * I) + round_up(M * 4);
}

// The above, then room for the split-K partials of either GEMM (the two run
// one after the other on the stream and share it).
size_t ck_swiglu_mlp_workspace_size(int64_t m, int64_t h, int64_t i)
{
    if (m <= 0 || h <= 0 || i <= 0) return 0;
    const size_t part = std::max(ck::gemm_splitk_bytes(m, 2 * i, h), ck::gemm_splitk_bytes(m, h, i));
    return mlp_base_bytes(m, h, i) + round_up(part);
}

ck_status ck_swiglu_mlp(const uint16_t* x, const int8_t* w_gu, const float* s_gu,
                        const int8_t* w_down, const float* s_down, int32_t layout, int64_t m,
                        int64_t h, int64_t i, int32_t group, uint16_t* y, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    CK_TRY(check_k(h, group));   // stage 1 contracts over h
    CK_TRY(check_k(i, group));   // stage 2 contracts over i
    CK_TRY(check_weight_layout(layout, m));
    if (m < 0 || h % 16 != 0) return CK_ESHAPE;
    CK_TRY(check_gemm_extent(m, 2 * i, h));
    CK_TRY(check_gemm_extent(m, h, i));
    if (m == 0) return CK_OK;
    const bool dec = layout == CK_LAYOUT_DECODE;   // scales inside the weights
    if (!x || !w_gu || !w_down || !y || (!dec && (!s_gu || !s_down))) return CK_EINVAL;
    if (!aligned16(x) || !aligned16(w_gu) || !aligned16(w_down) || !aligned16(y) ||
        (!dec && (!aligned16(s_gu) || !aligned16(s_down))))
        return CK_EINVAL;
    const size_t base = mlp_base_bytes(m, h, i);
    if (!workspace || workspace_bytes < base || ((uintptr_t)workspace % kAlign) != 0)
        return CK_EWORKSPACE;
    const size_t M = (size_t)m, MP = (size_t)pad_rows(m), H = (size_t)h, I = (size_t)i;
    const bool blocked = layout != CK_LAYOUT_ROWS;
    char* p = static_cast<char*>(workspace);
    int8_t* xq = reinterpret_cast<int8_t*>(p);          p += round_up(MP * H);
    float* sx = reinterpret_cast<float*>(p);            p += round_up(M * 4);
    uint16_t* y1 = reinterpret_cast<uint16_t*>(p);      p += round_up(M * 2 * I * 2);
    int8_t* hq = reinterpret_cast<int8_t*>(p);          p += round_up(MP * I);
    float* sh = reinterpret_cast<float*>(p);
    char* part = static_cast<char*>(workspace) + base;   // split-K partials, if room
    const size_t part_bytes = workspace_bytes - base;
    hipStream_t st = (hipStream_t)stream;
    // stage 1: packed [gate | up] projection, BF16 [m, 2i]; at the fewest rows
    // (blocked or decode weights) each stage's quantizer runs inside its GEMM
    if (blocked && ck::use_fused_decode(0, m, h, group)) {
        CK_TRY(from_hip(ck::launch_gemm_dec_fused(0, x, h, m, h, group, w_gu, s_gu, dec, 2 * i, y1, st)));
    } else {
        CK_TRY(from_hip(ck::launch_quant_rows(0, x, h, m, h, group, xq, sx, nullptr, blocked, st)));
        CK_TRY(from_hip(ck::launch_gemm_bf16(xq, sx, w_gu, s_gu, m, 2 * i, h, y1, layout, st, ck::EpiExtra{}, part,
                                             part_bytes)));
    }
    // stage 2: silu(gate) * up inside the down projection's quantizer
    if (blocked && ck::use_fused_decode(1, m, i, group))
        return from_hip(ck::launch_gemm_dec_fused(1, y1, 2 * i, m, i, group, w_down, s_down, dec, h, y, st));
    CK_TRY(from_hip(ck::launch_quant_rows(1, y1, 2 * i, m, i, group, hq, sh, nullptr, blocked, st)));
    return from_hip(ck::launch_gemm_bf16(hq, sh, w_down, s_down, m, h, i, y, layout, st, ck::EpiExtra{}, part,
                                         part_bytes));
}

// ---- W8A16 ----------------------------------------------------------------

ck_status ck_act_rotate_bf16(const uint16_t* x, int64_t ldx, int64_t m, int64_t k, int32_t act,
                             int32_t group, int32_t layout, uint16_t* x_rot, void* stream)
{
    CK_TRY(check_k(k, group));
    CK_TRY(check_act(act, ldx, k));
    CK_TRY(check_layout(layout));
    if (m < 0) return CK_ESHAPE;
    if (pad_rows(m) * k * 2 > CK_MAX_ELEMS) return CK_EUNSUPPORTED;
    if (m == 0) return CK_OK;
    if (!x || !x_rot) return CK_EINVAL;
    if (!aligned16(x) || !aligned16(x_rot)) return CK_EINVAL;
    return from_hip(ck::launch_rotate_bf16(act == CK_ACT_SWIGLU ? 1 : 0, x, ldx, m, k, group, x_rot,
                                           layout == CK_LAYOUT_BLOCKED, (hipStream_t)stream));
}

static ck_status check_w8a16_args(const uint16_t* x_rot, const int8_t* w_q, int64_t m, int64_t n,
                                  int64_t k, const void* y)
{
    if (k < 1 || k % 64 != 0) return CK_ESHAPE;
    if (k > CK_MAX_K) return CK_EUNSUPPORTED;
    if (m < 0 || n < 0 || n % 16 != 0) return CK_ESHAPE;
    CK_TRY(check_gemm_extent(m, n, k));
    if (pad_rows(m) * k * 2 > CK_MAX_ELEMS) return CK_EUNSUPPORTED;
    if (m == 0 || n == 0) return CK_OK;
    if (!x_rot || !w_q || !y) return CK_EINVAL;
    if (!aligned16(x_rot) || !aligned16(w_q) || !aligned16(y)) return CK_EINVAL;
    return CK_OK;
}

ck_status ck_w8a16_gemm_bf16(const uint16_t* x_rot, const int8_t* w_q, const float* w_scale,
                             const float* bias, const uint16_t* residual, int64_t m, int64_t n,
                             int64_t k, uint16_t* y, void* stream)
{
    CK_TRY(check_w8a16_args(x_rot, w_q, m, n, k, y));
    if (m == 0 || n == 0) return CK_OK;
    if (!w_scale || !aligned16(w_scale)) return CK_EINVAL;
    CK_TRY(check_extra(bias, residual));
    return from_hip(ck::launch_gemm_w8a16(x_rot, w_q, w_scale, m, n, k, y, false, (hipStream_t)stream,
                                          ck::EpiExtra{bias, residual}));
}

ck_status ck_w8a16_gemm_f32(const uint16_t* x_rot, const int8_t* w_q, int64_t m, int64_t n,
                            int64_t k, float* acc, void* stream)
{
    CK_TRY(check_w8a16_args(x_rot, w_q, m, n, k, acc));
    if (m == 0 || n == 0) return CK_OK;
    return from_hip(ck::launch_gemm_w8a16(x_rot, w_q, nullptr, m, n, k, acc, true, (hipStream_t)stream));
}

size_t ck_int8_linear_w8a16_workspace_size(int64_t m, int64_t k)
{
    if (m <= 0 || k <= 0) return 0;
    return round_up((size_t)pad_rows(m) * (size_t)k * 2);
}

ck_status ck_int8_linear_w8a16(const uint16_t* x, int64_t ldx, int32_t act, const int8_t* w_q,
                               const float* w_scale, const float* bias, const uint16_t* residual,
                               int64_t m, int64_t n, int64_t k, int32_t group, uint16_t* y,
                               void* workspace, size_t workspace_bytes, void* stream)
{
    CK_TRY(check_k(k, group));
    CK_TRY(check_act(act, ldx, k));
    CK_TRY(check_w8a16_args(reinterpret_cast<const uint16_t*>(x), w_q, m, n, k, y));
    if (m == 0 || n == 0) return CK_OK;
    if (!w_scale || !aligned16(w_scale)) return CK_EINVAL;
    CK_TRY(check_extra(bias, residual));
    const size_t need = ck_int8_linear_w8a16_workspace_size(m, k);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0)
        return CK_EWORKSPACE;
    uint16_t* xr = static_cast<uint16_t*>(workspace);
    hipStream_t st = (hipStream_t)stream;
    const int kind = act == CK_ACT_SWIGLU ? 1 : 0;
    if (ck::use_fused_decode(kind, m, k, group))   // rotation inside the GEMM: one launch
        return from_hip(ck::launch_gemm_w8a16_fused(kind, x, ldx, m, k, group, w_q, w_scale, n, y, st,
                                                    ck::EpiExtra{bias, residual}));
    CK_TRY(from_hip(ck::launch_rotate_bf16(kind, x, ldx, m, k, group, xr, true, st)));
    return from_hip(ck::launch_gemm_w8a16(xr, w_q, w_scale, m, n, k, y, false, st,
                                          ck::EpiExtra{bias, residual}));
}

// x rotated (BF16 blocked), the [m, 2i] BF16 gate|up output, its SwiGLU'd
// rotation (BF16 blocked).
size_t ck_swiglu_mlp_w8a16_workspace_size(int64_t m, int64_t h, int64_t i)
{
    if (m <= 0 || h <= 0 || i <= 0) return 0;
    const size_t M = (size_t)m, MP = (size_t)pad_rows(m), H = (size_t)h, I = (size_t)i;
    return round_up(MP * H * 2) + round_up(M * 2 * I * 2) + round_up(MP * I * 2);
}

ck_status ck_swiglu_mlp_w8a16(const uint16_t* x, const int8_t* w_gu, const float* s_gu,
                              const int8_t* w_down, const float* s_down, int64_t m, int64_t h,
                              int64_t i, int32_t group, uint16_t* y, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    CK_TRY(check_k(h, group));
    CK_TRY(check_k(i, group));
    if (m < 0 || h % 16 != 0) return CK_ESHAPE;
    CK_TRY(check_gemm_extent(m, 2 * i, h));
    CK_TRY(check_gemm_extent(m, h, i));
    if (pad_rows(m) * h * 2 > CK_MAX_ELEMS || pad_rows(m) * i * 2 > CK_MAX_ELEMS) return CK_EUNSUPPORTED;
    if (m == 0) return CK_OK;
    if (!x || !w_gu || !w_down || !y || !s_gu || !s_down) return CK_EINVAL;
    if (!aligned16(x) || !aligned16(w_gu) || !aligned16(w_down) || !aligned16(y) || !aligned16(s_gu) ||
        !aligned16(s_down))
        return CK_EINVAL;
    const size_t need = ck_swiglu_mlp_w8a16_workspace_size(m, h, i);
    if (!workspace || workspace_bytes < need || ((uintptr_t)workspace % kAlign) != 0)
        return CK_EWORKSPACE;
    const size_t M = (size_t)m, MP = (size_t)pad_rows(m), H = (size_t)h, I = (size_t)i;
    char* p = static_cast<char*>(workspace);
    uint16_t* xr = reinterpret_cast<uint16_t*>(p);      p += round_up(MP * H * 2);
    uint16_t* y1 = reinterpret_cast<uint16_t*>(p);      p += round_up(M * 2 * I * 2);
    uint16_t* hr = reinterpret_cast<uint16_t*>(p);
    hipStream_t st = (hipStream_t)stream;
    // at the fewest rows each stage's rotation runs inside its GEMM
    if (ck::use_fused_decode(0, m, h, group)) {
        CK_TRY(from_hip(ck::launch_gemm_w8a16_fused(0, x, h, m, h, group, w_gu, s_gu, 2 * i, y1, st)));
    } else {
        CK_TRY(from_hip(ck::launch_rotate_bf16(0, x, h, m, h, group, xr, true, st)));
        CK_TRY(from_hip(ck::launch_gemm_w8a16(xr, w_gu, s_gu, m, 2 * i, h, y1, false, st)));
    }
    if (ck::use_fused_decode(1, m, i, group))
        return from_hip(ck::launch_gemm_w8a16_fused(1, y1, 2 * i, m, i, group, w_down, s_down, h, y, st));
    CK_TRY(from_hip(ck::launch_rotate_bf16(1, y1, 2 * i, m, i, group, hr, true, st)));
    return from_hip(ck::launch_gemm_w8a16(hr, w_down, s_down, m, h, i, y, false, st));
}

ck_status ck_silu_f32(const uint16_t* gate, int64_t n, float* out, void* stream)
{
    if (n < 0) return CK_ESHAPE;
    if (n == 0) return CK_OK;
    if (!gate || !out) return CK_EINVAL;
    return from_hip(ck::launch_silu(gate, n, out, (hipStream_t)stream));
}

ck_status ck_act_rotate_f32(const uint16_t* x, int64_t ldx, int64_t m, int64_t k, int32_t act,
                            int32_t group, float* u, void* stream)
{
    CK_TRY(check_k(k, group));
    CK_TRY(check_act(act, ldx, k));
    if (m < 0) return CK_ESHAPE;
    if (m == 0) return CK_OK;
    if (!x || !u) return CK_EINVAL;
    if (!aligned16(x) || !aligned16(u)) return CK_EINVAL;
    return from_hip(ck::launch_quant_rows(act == CK_ACT_SWIGLU ? 1 : 0, x, ldx, m, k, group,
                                          nullptr, nullptr, u, false, (hipStream_t)stream));
}

// ---- measurement hooks ----------------------------------------------------

int64_t ck_probe_mfma_workgroups(void) { return ck::num_cus(); }

ck_status ck_probe_mfma_i8(const int8_t* ops, int64_t iters, int32_t lds, int32_t* sink, void* stream)
{
    if (iters < 0 || iters > 0x7fffffff || (iters & 1)) return CK_ESHAPE;
    if (!ops || !sink || !aligned16(ops) || ((uintptr_t)sink % 4) != 0) return CK_EINVAL;
    if (iters == 0) return CK_OK;
    return from_hip(ck::launch_probe_mfma(ops, iters, lds != 0, sink, (hipStream_t)stream));
}

ck_status ck_probe_stream_rows(const void* src, int64_t ld_bytes, int64_t m, int64_t read_bytes,
                               int64_t write_bytes, void* dst, void* stream)
{
    if (m < 0 || read_bytes < 16 || read_bytes % 16 != 0 || read_bytes > 65536 || write_bytes < 0 ||
        write_bytes % 8 != 0 || write_bytes / 8 > read_bytes / 16 || ld_bytes < read_bytes || ld_bytes % 16 != 0)
        return CK_ESHAPE;
    if (m > 0x7fffffff) return CK_EUNSUPPORTED;
    if (m == 0) return CK_OK;
    if (!src || !dst || !aligned16(src) || ((uintptr_t)dst % 8) != 0) return CK_EINVAL;
    return from_hip(ck::launch_probe_stream(src, ld_bytes, m, read_bytes, write_bytes, dst, (hipStream_t)stream));
}

}  // extern "C"
