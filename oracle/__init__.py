"""CPU oracle of the ConvRot INT8 linear and the SwiGLU MLP block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``swiglu_mlp_amd``) never imports it, and the two share no code.

The arithmetic lives in ``convrot_oracle.c`` (plain C, FP32 pinned, compiled
with ``-ffp-contract=off``); this module marshals numpy arrays in and out and
adds the FP64 reference used for the relative-L2 accuracy figure.

Sources (page title, section):
  * comfy-kitchen PR #277 "Add FP16 tensor-core fallback for int8_linear on
    devices without INT8 tensor cores", "The key observation" (rotated basis,
    activation quantized on the weight's INT8 grid) and "Measured results"
    (int32 accumulation; relative error against a float32 reference).
  * sglang PR #44196 (comfy_kitchen_swiglu_mlp), "Motivation" (packed
    [gate | up] GEMM, then the SwiGLU applied inside the down projection's
    quantizer) and "Accuracy Tests" (silu(gate) * up kept in FP32; relative L2
    against an FP32 reference; fused no worse than eager).
  * sglang PR #35994 report "[diffusion] Load serialized Comfy ConvRot INT8
    DiTs", key source excerpts (I8 weight + F32 [out, 1] row scale,
    per_channel=True, convrot=True; in_features divisible by the group size).
  * comfy-kitchen PR #277, "Notes for the reviewer": the variant that keeps
    the rotated activation in 16-bit floating point (W8A16), with the INT8
    weight widened on the fly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "convrot_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O3", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
          "-shared", "-std=c11", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.orc_hadamard.argtypes = [i32, p]
        L.orc_hadamard.restype = i32
        L.orc_exp_neg.argtypes = [ctypes.c_float]
        L.orc_exp_neg.restype = ctypes.c_float
        L.orc_rcp.argtypes = [ctypes.c_float]
        L.orc_rcp.restype = ctypes.c_float
        L.orc_silu.argtypes = [ctypes.c_float]
        L.orc_silu.restype = ctypes.c_float
        L.orc_norm_const.argtypes = [i32]
        L.orc_norm_const.restype = ctypes.c_float
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        for name in ("orc_exp_neg_v", "orc_rcp_v", "orc_silu_v"):
            getattr(L, name).argtypes = [p, i64, p]
            getattr(L, name).restype = None
        L.orc_fwht_groups.argtypes = [p, i64, i32]
        L.orc_fwht_groups.restype = None
        L.orc_quant_row.argtypes = [p, i64, i32, p, p]
        L.orc_quant_row.restype = None
        L.orc_act_quant.argtypes = [p, i64, i64, i64, i32, i32, p, p]
        L.orc_act_quant.restype = i32
        L.orc_act_rotate.argtypes = [p, i64, i64, i64, i32, i32, p]
        L.orc_act_rotate.restype = i32
        L.orc_weight_prep.argtypes = [p, i64, i64, i32, p, p]
        L.orc_weight_prep.restype = i32
        L.orc_gemm_i32.argtypes = [p, p, i64, i64, i64, p]
        L.orc_gemm_i32.restype = None
        L.orc_dequant_bf16.argtypes = [p, p, p, i64, i64, p]
        L.orc_dequant_bf16.restype = None
        L.orc_epilogue_bf16.argtypes = [p, p, p, p, p, i64, i64, p]
        L.orc_epilogue_bf16.restype = None
        L.orc_eager_swiglu_bf16.argtypes = [p, i64, i64, i64, p]
        L.orc_eager_swiglu_bf16.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# BF16 helpers (BF16 tensors are carried as uint16 bit patterns)
# --------------------------------------------------------------------------
def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(f) -> np.ndarray:
    """Round-to-nearest-even FP32 -> BF16 (finite inputs), vectorised."""
    f = _c(f, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Pinned scalar / vector functions
# --------------------------------------------------------------------------
def hadamard(g: int) -> np.ndarray:
    h = np.empty((g, g), dtype=np.float64)
    if lib().orc_hadamard(g, _ptr(h)) != 0:
        raise ValueError(f"group size {g} is not a power of two")
    return h


def norm_const(g: int) -> np.float32:
    return np.float32(lib().orc_norm_const(g))


def exp_neg(x) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().orc_exp_neg_v(_ptr(x), x.size, _ptr(y))
    return y


def rcp(x) -> np.ndarray:
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().orc_rcp_v(_ptr(x), x.size, _ptr(y))
    return y


def silu_bf16(gate_bits) -> np.ndarray:
    """Pinned FP32 silu of BF16 inputs given as uint16 bit patterns."""
    g = _c(gate_bits, np.uint16)
    y = np.empty(g.shape, dtype=np.float32)
    lib().orc_silu_v(_ptr(g), g.size, _ptr(y))
    return y


def fwht(v, g: int) -> np.ndarray:
    """Unnormalised blockwise FWHT over the last axis (a copy)."""
    v = np.array(v, dtype=np.float32, copy=True, order="C")
    if v.shape[-1] % g:
        raise ValueError("last axis must be a multiple of the group size")
    lib().orc_fwht_groups(_ptr(v), v.size, g)
    return v


def quant_row(u, g: int):
    u = _c(u, np.float32)
    q = np.empty(u.shape[0], dtype=np.int8)
    s = np.empty(1, dtype=np.float32)
    lib().orc_quant_row(_ptr(u), u.shape[0], g, _ptr(q), _ptr(s))
    return q, s[0]


# --------------------------------------------------------------------------
# Path steps
# --------------------------------------------------------------------------
ACT_NONE, ACT_SWIGLU = 0, 1


def _act_args(x, k, act):
    x = _c(x, np.uint16)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    if k is None:
        k = x.shape[1] // (2 if act == ACT_SWIGLU else 1)
    return x, int(k)


def act_quant(x_bf16, act: int, g: int, k: int | None = None):
    """x [m, ldx] BF16 bits -> (q int8 [m, k], s float32 [m])."""
    x, k = _act_args(x_bf16, k, act)
    m = x.shape[0]
    q = np.empty((m, k), dtype=np.int8)
    s = np.empty(m, dtype=np.float32)
    if lib().orc_act_quant(_ptr(x), x.shape[1], m, k, act, g, _ptr(q), _ptr(s)):
        raise ValueError("bad act_quant arguments")
    return q, s


def act_rotate(x_bf16, act: int, g: int, k: int | None = None) -> np.ndarray:
    x, k = _act_args(x_bf16, k, act)
    u = np.empty((x.shape[0], k), dtype=np.float32)
    if lib().orc_act_rotate(_ptr(x), x.shape[1], x.shape[0], k, act, g, _ptr(u)):
        raise ValueError("bad act_rotate arguments")
    return u


def weight_prep(w, g: int):
    """W [n, k] FP32 -> (W_q int8 [n, k], s_w float32 [n])."""
    w = _c(w, np.float32)
    n, k = w.shape
    q = np.empty((n, k), dtype=np.int8)
    s = np.empty(n, dtype=np.float32)
    if lib().orc_weight_prep(_ptr(w), n, k, g, _ptr(q), _ptr(s)):
        raise ValueError(f"in_features ({k}) must be divisible by group_size {g}")
    return q, s


def gemm_i32(xq, wq) -> np.ndarray:
    xq, wq = _c(xq, np.int8), _c(wq, np.int8)
    m, k = xq.shape
    n = wq.shape[0]
    assert wq.shape[1] == k
    acc = np.empty((m, n), dtype=np.int32)
    lib().orc_gemm_i32(_ptr(xq), _ptr(wq), m, n, k, _ptr(acc))
    return acc


def dequant(acc, sx, sw) -> np.ndarray:
    acc = _c(acc, np.int32)
    sx, sw = _c(sx, np.float32).reshape(-1), _c(sw, np.float32).reshape(-1)
    m, n = acc.shape
    y = np.empty((m, n), dtype=np.uint16)
    lib().orc_dequant_bf16(_ptr(acc), _ptr(sx), _ptr(sw), m, n, _ptr(y))
    return y


def epilogue(acc, sx, sw, bias=None, residual=None) -> np.ndarray:
    """Dequant with optional F32 bias [n] and BF16 residual [m, n] (uint16 bits)."""
    acc = _c(acc, np.int32)
    sx, sw = _c(sx, np.float32).reshape(-1), _c(sw, np.float32).reshape(-1)
    m, n = acc.shape
    b = None if bias is None else _c(bias, np.float32).reshape(-1)
    r = None if residual is None else _c(residual, np.uint16)
    assert b is None or b.shape == (n,)
    assert r is None or r.shape == (m, n)
    y = np.empty((m, n), dtype=np.uint16)
    lib().orc_epilogue_bf16(_ptr(acc), _ptr(sx), _ptr(sw), None if b is None else _ptr(b),
                            None if r is None else _ptr(r), m, n, _ptr(y))
    return y


def int8_linear(x_bf16, act: int, wq, sw, g: int, return_all: bool = False, bias=None,
                residual=None):
    """ConvRot int8_linear: quantize the (optionally SwiGLU'd) activation in the
    rotated basis, multiply against W_rot's codes, dequantize to BF16 (plus the
    optional bias and residual)."""
    xq, sx = act_quant(x_bf16, act, g, k=np.asarray(wq).shape[1])
    acc = gemm_i32(xq, wq)
    if bias is None and residual is None:
        y = dequant(acc, sx, sw)
    else:
        y = epilogue(acc, sx, sw, bias, residual)
    if return_all:
        return dict(xq=xq, sx=sx, acc=acc, y=y)
    return y


def swiglu_mlp(x_bf16, wgu_q, sgu, wd_q, sd, g: int, return_all: bool = False):
    """sglang PR #44196, "Motivation": one packed [gate | up] int8_linear, then
    int8_linear(..., input_act="swiglu") on its BF16 output."""
    s1 = int8_linear(x_bf16, ACT_NONE, wgu_q, sgu, g, return_all=True)
    s2 = int8_linear(s1["y"], ACT_SWIGLU, wd_q, sd, g, return_all=True)
    if return_all:
        return dict(stage1=s1, stage2=s2, y=s2["y"])
    return s2["y"]


# --------------------------------------------------------------------------
# W8A16: the rotated activation kept in BF16 (comfy-kitchen PR #277, "Notes
# for the reviewer"; "The key observation": the GEMM stays in the rotated basis)
# --------------------------------------------------------------------------
def act_rotate_bf16(x_bf16, act: int, g: int, k: int | None = None) -> np.ndarray:
    """x_rot = x H with the orthonormal H, rounded to BF16: the unnormalised
    FWHT u of the (optionally SwiGLU'd) row, then bf16(fl(u * fl(1/sqrt(g))) + 0).
    The + 0 writes an exact zero (also one the product underflows to) as +0:
    x H is defined over the reals, where a zero has no sign."""
    u = act_rotate(x_bf16, act, g, k)
    # float32 * float32: one FP32 rounding; + 0 changes no nonzero value
    return f32_to_bf16(u * norm_const(g) + np.float32(0.0))


def w8a16_acc(x_rot_bf16, wq) -> np.ndarray:
    """sum_k x_rot[m, k] * q[n, k] in float64 (each product is exact; the sum
    is exact up to float64 rounding)."""
    x = bf16_to_f32(_c(x_rot_bf16, np.uint16)).astype(np.float64)
    return x @ np.asarray(wq, dtype=np.float64).T


def w8a16_abs_acc(x_rot_bf16, wq) -> np.ndarray:
    """sum_k |x_rot[m, k] * q[n, k]|: the scale of the FP32 accumulation error."""
    x = np.abs(bf16_to_f32(_c(x_rot_bf16, np.uint16)).astype(np.float64))
    return x @ np.abs(np.asarray(wq, dtype=np.float64)).T


def w8a16_epilogue(acc, sw, bias=None, residual=None) -> np.ndarray:
    """y = bf16(f32(acc * s_w[n]) (+ bias[n]) (+ residual[m, n])), the sums in
    FP32 in that order, one BF16 rounding at the end."""
    t = (np.asarray(acc, dtype=np.float64) * _c(sw, np.float64).reshape(1, -1)).astype(np.float32)
    if bias is not None:
        t = t + _c(bias, np.float32).reshape(1, -1)
    if residual is not None:
        t = t + bf16_to_f32(_c(residual, np.uint16))
    return f32_to_bf16(t)


def w8a16_linear(x_bf16, act: int, wq, sw, g: int, bias=None, residual=None,
                 return_all: bool = False):
    """The W8A16 linear: BF16 rotated activation times the INT8 W_rot codes,
    accumulated exactly, scaled per output row."""
    x_rot = act_rotate_bf16(x_bf16, act, g, k=np.asarray(wq).shape[1])
    acc = w8a16_acc(x_rot, wq)
    y = w8a16_epilogue(acc, sw, bias, residual)
    if return_all:
        return dict(x_rot=x_rot, acc=acc, y=y)
    return y


def swiglu_mlp_w8a16(x_bf16, wgu_q, sgu, wd_q, sd, g: int, return_all: bool = False):
    """The SwiGLU MLP block with W8A16 linears: w8a16_linear of x against the
    packed [gate | up] codes, then w8a16_linear(..., swiglu) of its BF16 output."""
    s1 = w8a16_linear(x_bf16, ACT_NONE, wgu_q, sgu, g, return_all=True)
    s2 = w8a16_linear(s1["y"], ACT_SWIGLU, wd_q, sd, g, return_all=True)
    if return_all:
        return dict(stage1=s1, stage2=s2, y=s2["y"])
    return s2["y"]


def eager_swiglu_bf16(x_bf16) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    m, ldx = x.shape
    k = ldx // 2
    a = np.empty((m, k), dtype=np.uint16)
    lib().orc_eager_swiglu_bf16(_ptr(x), ldx, m, k, _ptr(a))
    return a


# --------------------------------------------------------------------------
# FP64 reference and accuracy figure
# --------------------------------------------------------------------------
def silu_f64(g: np.ndarray) -> np.ndarray:
    g = np.asarray(g, dtype=np.float64)
    return g / (1.0 + np.exp(-g))


def reference_linear_f64(x_bf16, act: int, w) -> np.ndarray:
    """Unrotated, unquantized y = a W^T in float64 (a = x, or silu(gate)*up)."""
    x = bf16_to_f32(_c(x_bf16, np.uint16)).astype(np.float64)
    w = np.asarray(w, dtype=np.float64)
    k = w.shape[1]
    a = x[:, :k] if act == ACT_NONE else silu_f64(x[:, :k]) * x[:, k:2 * k]
    return a @ w.T


def reference_mlp_f64(x_bf16, w_gu, w_down) -> np.ndarray:
    x = bf16_to_f32(_c(x_bf16, np.uint16)).astype(np.float64)
    h = x @ np.asarray(w_gu, dtype=np.float64).T
    i = h.shape[1] // 2
    a = silu_f64(h[:, :i]) * h[:, i:]
    return a @ np.asarray(w_down, dtype=np.float64).T


def rel_l2(y, y_ref) -> float:
    """||y - y_ref||_F / ||y_ref||_F in float64; y may be BF16 bits."""
    y = np.asarray(y)
    if y.dtype == np.uint16:
        y = bf16_to_f32(y)
    y = y.astype(np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    return float(np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref))
