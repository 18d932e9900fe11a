"""MI355X (gfx950) ConvRot INT8 linear and SwiGLU MLP: Python binding.

This module only marshals arguments: it checks dtypes and shapes, takes device
pointers and the current HIP stream from torch tensors, and calls the C ABI of
``libck_convrot.so`` (declared in ``include/ck.h``).  Every step of the path
runs in that library's HIP kernels; there is no fallback.  If the library is
missing, importing any entry point raises.

Entry points keep the C names:

* ``ck_weight_prep(w, group)``           -> (w_q int8 [n, k], w_scale f32 [n, 1])
* ``ck_weight_pack(w_q)``                 -> w_q in the blocked layout [n_pad, k]
* ``ck_weight_pack_decode(w_q, w_scale)`` -> codes and scales in the decode layout
* ``ck_act_quant(x, act, group, k=None, layout=...)`` -> (x_q, x_scale f32 [m, 1])
* ``ck_int8_linear(x, w_q, w_scale, group, input_act=None, layout=..., bias=None, residual=None)``
* ``ck_int8_gemm_bf16(x_q, x_scale, w_q, w_scale, layout=..., bias=None, residual=None)``
* ``ck_swiglu_mlp(x, w_gu, s_gu, w_down, s_down, group, layout=...)`` -> y bf16
* W8A16 (BF16 activations, INT8 weights in the blocked layout):
  ``ck_act_rotate_bf16``, ``ck_w8a16_gemm_bf16``, ``ck_int8_linear_w8a16``,
  ``ck_swiglu_mlp_w8a16``
* test hooks ``ck_int8_gemm_i32``, ``ck_w8a16_gemm_f32``, ``ck_silu_f32``, ``ck_act_rotate_f32``

``layout`` is ``"rows"`` (row-major int8, the serialized checkpoint format),
``"blocked"`` (the GEMM-native layout of include/ck.h, rows padded to 256) or
``"decode"`` (weights only, at most 64 token rows: each 16-row group of the
weight one linear stream with its row scales in front; activation codes are
then blocked).  With blocked operands the logical row counts come from the
scale vectors; a decode weight is a uint8 [n / 16, 64 + 16 k] tensor that
carries its scales, and its ``w_scale`` argument may be None.

Shapes and error behaviour follow sglang PR #35994 report, key source excerpts:
an INT8 weight is 2-D ``[out_features, in_features]`` with an F32
``[out_features, 1]`` scale, and in_features must be divisible by the group
size; violations raise ``ValueError`` before anything is launched.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libck_convrot.so")

CK_ACT_NONE, CK_ACT_SWIGLU = 0, 1
CK_LAYOUT_ROWS, CK_LAYOUT_BLOCKED, CK_LAYOUT_DECODE = 0, 1, 2
_STATUS = {0: "CK_OK", 1: "CK_EINVAL", 2: "CK_ESHAPE", 3: "CK_EUNSUPPORTED",
           4: "CK_EWORKSPACE", 5: "CK_EHIP"}


class CKError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} ({text})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libck_convrot.so (after torch, so both use one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m swiglu_mlp_amd.build` (hipcc, gfx950)")
        _lib = bind(LIB_PATH)
    return _lib


def bind(path: str) -> ctypes.CDLL:
    """Load a build of the library at `path` with every entry point's C
    signature declared.  Without declared argument types ctypes passes Python
    ints as C int, masking 64-bit pointers and sizes to 32 bits."""
    import torch  # noqa: F401  -- loads torch's HIP runtime first
    L = ctypes.CDLL(path)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "ck_weight_prep": [p, i64, i64, i32, p, p, p],
        "ck_weight_pack": [p, i64, i64, p, p],
        "ck_weight_pack_decode": [p, p, i64, i64, p, p],
        "ck_act_quant": [p, i64, i64, i64, i32, i32, i32, p, p, p],
        "ck_int8_linear": [p, i64, i32, p, p, p, p, i32, i64, i64, i64, i32, p, p, sz, p],
        "ck_int8_gemm_bf16": [p, p, p, p, p, p, i32, i64, i64, i64, p, p],
        "ck_swiglu_mlp": [p, p, p, p, p, i32, i64, i64, i64, i32, p, p, sz, p],
        "ck_int8_gemm_i32": [p, p, i32, i64, i64, i64, p, p],
        "ck_act_rotate_bf16": [p, i64, i64, i64, i32, i32, i32, p, p],
        "ck_w8a16_gemm_bf16": [p, p, p, p, p, i64, i64, i64, p, p],
        "ck_w8a16_gemm_f32": [p, p, i64, i64, i64, p, p],
        "ck_int8_linear_w8a16": [p, i64, i32, p, p, p, p, i64, i64, i64, i32, p, p, sz, p],
        "ck_swiglu_mlp_w8a16": [p, p, p, p, p, i64, i64, i64, i32, p, p, sz, p],
        "ck_silu_f32": [p, i64, p, p],
        "ck_act_rotate_f32": [p, i64, i64, i64, i32, i32, p, p],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.ck_int8_linear_workspace_size.argtypes = [i64, i64]
    L.ck_int8_linear_workspace_size.restype = sz
    L.ck_int8_linear_w8a16_workspace_size.argtypes = [i64, i64]
    L.ck_int8_linear_w8a16_workspace_size.restype = sz
    L.ck_swiglu_mlp_w8a16_workspace_size.argtypes = [i64, i64, i64]
    L.ck_swiglu_mlp_w8a16_workspace_size.restype = sz
    L.ck_swiglu_mlp_workspace_size.argtypes = [i64, i64, i64]
    L.ck_swiglu_mlp_workspace_size.restype = sz
    L.ck_blocked_rows.argtypes = [i64]
    L.ck_blocked_rows.restype = i64
    L.ck_blocked_size.argtypes = [i64, i64]
    L.ck_blocked_size.restype = sz
    L.ck_decode_size.argtypes = [i64, i64]
    L.ck_decode_size.restype = sz
    L.ck_status_str.argtypes = [ctypes.c_int]
    L.ck_status_str.restype = ctypes.c_char_p
    L.ck_version.argtypes = []
    L.ck_version.restype = ctypes.c_char_p
    return L


def _call(name: str, *args) -> None:
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise CKError(name, st, lib().ck_status_str(st).decode())


def _stream(t):
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t, dtype, ndim, what):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{what} must be on a GPU, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{what} needs dtype {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{what} needs a {ndim}D tensor, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _scale(s, rows, what):
    """Accept [rows, 1] (the serialized row-scale layout) or [rows]."""
    import torch
    if s.dim() == 2:
        if tuple(s.shape) != (rows, 1):
            raise ValueError(f"{what} needs scale shape ({rows}, 1), got {tuple(s.shape)}")
    else:
        _need(s, torch.float32, 1, what)
        if s.shape[0] != rows:
            raise ValueError(f"{what} needs {rows} scales, got {s.shape[0]}")
    _need(s, torch.float32, s.dim(), what)
    return s


def _check_group(k, group):
    if k % group:
        raise ValueError(f"in_features ({k}) must be divisible by group_size {group}")


def _layout_code(layout):
    if layout in ("rows", CK_LAYOUT_ROWS):
        return CK_LAYOUT_ROWS
    if layout in ("blocked", CK_LAYOUT_BLOCKED):
        return CK_LAYOUT_BLOCKED
    if layout in ("decode", CK_LAYOUT_DECODE):
        return CK_LAYOUT_DECODE
    raise ValueError(f"unknown layout {layout!r}")


def blocked_rows(rows: int) -> int:
    return int(lib().ck_blocked_rows(rows))


def _decode_shape(w, what):
    """(n, k) of a weight in the decode layout: uint8 [n / 16, 64 + 16 k]."""
    import torch
    _need(w, torch.uint8, 2, what)
    if (w.shape[1] - 64) % 1024 or w.shape[1] <= 64:
        raise ValueError(f"{what}: a decode-layout weight has 64 + 16 k columns with k % 64 == 0, "
                         f"got {w.shape[1]}")
    return 16 * w.shape[0], (w.shape[1] - 64) // 16


def _weight(w, w_scale, lay, what):
    """(n, k) of a weight operand in layout `lay`, with its scale checked."""
    import torch
    if lay == CK_LAYOUT_DECODE:
        n, k = _decode_shape(w, what)
        if w_scale is not None:
            raise ValueError(f"{what}: the decode layout carries its scales; pass w_scale=None")
        return n, k
    _need(w, torch.int8, 2, what)
    if w_scale is None:
        raise ValueError(f"{what}: weight scale missing")
    n = w_scale.shape[0]
    _operand_rows(w, n, lay, what)
    _scale(w_scale, n, what + " scale")
    return n, w.shape[1]


def _act_layout(lay):
    """Layout of the activation codes that go with a weight in layout `lay`."""
    return CK_LAYOUT_ROWS if lay == CK_LAYOUT_ROWS else CK_LAYOUT_BLOCKED


def _ptr(t):
    return None if t is None else t.data_ptr()


def _operand_rows(t, rows, layout, what):
    """Check an int8 operand buffer holds `rows` logical rows in `layout`."""
    need = rows if layout == CK_LAYOUT_ROWS else blocked_rows(rows)
    if t.shape[0] != need:
        raise ValueError(f"{what} needs {need} rows for {rows} logical rows in "
                         f"{'row-major' if layout == CK_LAYOUT_ROWS else 'blocked'} layout, "
                         f"got {t.shape[0]}")


def _act_code(input_act):
    if input_act in (None, "none", CK_ACT_NONE):
        return CK_ACT_NONE
    if input_act in ("swiglu", CK_ACT_SWIGLU):
        return CK_ACT_SWIGLU
    raise ValueError(f"unknown input_act {input_act!r}")


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def ck_weight_prep(w, group: int = 128):
    import torch
    _need(w, torch.float32, 2, "weight")
    n, k = w.shape
    _check_group(k, group)
    w_q = torch.empty((n, k), dtype=torch.int8, device=w.device)
    w_scale = torch.empty((n, 1), dtype=torch.float32, device=w.device)
    _call("ck_weight_prep", w.data_ptr(), n, k, group, w_q.data_ptr(), w_scale.data_ptr(),
          _stream(w))
    return w_q, w_scale


def ck_weight_pack(w_q):
    """Relayout row-major int8 weight codes [n, k] into the blocked layout."""
    import torch
    _need(w_q, torch.int8, 2, "weight")
    n, k = w_q.shape
    out = torch.empty((blocked_rows(n), k), dtype=torch.int8, device=w_q.device)
    _call("ck_weight_pack", w_q.data_ptr(), n, k, out.data_ptr(), _stream(w_q))
    return out


def ck_weight_pack_decode(w_q, w_scale):
    """Row-major int8 codes [n, k] and FP32 row scales [n] (or [n, 1]) ->
    the decode layout, a uint8 tensor [n / 16, 64 + 16 k]."""
    import torch
    _need(w_q, torch.int8, 2, "weight")
    n, k = w_q.shape
    _scale(w_scale, n, "weight_scale")
    if n % 16:
        raise ValueError(f"the decode layout needs out_features % 16 == 0, got {n}")
    out = torch.empty((n // 16, 64 + 16 * k), dtype=torch.uint8, device=w_q.device)
    assert out.numel() == lib().ck_decode_size(n, k)
    _call("ck_weight_pack_decode", w_q.data_ptr(), w_scale.data_ptr(), n, k, out.data_ptr(),
          _stream(w_q))
    return out


def ck_act_quant(x, input_act=None, group: int = 128, k: int | None = None, layout="rows"):
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    act = _act_code(input_act)
    lay = _layout_code(layout)
    m, ldx = x.shape
    if k is None:
        k = ldx // 2 if act == CK_ACT_SWIGLU else ldx
    _check_group(k, group)
    rows = m if lay == CK_LAYOUT_ROWS else blocked_rows(m)
    x_q = torch.empty((rows, k), dtype=torch.int8, device=x.device)
    x_scale = torch.empty((m, 1), dtype=torch.float32, device=x.device)
    _call("ck_act_quant", x.data_ptr(), ldx, m, k, act, group, lay, x_q.data_ptr(),
          x_scale.data_ptr(), _stream(x))
    return x_q, x_scale


def _extra(bias, residual, m, n, dev):
    """Optional epilogue terms: F32 bias [n] and BF16 residual [m, n]."""
    import torch
    bp = rp = None
    if bias is not None:
        _need(bias, torch.float32, 1, "bias")
        if bias.shape[0] != n or bias.device != dev or not bias.is_contiguous():
            raise ValueError(f"bias needs a contiguous ({n},) float32 tensor on {dev}")
        bp = bias.data_ptr()
    if residual is not None:
        _need(residual, torch.bfloat16, 2, "residual")
        if tuple(residual.shape) != (m, n) or residual.device != dev or not residual.is_contiguous():
            raise ValueError(f"residual needs a contiguous ({m}, {n}) bfloat16 tensor on {dev}")
        rp = residual.data_ptr()
    return bp, rp


def ck_int8_linear(x, w_q, w_scale, group: int = 128, input_act=None, out=None,
                   workspace=None, layout="rows", bias=None, residual=None):
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    lay = _layout_code(layout)
    n, k = _weight(w_q, w_scale, lay, "weight")
    act = _act_code(input_act)
    m, ldx = x.shape
    need_ld = 2 * k if act == CK_ACT_SWIGLU else k
    if ldx != need_ld:
        raise ValueError(f"activation needs {need_ld} columns for in_features {k}, got {ldx}")
    _check_group(k, group)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    ws_bytes = lib().ck_int8_linear_workspace_size(m, k)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    bp, rp = _extra(bias, residual, m, n, x.device)
    _call("ck_int8_linear", x.data_ptr(), ldx, act, w_q.data_ptr(), _ptr(w_scale), bp, rp,
          lay, m, n, k, group, y.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(x))
    return y


def ck_int8_gemm_bf16(x_q, x_scale, w_q, w_scale, out=None, layout="rows", bias=None,
                      residual=None):
    import torch
    _need(x_q, torch.int8, 2, "activation codes")
    lay = _layout_code(layout)
    k = x_q.shape[1]
    m = x_scale.shape[0]
    n, kw = _weight(w_q, w_scale, lay, "weight")
    if kw != k:
        raise ValueError(f"in_features mismatch: activation {k}, weight {kw}")
    _operand_rows(x_q, m, _act_layout(lay), "activation codes")
    _scale(x_scale, m, "activation scale")
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x_q.device)
    bp, rp = _extra(bias, residual, m, n, x_q.device)
    _call("ck_int8_gemm_bf16", x_q.data_ptr(), x_scale.data_ptr(), w_q.data_ptr(),
          _ptr(w_scale), bp, rp, lay, m, n, k, y.data_ptr(), _stream(x_q))
    return y


def ck_swiglu_mlp(x, w_gu, s_gu, w_down, s_down, group: int = 128, out=None, workspace=None,
                  layout="rows"):
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    lay = _layout_code(layout)
    m, h = x.shape
    i2, kg = _weight(w_gu, s_gu, lay, "gate_up weight")
    if kg != h or i2 % 2:
        raise ValueError(f"gate_up weight needs (2*intermediate, {h}), got ({i2}, {kg})")
    i = i2 // 2
    hd, kd = _weight(w_down, s_down, lay, "down weight")
    if kd != i or hd != h:
        raise ValueError(f"down weight needs ({h}, {i}), got ({hd}, {kd})")
    _check_group(h, group)
    _check_group(i, group)
    y = out if out is not None else torch.empty((m, h), dtype=torch.bfloat16, device=x.device)
    ws_bytes = lib().ck_swiglu_mlp_workspace_size(m, h, i)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _call("ck_swiglu_mlp", x.data_ptr(), w_gu.data_ptr(), _ptr(s_gu), w_down.data_ptr(),
          _ptr(s_down), lay, m, h, i, group, y.data_ptr(), workspace.data_ptr(),
          workspace.numel(), _stream(x))
    return y


def ck_int8_gemm_i32(x_q, w_q, layout="rows", m: int | None = None, n: int | None = None):
    """Raw int32 accumulators; with blocked operands pass the logical m and n."""
    import torch
    _need(x_q, torch.int8, 2, "activation codes")
    lay = _layout_code(layout)
    k = x_q.shape[1]
    m = x_q.shape[0] if m is None else m
    if lay == CK_LAYOUT_DECODE:
        n, kw = _decode_shape(w_q, "weight")
    else:
        _need(w_q, torch.int8, 2, "weight")
        n = w_q.shape[0] if n is None else n
        kw = w_q.shape[1]
        _operand_rows(w_q, n, lay, "weight")
    if kw != k:
        raise ValueError(f"in_features mismatch: activation {k}, weight {kw}")
    _operand_rows(x_q, m, _act_layout(lay), "activation codes")
    acc = torch.empty((m, n), dtype=torch.int32, device=x_q.device)
    _call("ck_int8_gemm_i32", x_q.data_ptr(), w_q.data_ptr(), lay, m, n, k, acc.data_ptr(),
          _stream(x_q))
    return acc


def ck_act_rotate_bf16(x, input_act=None, group: int = 128, k: int | None = None, layout="rows"):
    """Rotated activation in BF16 (no quantization): [m, k] row-major, or the
    BF16 blocked layout of include/ck.h as a [blocked_rows(m), k] tensor."""
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    act = _act_code(input_act)
    lay = _layout_code(layout)
    m, ldx = x.shape
    if k is None:
        k = ldx // 2 if act == CK_ACT_SWIGLU else ldx
    _check_group(k, group)
    rows = m if lay == CK_LAYOUT_ROWS else blocked_rows(m)
    xr = torch.empty((rows, k), dtype=torch.bfloat16, device=x.device)
    _call("ck_act_rotate_bf16", x.data_ptr(), ldx, m, k, act, group, lay, xr.data_ptr(), _stream(x))
    return xr


def _w8a16_operands(x_rot, w_q, m, n):
    import torch
    _need(x_rot, torch.bfloat16, 2, "rotated activation")
    _need(w_q, torch.int8, 2, "weight")
    k = x_rot.shape[1]
    if w_q.shape[1] != k:
        raise ValueError(f"in_features mismatch: activation {k}, weight {w_q.shape[1]}")
    _operand_rows(x_rot, m, CK_LAYOUT_BLOCKED, "rotated activation")
    _operand_rows(w_q, n, CK_LAYOUT_BLOCKED, "weight")
    return k


def ck_w8a16_gemm_bf16(x_rot, w_q, w_scale, m: int, out=None, bias=None, residual=None):
    """y = bf16(acc * w_scale (+ bias) (+ residual)); x_rot in the BF16 blocked
    layout with m logical rows, w_q blocked."""
    import torch
    n = w_scale.shape[0]
    _scale(w_scale, n, "weight_scale")
    k = _w8a16_operands(x_rot, w_q, m, n)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x_rot.device)
    bp, rp = _extra(bias, residual, m, n, x_rot.device)
    _call("ck_w8a16_gemm_bf16", x_rot.data_ptr(), w_q.data_ptr(), w_scale.data_ptr(), bp, rp, m, n, k,
          y.data_ptr(), _stream(x_rot))
    return y


def ck_w8a16_gemm_f32(x_rot, w_q, m: int, n: int):
    """Raw FP32 accumulators of the W8A16 GEMM."""
    import torch
    k = _w8a16_operands(x_rot, w_q, m, n)
    acc = torch.empty((m, n), dtype=torch.float32, device=x_rot.device)
    _call("ck_w8a16_gemm_f32", x_rot.data_ptr(), w_q.data_ptr(), m, n, k, acc.data_ptr(),
          _stream(x_rot))
    return acc


def ck_int8_linear_w8a16(x, w_q, w_scale, group: int = 128, input_act=None, out=None,
                         workspace=None, bias=None, residual=None):
    """W8A16 linear: BF16 rotated activation times the blocked INT8 weight."""
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    _need(w_q, torch.int8, 2, "weight")
    n = w_scale.shape[0]
    _scale(w_scale, n, "weight_scale")
    _operand_rows(w_q, n, CK_LAYOUT_BLOCKED, "weight")
    k = w_q.shape[1]
    act = _act_code(input_act)
    m, ldx = x.shape
    need_ld = 2 * k if act == CK_ACT_SWIGLU else k
    if ldx != need_ld:
        raise ValueError(f"activation needs {need_ld} columns for in_features {k}, got {ldx}")
    _check_group(k, group)
    y = out if out is not None else torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    ws_bytes = lib().ck_int8_linear_w8a16_workspace_size(m, k)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    bp, rp = _extra(bias, residual, m, n, x.device)
    _call("ck_int8_linear_w8a16", x.data_ptr(), ldx, act, w_q.data_ptr(), w_scale.data_ptr(), bp, rp,
          m, n, k, group, y.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(x))
    return y


def ck_swiglu_mlp_w8a16(x, w_gu, s_gu, w_down, s_down, group: int = 128, out=None, workspace=None):
    """The SwiGLU MLP block with W8A16 linears; weights in the blocked layout."""
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    m, h = x.shape
    i2, kg = _weight(w_gu, s_gu, CK_LAYOUT_BLOCKED, "gate_up weight")
    if kg != h or i2 % 2:
        raise ValueError(f"gate_up weight needs (2*intermediate, {h}), got ({i2}, {kg})")
    i = i2 // 2
    hd, kd = _weight(w_down, s_down, CK_LAYOUT_BLOCKED, "down weight")
    if kd != i or hd != h:
        raise ValueError(f"down weight needs ({h}, {i}), got ({hd}, {kd})")
    _check_group(h, group)
    _check_group(i, group)
    y = out if out is not None else torch.empty((m, h), dtype=torch.bfloat16, device=x.device)
    ws_bytes = lib().ck_swiglu_mlp_w8a16_workspace_size(m, h, i)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    _call("ck_swiglu_mlp_w8a16", x.data_ptr(), w_gu.data_ptr(), s_gu.data_ptr(), w_down.data_ptr(),
          s_down.data_ptr(), m, h, i, group, y.data_ptr(), workspace.data_ptr(), workspace.numel(),
          _stream(x))
    return y


def ck_silu_f32(gate):
    import torch
    if gate.dtype != torch.bfloat16 or gate.device.type != "cuda" or not gate.is_contiguous():
        raise ValueError("gate must be a contiguous bf16 GPU tensor")
    out = torch.empty(gate.shape, dtype=torch.float32, device=gate.device)
    _call("ck_silu_f32", gate.data_ptr(), gate.numel(), out.data_ptr(), _stream(gate))
    return out


def ck_act_rotate_f32(x, input_act=None, group: int = 128, k: int | None = None):
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    act = _act_code(input_act)
    m, ldx = x.shape
    if k is None:
        k = ldx // 2 if act == CK_ACT_SWIGLU else ldx
    _check_group(k, group)
    u = torch.empty((m, k), dtype=torch.float32, device=x.device)
    _call("ck_act_rotate_f32", x.data_ptr(), ldx, m, k, act, group, u.data_ptr(), _stream(x))
    return u


# short aliases
weight_prep = ck_weight_prep
weight_pack = ck_weight_pack
act_quant = ck_act_quant
int8_linear = ck_int8_linear
int8_gemm_bf16 = ck_int8_gemm_bf16
swiglu_mlp = ck_swiglu_mlp
