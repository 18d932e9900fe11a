"""MI355X (gfx950) ConvRot INT8 linear and SwiGLU MLP: Python binding.

This module only marshals arguments: it checks dtypes and shapes, takes device
pointers and the current HIP stream from torch tensors, and calls the C ABI of
``libck_convrot.so`` (declared in ``include/ck.h``).  Every step of the path
runs in that library's HIP kernels; there is no fallback.  If the library is
missing, importing any entry point raises.

Entry points keep the C names:

* ``ck_weight_prep(w, group, layout="blocked")`` -> (w_q int8, w_scale f32 [n, 1])
* ``ck_weight_pack(w_q)``                 -> w_q in the blocked layout
* ``ck_weight_pack_decode(w_q, w_scale)`` -> codes and scales in the decode layout
* ``ck_act_quant(x, act, group, k=None, layout="blocked")`` -> (x_q, x_scale f32 [m, 1])
* ``ck_int8_linear(x, w_q, w_scale, group, input_act=None, layout=None, bias=None, residual=None)``
* ``ck_int8_linear_noalloc(x, w_q, w_scale, group, input_act=None, out=..., ...)``: the same
  linear with no workspace (the library's own device scratch), for callers that
  cannot allocate
* ``ck_int8_gemm_bf16(x_q, x_scale, w_q, w_scale, layout=None, bias=None, residual=None)``
* ``ck_swiglu_mlp(x, w_gu, s_gu, w_down, s_down, group, layout=None)`` -> y bf16
* W8A16 (BF16 activations, INT8 weights in the blocked layout):
  ``ck_act_rotate_bf16``, ``ck_w8a16_gemm_bf16``, ``ck_int8_linear_w8a16``,
  ``ck_swiglu_mlp_w8a16``
* test hooks ``ck_int8_gemm_i32``, ``ck_w8a16_gemm_f32``, ``ck_silu_f32``, ``ck_act_rotate_f32``

INT8 operand layouts, each with its own tensor form so that a call can tell
them apart:

* blocked (the GEMMs' fast path, include/ck.h ``CK_LAYOUT_BLOCKED``): int8
  ``[R / 32, k / 32, 1024]`` with R the row count padded to 256; entry (i, j)
  is the 1 KB MFMA operand block of rows 32 i .. 32 i + 31 and columns
  32 j .. 32 j + 31.  ``ck_weight_prep`` and ``ck_act_quant`` return it by
  default, so ``ck_int8_linear(x, *ck_weight_prep(w))`` runs the blocked GEMM.
* row-major (``layout="rows"``): int8 ``[rows, k]``, the serialized checkpoint
  format.
* decode (weights only, at most 64 token rows): uint8 ``[n / 16, 64 + 16 k]``,
  each 16-row group of the weight one linear stream with its row scales in
  front; its ``w_scale`` argument is None and the activation codes are blocked.

With ``layout=None`` (the default of the linear, GEMM and MLP calls) the layout
is read off the weight tensor; an explicit ``layout`` string also accepts a
blocked operand as the same bytes viewed ``[R, k]``.  With blocked operands the
logical row counts come from the scale vectors.  ``out`` must be a contiguous
BF16 tensor of the output's shape on the input's device that shares no memory
with the inputs (it may be the residual itself).

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
        "ck_int8_linear_noalloc": [p, i64, i32, p, p, p, p, i32, i64, i64, i64, i32, p, p],
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
        "ck_probe_mfma_i8": [p, i64, i32, p, p],
        "ck_probe_stream_rows": [p, i64, i64, i64, i64, p, p],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.ck_int8_linear_workspace_size.argtypes = [i64, i64, i64]
    L.ck_int8_linear_workspace_size.restype = sz
    L.ck_int8_linear_w8a16_workspace_size.argtypes = [i64, i64]
    L.ck_int8_linear_w8a16_workspace_size.restype = sz
    L.ck_swiglu_mlp_w8a16_workspace_size.argtypes = [i64, i64, i64]
    L.ck_swiglu_mlp_w8a16_workspace_size.restype = sz
    L.ck_swiglu_mlp_workspace_size.argtypes = [i64, i64, i64]
    L.ck_swiglu_mlp_workspace_size.restype = sz
    L.ck_probe_mfma_workgroups.argtypes = []
    L.ck_probe_mfma_workgroups.restype = i64
    L.ck_noalloc_scratch_bytes.argtypes = []
    L.ck_noalloc_scratch_bytes.restype = sz
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


def _weight_layout(layout, w):
    """The layout code of a weight operand: `layout` when given, else read off
    the tensor (3-D int8: blocked; 2-D uint8: decode; 2-D int8: row-major)."""
    import torch
    if layout is not None:
        return _layout_code(layout)
    if not isinstance(w, torch.Tensor):
        raise ValueError("weight must be a torch.Tensor")
    if w.dtype == torch.uint8:
        return CK_LAYOUT_DECODE
    return CK_LAYOUT_BLOCKED if w.dim() == 3 else CK_LAYOUT_ROWS


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


def _operand(t, rows, layout, what):
    """Check an int8 operand holds `rows` logical rows in `layout`; returns k.
    Row-major: [rows, k].  Blocked: [R / 32, k / 32, 1024] (one 1 KB block
    per entry), or the same bytes as [R, k], with R = blocked_rows(rows)."""
    import torch
    if layout == CK_LAYOUT_ROWS:
        _need(t, torch.int8, 2, what)
        if t.shape[0] != rows:
            raise ValueError(f"{what} needs {rows} rows in the row-major layout, got {t.shape[0]}")
        return t.shape[1]
    need = blocked_rows(rows)
    if isinstance(t, torch.Tensor) and t.dim() == 3:
        _need(t, torch.int8, 3, what)
        if t.shape[0] * 32 != need or t.shape[2] != 1024:
            raise ValueError(f"{what} needs shape ({need // 32}, k / 32, 1024) for {rows} logical rows "
                             f"in the blocked layout, got {tuple(t.shape)}")
        return t.shape[1] * 32
    _need(t, torch.int8, 2, what)
    if t.shape[0] != need:
        raise ValueError(f"{what} needs {need} rows for {rows} logical rows in the blocked layout, "
                         f"got {t.shape[0]}")
    return t.shape[1]


def _weight(w, w_scale, lay, what):
    """(n, k) of a weight operand in layout `lay`, with its scale checked."""
    if lay == CK_LAYOUT_DECODE:
        n, k = _decode_shape(w, what)
        if w_scale is not None:
            raise ValueError(f"{what}: the decode layout carries its scales; pass w_scale=None")
        return n, k
    if w_scale is None:
        raise ValueError(f"{what}: weight scale missing")
    n = w_scale.shape[0]
    _scale(w_scale, n, what + " scale")
    return n, _operand(w, n, lay, what)


def _act_layout(lay):
    """Layout of the activation codes that go with a weight in layout `lay`."""
    return CK_LAYOUT_ROWS if lay == CK_LAYOUT_ROWS else CK_LAYOUT_BLOCKED


def _ptr(t):
    return None if t is None else t.data_ptr()


def _span(t):
    a = t.data_ptr()
    return a, a + t.numel() * t.element_size()


def _overlaps(a, b):
    (a0, a1), (b0, b1) = _span(a), _span(b)
    return a0 < b1 and b0 < a1


def _out(out, m, n, dev, inputs, residual=None):
    """The BF16 [m, n] output: a new tensor, or `out` checked for dtype, shape,
    device and contiguity.  It may not share memory with any of `inputs` (the
    kernels read those while y is written); it may be the residual itself."""
    import torch
    if out is None:
        return torch.empty((m, n), dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, 2, "out")
    if tuple(out.shape) != (m, n) or out.device != dev:
        raise ValueError(f"out needs a contiguous ({m}, {n}) bfloat16 tensor on {dev}, "
                         f"got {tuple(out.shape)} on {out.device}")
    for name, t in inputs:
        if t is not None and out.numel() and t.numel() and _overlaps(out, t):
            raise ValueError(f"out must not share memory with {name}")
    if residual is not None and _overlaps(out, residual) and residual.data_ptr() != out.data_ptr():
        raise ValueError("residual must be out itself or not overlap it")
    return out


def _workspace(ws, nbytes, dev, min_bytes=None):
    """A caller's workspace: a contiguous uint8 tensor on `dev` of at least
    `min_bytes` bytes (default `nbytes`; a new one of `nbytes` when None)."""
    import torch
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(ws, torch.uint8, 1, "workspace")
    if ws.device != dev:
        raise ValueError(f"workspace must be on {dev}, got {ws.device}")
    need = nbytes if min_bytes is None else min_bytes
    if ws.numel() < need:
        raise ValueError(f"workspace needs {need} bytes, got {ws.numel()}")
    return ws


def _round256(v: int) -> int:
    return (v + 255) // 256 * 256


def _linear_codes_bytes(m: int, k: int) -> int:
    """The part of ck_int8_linear's workspace that holds the activation codes
    and row scales (the least it accepts; the rest is room for split-K
    partials)."""
    return _round256(lib().ck_blocked_size(m, k)) + _round256(4 * m)


def _act_code(input_act):
    if input_act in (None, "none", CK_ACT_NONE):
        return CK_ACT_NONE
    if input_act in ("swiglu", CK_ACT_SWIGLU):
        return CK_ACT_SWIGLU
    raise ValueError(f"unknown input_act {input_act!r}")


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def ck_weight_prep(w, group: int = 128, layout="blocked"):
    """Rotate and quantize an FP32 weight [n, k] -> (w_q, w_scale [n, 1]).
    layout "blocked" (default, the GEMMs' fast path): w_q [R / 32, k / 32, 1024];
    "rows": row-major [n, k] (the serialized checkpoint format); "decode":
    (uint8 [n / 16, 64 + 16 k] with the scales inside, None)."""
    import torch
    _need(w, torch.float32, 2, "weight")
    lay = _layout_code(layout)
    n, k = w.shape
    _check_group(k, group)
    w_q = torch.empty((n, k), dtype=torch.int8, device=w.device)
    w_scale = torch.empty((n, 1), dtype=torch.float32, device=w.device)
    _call("ck_weight_prep", w.data_ptr(), n, k, group, w_q.data_ptr(), w_scale.data_ptr(),
          _stream(w))
    if lay == CK_LAYOUT_BLOCKED:
        return ck_weight_pack(w_q), w_scale
    if lay == CK_LAYOUT_DECODE:
        return ck_weight_pack_decode(w_q, w_scale), None
    return w_q, w_scale


def ck_weight_pack(w_q):
    """Relayout row-major int8 weight codes [n, k] into the blocked layout,
    returned as [R / 32, k / 32, 1024] (R = blocked_rows(n)): entry (i, j) is
    the 1 KB block of rows 32 i .. 32 i + 31 and columns 32 j .. 32 j + 31."""
    import torch
    _need(w_q, torch.int8, 2, "weight")
    n, k = w_q.shape
    if k % 64:
        raise ValueError(f"in_features must be a multiple of 64, got {k}")
    out = torch.empty((blocked_rows(n) // 32, k // 32, 1024), dtype=torch.int8, device=w_q.device)
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


def ck_act_quant(x, input_act=None, group: int = 128, k: int | None = None, layout="blocked"):
    """Activation codes and per-row scales (x_q, x_scale [m, 1]).  layout
    "blocked" (default): x_q [R / 32, k / 32, 1024], the operand form of the
    blocked GEMMs; "rows": row-major [m, k]."""
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    act = _act_code(input_act)
    lay = _layout_code(layout)
    if lay == CK_LAYOUT_DECODE:
        raise ValueError("activation codes use the rows or blocked layout")
    m, ldx = x.shape
    if k is None:
        k = ldx // 2 if act == CK_ACT_SWIGLU else ldx
    _check_group(k, group)
    if lay == CK_LAYOUT_ROWS:
        x_q = torch.empty((m, k), dtype=torch.int8, device=x.device)
    else:
        if k % 64:
            raise ValueError(f"in_features must be a multiple of 64, got {k}")
        x_q = torch.empty((blocked_rows(m) // 32, k // 32, 1024), dtype=torch.int8, device=x.device)
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
                   workspace=None, layout=None, bias=None, residual=None):
    """y = int8_linear(x) (+ bias + residual).  layout None: read off w_q (a
    blocked weight from ck_weight_prep / ck_weight_pack is 3-D)."""
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    lay = _weight_layout(layout, w_q)
    n, k = _weight(w_q, w_scale, lay, "weight")
    act = _act_code(input_act)
    m, ldx = x.shape
    need_ld = 2 * k if act == CK_ACT_SWIGLU else k
    if ldx != need_ld:
        raise ValueError(f"activation needs {need_ld} columns for in_features {k}, got {ldx}")
    _check_group(k, group)
    bp, rp = _extra(bias, residual, m, n, x.device)
    y = _out(out, m, n, x.device, [("the activation", x), ("the weight", w_q), ("the weight scale", w_scale),
                                   ("the bias", bias)], residual)
    ws = _workspace(workspace, lib().ck_int8_linear_workspace_size(m, k, n), x.device, _linear_codes_bytes(m, k))
    _call("ck_int8_linear", x.data_ptr(), ldx, act, w_q.data_ptr(), _ptr(w_scale), bp, rp,
          lay, m, n, k, group, y.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x))
    return y


def ck_int8_linear_noalloc(x, w_q, w_scale, group: int = 128, input_act=None, out=None,
                           layout=None, bias=None, residual=None):
    """ck_int8_linear with its codes and scales in the library's own device
    scratch (no workspace; ck_noalloc_scratch_bytes() per GPU).  Calls that
    overlap on one GPU race on that scratch; calls in one stream are ordered."""
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    lay = _weight_layout(layout, w_q)
    n, k = _weight(w_q, w_scale, lay, "weight")
    act = _act_code(input_act)
    m, ldx = x.shape
    need_ld = 2 * k if act == CK_ACT_SWIGLU else k
    if ldx != need_ld:
        raise ValueError(f"activation needs {need_ld} columns for in_features {k}, got {ldx}")
    _check_group(k, group)
    if _linear_codes_bytes(m, k) > lib().ck_noalloc_scratch_bytes():
        raise ValueError(f"m = {m}, k = {k} needs more than the {lib().ck_noalloc_scratch_bytes()} "
                         "bytes of scratch; use ck_int8_linear with a workspace")
    bp, rp = _extra(bias, residual, m, n, x.device)
    if out is None:
        raise ValueError("ck_int8_linear_noalloc allocates nothing: pass out")
    y = _out(out, m, n, x.device, [("the activation", x), ("the weight", w_q), ("the weight scale", w_scale),
                                   ("the bias", bias)], residual)
    _call("ck_int8_linear_noalloc", x.data_ptr(), ldx, act, w_q.data_ptr(), _ptr(w_scale), bp, rp,
          lay, m, n, k, group, y.data_ptr(), _stream(x))
    return y


def ck_int8_gemm_bf16(x_q, x_scale, w_q, w_scale, out=None, layout=None, bias=None,
                      residual=None):
    import torch
    lay = _weight_layout(layout, w_q)
    m = x_scale.shape[0]
    _scale(x_scale, m, "activation scale")
    k = _operand(x_q, m, _act_layout(lay), "activation codes")
    n, kw = _weight(w_q, w_scale, lay, "weight")
    if kw != k:
        raise ValueError(f"in_features mismatch: activation {k}, weight {kw}")
    bp, rp = _extra(bias, residual, m, n, x_q.device)
    y = _out(out, m, n, x_q.device, [("the activation codes", x_q), ("the activation scale", x_scale),
                                     ("the weight", w_q), ("the weight scale", w_scale), ("the bias", bias)],
             residual)
    _call("ck_int8_gemm_bf16", x_q.data_ptr(), x_scale.data_ptr(), w_q.data_ptr(),
          _ptr(w_scale), bp, rp, lay, m, n, k, y.data_ptr(), _stream(x_q))
    return y


def ck_swiglu_mlp(x, w_gu, s_gu, w_down, s_down, group: int = 128, out=None, workspace=None,
                  layout=None):
    """The SwiGLU MLP block.  layout None: read off w_gu (both weights must
    share it)."""
    import torch
    _need(x, torch.bfloat16, 2, "activation")
    lay = _weight_layout(layout, w_gu)
    if layout is None and _weight_layout(None, w_down) != lay:
        raise ValueError("gate_up and down weights must use the same layout")
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
    y = _out(out, m, h, x.device, [("the activation", x), ("the gate_up weight", w_gu), ("its scale", s_gu),
                                   ("the down weight", w_down), ("its scale", s_down)])
    ws = _workspace(workspace, lib().ck_swiglu_mlp_workspace_size(m, h, i), x.device)
    if _overlaps(ws, y) or _overlaps(ws, x):
        raise ValueError("the workspace must not share memory with the activation or out")
    _call("ck_swiglu_mlp", x.data_ptr(), w_gu.data_ptr(), _ptr(s_gu), w_down.data_ptr(),
          _ptr(s_down), lay, m, h, i, group, y.data_ptr(), ws.data_ptr(),
          ws.numel(), _stream(x))
    return y


def ck_int8_gemm_i32(x_q, w_q, layout=None, m: int | None = None, n: int | None = None):
    """Raw int32 accumulators; with blocked operands pass the logical m and n."""
    import torch
    lay = _weight_layout(layout, w_q)
    if m is None:
        if lay != CK_LAYOUT_ROWS:
            raise ValueError("blocked activation codes need the logical row count m")
        m = x_q.shape[0]
    k = _operand(x_q, m, _act_layout(lay), "activation codes")
    if lay == CK_LAYOUT_DECODE:
        n, kw = _decode_shape(w_q, "weight")
    else:
        if n is None:
            if lay != CK_LAYOUT_ROWS:
                raise ValueError("a blocked weight needs the logical row count n")
            n = w_q.shape[0]
        kw = _operand(w_q, n, lay, "weight")
    if kw != k:
        raise ValueError(f"in_features mismatch: activation {k}, weight {kw}")
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
    k = x_rot.shape[1]
    if x_rot.shape[0] != blocked_rows(m):
        raise ValueError(f"rotated activation needs {blocked_rows(m)} rows for {m} logical rows in "
                         f"the blocked layout, got {x_rot.shape[0]}")
    kw = _operand(w_q, n, CK_LAYOUT_BLOCKED, "weight")
    if kw != k:
        raise ValueError(f"in_features mismatch: activation {k}, weight {kw}")
    return k


def ck_w8a16_gemm_bf16(x_rot, w_q, w_scale, m: int, out=None, bias=None, residual=None):
    """y = bf16(acc * w_scale (+ bias) (+ residual)); x_rot in the BF16 blocked
    layout with m logical rows, w_q blocked."""
    n = w_scale.shape[0]
    _scale(w_scale, n, "weight_scale")
    k = _w8a16_operands(x_rot, w_q, m, n)
    bp, rp = _extra(bias, residual, m, n, x_rot.device)
    y = _out(out, m, n, x_rot.device, [("the rotated activation", x_rot), ("the weight", w_q),
                                       ("the weight scale", w_scale), ("the bias", bias)], residual)
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
    n = w_scale.shape[0]
    _scale(w_scale, n, "weight_scale")
    k = _operand(w_q, n, CK_LAYOUT_BLOCKED, "weight")
    act = _act_code(input_act)
    m, ldx = x.shape
    need_ld = 2 * k if act == CK_ACT_SWIGLU else k
    if ldx != need_ld:
        raise ValueError(f"activation needs {need_ld} columns for in_features {k}, got {ldx}")
    _check_group(k, group)
    bp, rp = _extra(bias, residual, m, n, x.device)
    y = _out(out, m, n, x.device, [("the activation", x), ("the weight", w_q), ("the weight scale", w_scale),
                                   ("the bias", bias)], residual)
    ws = _workspace(workspace, lib().ck_int8_linear_w8a16_workspace_size(m, k), x.device)
    _call("ck_int8_linear_w8a16", x.data_ptr(), ldx, act, w_q.data_ptr(), w_scale.data_ptr(), bp, rp,
          m, n, k, group, y.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x))
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
    y = _out(out, m, h, x.device, [("the activation", x), ("the gate_up weight", w_gu), ("its scale", s_gu),
                                   ("the down weight", w_down), ("its scale", s_down)])
    ws = _workspace(workspace, lib().ck_swiglu_mlp_w8a16_workspace_size(m, h, i), x.device)
    if _overlaps(ws, y) or _overlaps(ws, x):
        raise ValueError("the workspace must not share memory with the activation or out")
    _call("ck_swiglu_mlp_w8a16", x.data_ptr(), w_gu.data_ptr(), s_gu.data_ptr(), w_down.data_ptr(),
          s_down.data_ptr(), m, h, i, group, y.data_ptr(), ws.data_ptr(), ws.numel(),
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
