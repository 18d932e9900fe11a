"""Intake of serialized ConvRot INT8 layers (pre-quantized weights).

Sources: sglang PR #35994 report "[diffusion] Load serialized Comfy ConvRot INT8
DiTs", section "关键源码片段" (key source excerpts):
  * a serialized layer carries final INT8 weights and an F32 per-output-row
    scale of shape [out_features, 1]; the weights are used as they are, with no
    re-quantization at load;
  * before the model is built, every layer marked INT8 must have both its
    weight and weight_scale tensors, the weight must be I8 and 2-D, the scale
    F32 of shape exactly (rows of the weight, 1); anything else is rejected
    with a ValueError naming the layer;
  * in_features must be divisible by the rotation group size.
comfy-kitchen PR #277, "Changes": the INT8 linear is also tested with a scalar
(per-tensor) weight scale, which is taken here as one scale for every row.

The weights in such a checkpoint are already rotated (W_rot = W H^T, group 128
or 256) and quantized, so they enter the path after ck_weight_prep: this
module only validates, expands a scalar scale, and re-lays the codes out for
the GPU kernels.  Host-side only; it calls ck_weight_pack on the device.
"""
from __future__ import annotations

import json

INT8_FORMAT = "int8_tensorwise"
MARKER_SUFFIX = ".comfy_quant"


def check_int8_layer(prefix: str, keys, meta: dict) -> None:
    """Validate one INT8 layer's tensors from checkpoint metadata.

    keys: the checkpoint's tensor names; meta: name -> (dtype string, shape
    tuple) with safetensors dtype names ("I8", "F32", ...)."""
    w_key, s_key = f"{prefix}.weight", f"{prefix}.weight_scale"
    missing = sorted({w_key, s_key} - set(keys))
    if missing:
        raise ValueError(f"INT8 layer {prefix!r}: checkpoint lacks {missing}")
    w_dtype, w_shape = meta[w_key]
    s_dtype, s_shape = meta[s_key]
    if w_dtype != "I8" or s_dtype != "F32":
        raise ValueError(f"INT8 layer {prefix!r}: weight must be I8 and scale F32, "
                         f"found {w_dtype} and {s_dtype}")
    if len(w_shape) != 2:
        raise ValueError(f"INT8 layer {prefix!r}: weight must be 2-D, found shape {tuple(w_shape)}")
    want = (int(w_shape[0]), 1)
    if tuple(int(v) for v in s_shape) != want:
        raise ValueError(f"INT8 layer {prefix!r}: scale must have shape {want}, "
                         f"found {tuple(s_shape)}")


def read_markers(path: str) -> dict:
    """Per-layer quantization markers of a safetensors file: tensors named
    '<prefix>.comfy_quant' holding UTF-8 JSON (a U8 byte vector)."""
    from safetensors import safe_open
    out = {}
    with safe_open(path, framework="numpy") as f:
        for name in f.keys():
            if name.endswith(MARKER_SUFFIX):
                raw = bytes(f.get_tensor(name).tobytes())
                try:
                    out[name[: -len(MARKER_SUFFIX)]] = json.loads(raw.decode("utf-8"))
                except (UnicodeDecodeError, json.JSONDecodeError) as e:
                    raise ValueError(f"layer {name[:-len(MARKER_SUFFIX)]!r}: unreadable "
                                     f"quantization marker ({e})") from None
    return out


def inspect_safetensors(path: str):
    """(keys, meta, markers) of a safetensors file, reading headers only (and
    the small marker tensors); no weight data is loaded."""
    from safetensors import safe_open
    meta = {}
    with safe_open(path, framework="numpy") as f:
        keys = list(f.keys())
        for name in keys:
            sl = f.get_slice(name)
            meta[name] = (sl.get_dtype(), tuple(sl.get_shape()))
    return keys, meta, read_markers(path)


def check_checkpoint(keys, meta: dict, markers: dict) -> list:
    """Validate every layer whose marker says INT8; returns those prefixes."""
    layers = []
    for prefix, marker in markers.items():
        if not isinstance(marker, dict) or marker.get("format") != INT8_FORMAT:
            continue
        check_int8_layer(prefix, keys, meta)
        layers.append(prefix)
    return layers


def serialized_linear_weights(weight, weight_scale, group: int = 128, layout: str = "blocked"):
    """Device tensors of one serialized layer -> (w_q for `layout`, w_scale [n]).

    weight: int8 [out, in] (already rotated and quantized); weight_scale: F32
    [out, 1], [out] or a single value (one scale for all rows).  For
    layout="decode" the scales go inside the packed weight and the second
    result is None."""
    import torch
    import swiglu_mlp_amd as ck
    if not isinstance(weight, torch.Tensor) or weight.dtype != torch.int8 or weight.dim() != 2:
        raise ValueError("serialized weight must be a 2-D int8 tensor")
    if weight.device.type != "cuda":
        raise ValueError(f"serialized weight must be on a GPU, got {weight.device}")
    n, k = weight.shape
    if k % group:
        raise ValueError(f"in_features ({k}) must be divisible by the rotation group {group}")
    if k % 64 or n % 16:
        raise ValueError(f"the GEMM needs in_features % 64 == 0 and out_features % 16 == 0, "
                         f"got ({n}, {k})")
    s = torch.as_tensor(weight_scale)
    if s.dtype != torch.float32:
        raise ValueError(f"weight_scale must be float32, got {s.dtype}")
    if s.numel() == 1:
        s = s.reshape(1).to(weight.device).expand(n)
    elif tuple(s.shape) in ((n, 1), (n,)):
        s = s.reshape(n).to(weight.device)
    else:
        raise ValueError(f"weight_scale must have shape ({n}, 1), ({n},) or be a single value, "
                         f"got {tuple(s.shape)}")
    s = s.contiguous()
    w = weight.contiguous()
    if layout == "blocked":
        w = ck.ck_weight_pack(w)
    elif layout == "decode":
        return ck.ck_weight_pack_decode(w, s), None
    elif layout != "rows":
        raise ValueError(f"unknown layout {layout!r}")
    return w, s
