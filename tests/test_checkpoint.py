"""Serialized INT8 layer intake (sglang PR #35994 report, key source excerpts:
I8 weight + F32 [out, 1] row scale, validated before the model is built)."""
import json
import os

import numpy as np
import pytest

from swiglu_mlp_amd import checkpoint as C


def meta_of(w_dtype="I8", w_shape=(64, 256), s_dtype="F32", s_shape=(64, 1)):
    return {"blk.0.fc.weight": (w_dtype, w_shape), "blk.0.fc.weight_scale": (s_dtype, s_shape)}


def test_valid_layer_passes():
    m = meta_of()
    C.check_int8_layer("blk.0.fc", m.keys(), m)


@pytest.mark.parametrize("kw,msg", [
    (dict(w_dtype="F16"), "I8"), (dict(s_dtype="BF16"), "F32"), (dict(w_shape=(64, 16, 16)), "2-D"),
    (dict(s_shape=(64,)), r"\(64, 1\)"), (dict(s_shape=(32, 1)), r"\(64, 1\)"),
])
def test_contract_violations_raise(kw, msg):
    m = meta_of(**kw)
    with pytest.raises(ValueError, match=msg):
        C.check_int8_layer("blk.0.fc", m.keys(), m)


def test_missing_tensor_raises():
    m = meta_of()
    del m["blk.0.fc.weight_scale"]
    with pytest.raises(ValueError, match="lacks"):
        C.check_int8_layer("blk.0.fc", m.keys(), m)


def test_only_int8_marked_layers_are_checked():
    m = meta_of(s_shape=(64,))             # broken, but marked as another format
    assert C.check_checkpoint(m.keys(), m, {"blk.0.fc": {"format": "float8_e4m3fn"}}) == []
    with pytest.raises(ValueError):
        C.check_checkpoint(m.keys(), m, {"blk.0.fc": {"format": "int8_tensorwise"}})


def test_safetensors_round_trip(tmp_path):
    from safetensors.numpy import save_file
    marker = np.frombuffer(json.dumps({"format": "int8_tensorwise"}).encode(), dtype=np.uint8)
    good = {"a.weight": np.zeros((32, 128), np.int8), "a.weight_scale": np.ones((32, 1), np.float32),
            "a.comfy_quant": marker.copy(), "b.weight": np.zeros((8, 8), np.float32)}
    p = os.path.join(tmp_path, "good.safetensors")
    save_file(good, p)
    keys, meta, markers = C.inspect_safetensors(p)
    assert meta["a.weight"] == ("I8", (32, 128)) and markers == {"a": {"format": "int8_tensorwise"}}
    assert C.check_checkpoint(keys, meta, markers) == ["a"]
    bad = dict(good)
    bad["a.weight_scale"] = np.ones((32,), np.float32)
    p2 = os.path.join(tmp_path, "bad.safetensors")
    save_file(bad, p2)
    with pytest.raises(ValueError, match="shape"):
        C.check_checkpoint(*C.inspect_safetensors(p2))


def test_serialized_weights_rejects_host_and_bad_shapes():
    import torch
    with pytest.raises(ValueError, match="GPU"):
        C.serialized_linear_weights(torch.zeros((16, 128), dtype=torch.int8), torch.ones(16, 1))
    with pytest.raises(ValueError, match="int8"):
        C.serialized_linear_weights(torch.zeros((16, 128)), torch.ones(16, 1))
