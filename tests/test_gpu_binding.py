"""The Python binding on the GPU: the default (blocked) path and the argument
checks that must raise ValueError before anything is launched."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import swiglu_mlp_amd as ck  # noqa: E402
from swiglu_mlp_amd import workloads as W  # noqa: E402

DEV = "cuda:0"


def say(msg):
    print(f"[gpu-binding] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(a_u16):
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.mark.parametrize("name", ["c1", "c2"])
def test_default_path_is_blocked_and_bit_exact(orc, name):
    """ck_int8_linear(x, *ck_weight_prep(w)) takes the blocked layout (the
    weight comes back as [R / 32, k / 32, 1024]) and equals the oracle."""
    wl = W.WORKLOADS[name]
    d = W.linear_inputs(wl)
    say(f"default path {name}")
    wq, sw = ck.ck_weight_prep(dev(d["w"]), wl.group)
    assert wq.dim() == 3 and wq.shape[2] == 1024
    y = bf16_host(ck.ck_int8_linear(bf16_dev(d["x"]), wq, sw, wl.group, wl.act))
    wq_o, sw_o = orc.weight_prep(d["w"], wl.group)
    np.testing.assert_array_equal(y, orc.int8_linear(d["x"], wl.act, wq_o, sw_o, wl.group))
    # the same weight row-major, and the GEMM fed by the default act_quant
    wr, sr = ck.ck_weight_prep(dev(d["w"]), wl.group, layout="rows")
    y_rows = bf16_host(ck.ck_int8_linear(bf16_dev(d["x"]), wr, sr, wl.group, wl.act))
    np.testing.assert_array_equal(y_rows, y)
    xq, sx = ck.ck_act_quant(bf16_dev(d["x"]), wl.act, wl.group)
    np.testing.assert_array_equal(bf16_host(ck.ck_int8_gemm_bf16(xq, sx, wq, sw)), y)


def test_default_mlp_and_decode_prep(orc):
    m, h, i, g = 40, 256, 512, 128
    wl = W.Workload("bind", "mlp", m, h, i, 1, 0.02, sigma_down=0.01, seed=5)
    d = W.mlp_inputs(wl)
    say("default swiglu_mlp, decode prep")
    x = bf16_dev(d["x"])
    y = bf16_host(ck.ck_swiglu_mlp(x, *ck.ck_weight_prep(dev(d["w_gu"]), g),
                                   *ck.ck_weight_prep(dev(d["w_down"]), g), g))
    gq, gs = orc.weight_prep(d["w_gu"], g)
    dq, ds = orc.weight_prep(d["w_down"], g)
    np.testing.assert_array_equal(y, orc.swiglu_mlp(d["x"], gq, gs, dq, ds, g))
    y_dec = bf16_host(ck.ck_swiglu_mlp(x, *ck.ck_weight_prep(dev(d["w_gu"]), g, layout="decode"),
                                       *ck.ck_weight_prep(dev(d["w_down"]), g, layout="decode"), g))
    np.testing.assert_array_equal(y_dec, y)


def _linear_args():
    rng = np.random.default_rng(3)
    m, k, n = 8, 256, 64
    x = bf16_dev(W.to_bf16_bits(rng.standard_normal((m, k)).astype(np.float32)))
    wq, sw = ck.ck_weight_prep(dev((0.02 * rng.standard_normal((n, k))).astype(np.float32)), 128)
    return x, wq, sw, m, n


def test_out_checked_before_launch():
    x, wq, sw, m, n = _linear_args()
    say("out= checks")
    bad = [torch.empty((m, n), dtype=torch.float32, device=DEV),          # dtype
           torch.empty((m, n - 16), dtype=torch.bfloat16, device=DEV),    # too small
           torch.empty((m + 1, n), dtype=torch.bfloat16, device=DEV),     # wrong shape
           torch.empty((n, m), dtype=torch.bfloat16, device=DEV).t(),     # not contiguous
           torch.empty((m, n), dtype=torch.bfloat16)]                     # host memory
    for out in bad:
        with pytest.raises(ValueError):
            ck.ck_int8_linear(x, wq, sw, 128, out=out)
    # y may not alias the activation (k == n here, so the shapes agree)
    xs = x[:, :n].contiguous()
    wsq, ssw = ck.ck_weight_prep(torch.zeros((n, n), dtype=torch.float32, device=DEV), 64)
    with pytest.raises(ValueError, match="activation"):
        ck.ck_int8_linear(xs, wsq, ssw, 64, out=xs)
    # the residual may be out itself, but not partly overlap it
    buf = torch.zeros((2 * m, n), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError, match="residual"):
        ck.ck_int8_linear(x, wq, sw, 128, out=buf[:m], residual=buf[m // 2: m // 2 + m])
    y = torch.zeros((m, n), dtype=torch.bfloat16, device=DEV)
    ck.ck_int8_linear(x, wq, sw, 128, out=y, residual=y)
    torch.cuda.synchronize()


def test_workspace_and_layout_checked_before_launch():
    x, wq, sw, m, n = _linear_args()
    say("workspace and layout checks")
    with pytest.raises(ValueError):
        ck.ck_int8_linear(x, wq, sw, 128, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    with pytest.raises(ValueError):
        ck.ck_int8_linear(x, wq, sw, 128, workspace=torch.empty(1 << 20, dtype=torch.float32, device=DEV))
    # a blocked weight handed over as row-major has the wrong row count
    with pytest.raises(ValueError):
        ck.ck_int8_linear(x, wq.view(-1, wq.shape[1] * 32), sw, 128, layout="rows")
    # row-major activation codes with a blocked weight
    xq, sx = ck.ck_act_quant(x, None, 128, layout="rows")
    with pytest.raises(ValueError):
        ck.ck_int8_gemm_bf16(xq, sx, wq, sw)
