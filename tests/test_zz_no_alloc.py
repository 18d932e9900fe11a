"""ck_int8_linear_noalloc (the allocation-free linear) against ck_int8_linear
through the C ABI: two calls in a row on one stream, the second smaller, each
bit for bit equal to the workspace call on the same inputs; a size past the
scratch limit is refused before anything is enqueued."""
import ctypes
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
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _case(m, k, n, act, g, layout, seed):
    rng = np.random.default_rng(seed)
    ldx = 2 * k if act else k
    x = torch.from_numpy(W.to_bf16_bits(rng.standard_normal((m, ldx)).astype(np.float32)).view(np.int16))
    x = x.to(DEV).view(torch.bfloat16)
    w = torch.from_numpy((0.02 * rng.standard_normal((n, k))).astype(np.float32)).to(DEV)
    wq, sw = ck.ck_weight_prep(w, g, layout=layout)
    return x, ldx, wq, sw


def _noalloc(L, x, ldx, act, wq, sw, lay, m, n, k, g, y, stream):
    return L.ck_int8_linear_noalloc(x.data_ptr(), ldx, act, wq.data_ptr(),
                                    None if sw is None else sw.data_ptr(), None, None, lay, m, n, k, g,
                                    y.data_ptr(), stream)


def test_noalloc_equals_workspace_call_twice_then_smaller():
    L = ck.lib()
    stream = torch.cuda.current_stream(DEV).cuda_stream
    cases = [  # (m, k, n, act, g, layout): the second is smaller in every dimension
        (2048, 3072, 1024, 1, 128, "blocked"),
        (300, 1024, 512, 0, 64, "blocked"),
        (77, 512, 256, 1, 128, "rows"),
        (2, 3072, 1024, 0, 128, "decode"),
    ]
    for a, b in zip(cases[:-1], cases[1:]):
        outs = []
        for (m, k, n, act, g, layout), seed in ((a, 1), (b, 2)):
            say(f"m={m} k={k} n={n} act={act} g={g} {layout}")
            x, ldx, wq, sw = _case(m, k, n, act, g, layout, seed)
            lay = ck._layout_code(layout)
            y = torch.full((m, n), -1.0, dtype=torch.bfloat16, device=DEV)
            assert _noalloc(L, x, ldx, act, wq, sw, lay, m, n, k, g, y, stream) == 0
            outs.append((y, x, wq, sw, act, g, layout))
        torch.cuda.synchronize()
        for y, x, wq, sw, act, g, layout in outs:
            want = ck.ck_int8_linear(x, wq, sw, g, act, layout=layout)
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16), want.view(torch.int16)), layout


def test_noalloc_split_k_twice_then_smaller():
    """Few-tile blocked shapes take split K, with the int32 partials in the
    scratch past the codes: two calls in a row, the second smaller, each equal
    to the workspace call (which splits the same way)."""
    L = ck.lib()
    stream = torch.cuda.current_stream(DEV).cuda_stream
    outs = []
    for (m, k, n, act, g), seed in (((256, 12288, 3072, 1, 128), 3), ((64, 8192, 2048, 0, 64), 4)):
        assert L.ck_int8_linear_workspace_size(m, k, n) > ck._linear_codes_bytes(m, k), "meant to split"
        say(f"split-k m={m} k={k} n={n} act={act} g={g}")
        x, ldx, wq, sw = _case(m, k, n, act, g, "blocked", seed)
        y = torch.full((m, n), -1.0, dtype=torch.bfloat16, device=DEV)
        assert _noalloc(L, x, ldx, act, wq, sw, 1, m, n, k, g, y, stream) == 0
        outs.append((y, x, wq, sw, act, g))
    torch.cuda.synchronize()
    for y, x, wq, sw, act, g in outs:
        want = ck.ck_int8_linear(x, wq, sw, g, act, layout="blocked")
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16))


def test_noalloc_refuses_past_the_scratch():
    L = ck.lib()
    cap = L.ck_noalloc_scratch_bytes()
    k = 16384
    m = cap // k + 1                  # the codes alone exceed the scratch
    assert L.ck_int8_linear_workspace_size(m, k, 16) > cap
    y = torch.empty((m, 16), dtype=torch.bfloat16, device=DEV)
    x = torch.zeros((m, k), dtype=torch.bfloat16, device=DEV)
    wq = torch.zeros((16, k), dtype=torch.int8, device=DEV)
    sw = torch.ones(16, dtype=torch.float32, device=DEV)
    st = L.ck_int8_linear_noalloc(x.data_ptr(), k, 0, wq.data_ptr(), sw.data_ptr(), None, None, 0, m, 16,
                                  k, 128, y.data_ptr(), None)
    assert st == 4  # CK_EWORKSPACE
    with pytest.raises(ValueError):
        ck.ck_int8_linear_noalloc(x, wq, sw, 128, out=y, layout="rows")
