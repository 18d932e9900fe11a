"""GPU route grids: every kernel route of the activation quantizer, the BF16
rotation, the linear and the MLP blocks, over shape grids that straddle each
route's size thresholds (k from the group to CK_MAX_K, m from 1 to 8192).

Every call must succeed (a route whose launcher cannot take a shape it was
given returns an error status, which the binding raises); the calls small
enough for the CPU oracle to finish in milliseconds are compared with it bit
for bit (W8A16 blocks: finite outputs only, their parity against the derived
bound is in test_gpu_parity.py).  Inputs are seeded draws on the device; the
oracle gets the same values copied to the host.
"""
import itertools
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import swiglu_mlp_amd as ck  # noqa: E402

DEV = "cuda:0"


def say(msg):
    print(f"[gpu-routes] {msg}", flush=True)
    sys.stdout.flush()


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_blocked(b, rows):
    """The int8 blocked layout of include/ck.h back to row-major [rows, k]."""
    if b.ndim == 3:
        b = b.reshape(b.shape[0] * 32, b.shape[1] * 32)
    rp, k = b.shape
    a = b.reshape(rp // 32, k // 32, 2, 32, 16).transpose(0, 3, 1, 2, 4).reshape(rp, k)
    return np.ascontiguousarray(a[:rows])


def from_blocked_bf16(b, rows):
    """The BF16 blocked layout of include/ck.h back to row-major [rows, k]."""
    rp, k = b.shape
    a = b.reshape(rp // 32, k // 32, 2, 2, 32, 8).transpose(0, 4, 1, 3, 2, 5).reshape(rp, k)
    return np.ascontiguousarray(a[:rows])


@pytest.fixture(scope="module")
def pool():
    """512 Mi seeded BF16 values (1 GiB) that the grids slice their inputs from."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5)
    half = (torch.randn(1 << 28, device=DEV, generator=gen) * 2).to(torch.bfloat16)
    return torch.cat([half, half.flip(0)])


@pytest.mark.parametrize("act,g", list(itertools.product((0, 1), (64, 128, 256))))
def test_quant_and_rotate_routes(orc, pool, act, g):
    calls = checked = 0
    for k in sorted({g, 512, 1024, 3072, 4096, 6656, 8192, 12288, 16384, 24576, 26624, 32768}):
        for m in (1, 3, 64, 300, 512, 1024, 2047, 2048, 3000, 4096, 8192):
            ld = 2 * k if act else k
            if m * ld * 2 >= (1 << 30):
                continue
            x = pool[: m * ld].view(m, ld)
            small = m * k <= (1 << 21)
            xh = u16(x) if small else None
            for lay in ("rows", "blocked"):
                what = f"act={act} g={g} k={k} m={m} {lay}"
                q, s = ck.ck_act_quant(x, act, g, k=k, layout=lay)
                r = ck.ck_act_rotate_bf16(x, act, g, k=k, layout=lay)
                torch.cuda.synchronize()
                calls += 2
                if not small:
                    continue
                q_o, s_o = orc.act_quant(xh, act, g, k=k)
                qh = q.cpu().numpy()
                rh = u16(r)
                if lay == "blocked":
                    qh, rh = from_blocked(qh, m), from_blocked_bf16(rh, m)
                np.testing.assert_array_equal(qh, q_o, err_msg=what)
                np.testing.assert_array_equal(s.cpu().numpy().reshape(-1).view(np.uint32), s_o.view(np.uint32),
                                              err_msg=what)
                np.testing.assert_array_equal(rh, orc.act_rotate_bf16(xh, act, g, k=k), err_msg=what)
                checked += 1
    say(f"act={act} g={g}: {calls} calls, {checked} compared with the oracle")


@pytest.mark.parametrize("k", [128, 256, 1024, 3072, 8192, 12288, 32768])
def test_linear_routes(orc, k):
    g = 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11 + k)
    calls = checked = 0
    for n in (16, 48, 128, 1024, 4112, 8192, 24576):
        if n * k > (1 << 28):
            continue
        wq = torch.randint(-127, 128, (n, k), device=DEV, generator=gen, dtype=torch.int32).to(torch.int8)
        sw = (torch.rand(n, device=DEV, generator=gen) * 1e-3 + 1e-4).float()
        weights = {"rows": (wq, sw), "blocked": (ck.ck_weight_pack(wq), sw),
                   "decode": (ck.ck_weight_pack_decode(wq, sw) if n % 16 == 0 else None, None)}
        wq_h, sw_h = wq.cpu().numpy(), sw.cpu().numpy()
        for m, act in itertools.product((1, 2, 3, 16, 33, 64, 65, 128, 129, 512, 1024, 2048, 4096), (0, 1)):
            ld = 2 * k if act else k
            if m * ld * 2 >= (1 << 30) or m * n * 2 >= (1 << 30):
                continue
            x = (torch.randn(m, ld, device=DEV, generator=gen) * 2).to(torch.bfloat16)
            bias = torch.randn(n, device=DEV, generator=gen).float()
            res = torch.randn(m, n, device=DEV, generator=gen).to(torch.bfloat16)
            small = m * n * k <= (1 << 27) and m * k <= (1 << 22)
            want = want_br = None
            if small:
                q_o, s_o = orc.act_quant(u16(x), act, g, k=k)
                acc = orc.gemm_i32(q_o, wq_h)
                want = orc.epilogue(acc, s_o, sw_h)
                want_br = orc.epilogue(acc, s_o, sw_h, bias.cpu().numpy(), u16(res))
            for lay, (w, s) in weights.items():
                if lay == "decode" and (m > 64 or w is None):
                    continue
                y = ck.ck_int8_linear(x, w, s, g, act, layout=lay)
                y_br = ck.ck_int8_linear(x, w, s, g, act, layout=lay, bias=bias, residual=res)
                torch.cuda.synchronize()
                calls += 2
                if small:
                    what = f"m={m} k={k} n={n} act={act} {lay}"
                    np.testing.assert_array_equal(u16(y), want, err_msg=what)
                    np.testing.assert_array_equal(u16(y_br), want_br, err_msg=what + " + bias + residual")
                    checked += 2
    say(f"k={k}: {calls} calls, {checked} compared with the oracle")


@pytest.mark.parametrize("h", [256, 1024, 3072])
def test_mlp_routes(orc, h):
    g = 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(13 + h)
    calls = checked = 0
    for i in (512, 3072, 12288):
        wgu = torch.randint(-127, 128, (2 * i, h), device=DEV, generator=gen, dtype=torch.int32).to(torch.int8)
        sgu = (torch.rand(2 * i, device=DEV, generator=gen) * 1e-3 + 1e-4).float()
        wd = torch.randint(-127, 128, (h, i), device=DEV, generator=gen, dtype=torch.int32).to(torch.int8)
        sd = (torch.rand(h, device=DEV, generator=gen) * 1e-3 + 1e-4).float()
        packs = {"rows": (wgu, sgu, wd, sd),
                 "blocked": (ck.ck_weight_pack(wgu), sgu, ck.ck_weight_pack(wd), sd),
                 "decode": (ck.ck_weight_pack_decode(wgu, sgu), None, ck.ck_weight_pack_decode(wd, sd), None)}
        host_w = (wgu.cpu().numpy(), sgu.cpu().numpy(), wd.cpu().numpy(), sd.cpu().numpy())
        for m in (1, 2, 3, 8, 64, 65, 300, 1024, 2048, 4096):
            x = torch.randn(m, h, device=DEV, generator=gen).to(torch.bfloat16)
            small = m * i * h <= (1 << 27)
            want = orc.swiglu_mlp(u16(x), *host_w, g) if small else None
            for lay in ("rows", "blocked", "decode", "w8a16"):
                if lay == "decode" and m > 64:
                    continue
                what = f"m={m} h={h} i={i} {lay}"
                if lay == "w8a16":
                    b = packs["blocked"]
                    y = ck.ck_swiglu_mlp_w8a16(x, b[0], b[1], b[2], b[3], g)
                else:
                    y = ck.ck_swiglu_mlp(x, *packs[lay], g)
                torch.cuda.synchronize()
                calls += 1
                got = u16(y)
                if lay == "w8a16":
                    assert np.isfinite(orc.bf16_to_f32(got)).all(), what
                elif small:
                    np.testing.assert_array_equal(got, want, err_msg=what)
                    checked += 1
    say(f"h={h}: {calls} calls, {checked} compared with the oracle")


def w8a16_within_bound(orc, got, ref, wq, sw, k):
    """|got - oracle| within the derived bound of FP32 accumulation in any
    order (gamma_k * sum |x q| * s_w), the epilogue's FP32 rounding and one
    BF16 ulp, element by element."""
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    s_abs = orc.w8a16_abs_acc(ref["x_rot"], wq) * sw.astype(np.float64)[None, :]
    t = np.abs(orc.w8a16_acc(ref["x_rot"], wq) * sw.astype(np.float64)[None, :])
    want = orc.bf16_to_f32(ref["y"]).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(want), 1e-38).astype(np.float32)).astype(np.float64) * 65536.0
    bound = ulp + gamma * s_abs + 2 * 2.0 ** -23 * t
    return bool((np.abs(orc.bf16_to_f32(got).astype(np.float64) - want) <= bound).all())


@pytest.mark.parametrize("k", [128, 1024, 3072, 12288, 32768])
def test_w8a16_linear_routes(orc, k):
    """The W8A16 linear's routes (the rotation inside the few-row GEMM, the
    weight-streaming and the tiled GEMMs, both rotation kernels): every call
    succeeds with finite outputs, and the small ones are within the derived
    FP32-summation bound of the oracle."""
    g = 128
    gen = torch.Generator(device=DEV)
    gen.manual_seed(17 + k)
    calls = checked = 0
    for n in (16, 128, 1024, 4112, 24576):
        if n * k > (1 << 28):
            continue
        wq = torch.randint(-127, 128, (n, k), device=DEV, generator=gen, dtype=torch.int32).to(torch.int8)
        sw = (torch.rand(n, device=DEV, generator=gen) * 1e-3 + 1e-4).float()
        wb = ck.ck_weight_pack(wq)
        wq_h, sw_h = wq.cpu().numpy(), sw.cpu().numpy()
        for m, act in itertools.product((1, 2, 3, 16, 64, 65, 512, 2048, 4096), (0, 1)):
            ld = 2 * k if act else k
            if m * ld * 2 >= (1 << 30) or m * n * 2 >= (1 << 30):
                continue
            x = (torch.randn(m, ld, device=DEV, generator=gen) * 2).to(torch.bfloat16)
            y = ck.ck_int8_linear_w8a16(x, wb, sw, g, act)
            torch.cuda.synchronize()
            calls += 1
            got = u16(y)
            what = f"m={m} k={k} n={n} act={act}"
            assert np.isfinite(orc.bf16_to_f32(got)).all(), what
            if m * n * k <= (1 << 26):
                ref = orc.w8a16_linear(u16(x), act, wq_h, sw_h, g, return_all=True)
                assert w8a16_within_bound(orc, got, ref, wq_h, sw_h, k), what
                checked += 1
    say(f"w8a16 k={k}: {calls} calls, {checked} within the bound of the oracle")


@pytest.mark.parametrize("g", [64, 128, 256])
def test_weight_prep_and_rotate_f32_routes(orc, g):
    """Weight preparation (rows and blocked codes) and the FP32 rotation
    diagnostic over n, k grids: every call succeeds, the small ones bit-exact."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(19 + g)
    calls = checked = 0
    for k in sorted({g, 1024, 3072, 12288, 32768}):
        for n in (16, 48, 300, 4112, 24576):
            if n * k > (1 << 28):
                continue
            w = (torch.randn(n, k, device=DEV, generator=gen) * 0.02).float()
            small = n * k <= (1 << 22)
            for lay in ("rows", "blocked"):
                wq, sw = ck.ck_weight_prep(w, g, layout=lay)
                torch.cuda.synchronize()
                calls += 1
                if small:
                    q_o, s_o = orc.weight_prep(w.cpu().numpy(), g)
                    qh = wq.cpu().numpy()
                    qh = qh if lay == "rows" else from_blocked(qh, n)
                    np.testing.assert_array_equal(qh, q_o, err_msg=f"n={n} k={k} g={g} {lay}")
                    np.testing.assert_array_equal(sw.cpu().numpy().reshape(-1).view(np.uint32), s_o.view(np.uint32))
                    checked += 1
            x = (torch.randn(min(n, 2048), k, device=DEV, generator=gen) * 2).to(torch.bfloat16)
            u = ck.ck_act_rotate_f32(x, 0, g)
            torch.cuda.synchronize()
            calls += 1
            if x.shape[0] * k <= (1 << 22):
                np.testing.assert_array_equal(u.cpu().numpy().view(np.uint32),
                                              orc.act_rotate(u16(x), 0, g).view(np.uint32))
                checked += 1
    say(f"g={g}: {calls} calls, {checked} compared with the oracle")
