"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded inputs.

Bars (stated per check below):
  * INT8 codes, FP32 scales and int32 accumulators: bit-exact.
  * BF16 outputs: within 1 BF16 ulp or 1e-2 relative per element; the pinned
    epilogue makes them bit-exact, which is asserted too.
  * relative L2 against the float64 reference: GPU <= oracle + 1e-4.
Full-size workloads are compared on every element: the oracle runs each whole
workload once (cached for the row-major and blocked tests alike).
"""
import functools
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

# row-major weight codes and activation codes (the bindings default to the
# blocked layout; these tests also cover the row-major path)
prep_rows = functools.partial(ck.ck_weight_prep, layout="rows")
act_quant = functools.partial(ck.ck_act_quant, layout="rows")


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def bf16_dev(a_u16):
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).to(DEV).view(torch.bfloat16)


def bf16_host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.cpu().numpy()


def assert_bf16_close(got, want, what):
    """1 BF16 ulp or 1e-2 relative per element; then bit-exact."""
    g = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = (want.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ulp = np.spacing(np.abs(w).astype(np.float32)).astype(np.float64) * 65536.0
    ok = (np.abs(g - w) <= ulp) | (np.abs(g - w) <= 1e-2 * np.abs(w))
    assert ok.all(), f"{what}: {np.count_nonzero(~ok)} elements beyond tolerance"
    mism = np.count_nonzero(got != want)
    assert mism == 0, f"{what}: {mism} BF16 elements differ (within tolerance, not bit-exact)"


def to_blocked(a):
    """Row-major int8 [R, K] -> the blocked layout of include/ck.h: rows padded
    to a multiple of 256 with zeros, 1 KB blocks (r/32, k/32) in row-block-major
    order, inside a block ((k%32)/16, r%32, k%16)."""
    r, k = a.shape
    rp = -(-r // 256) * 256
    p = np.zeros((rp, k), dtype=np.int8)
    p[:r] = a
    return np.ascontiguousarray(
        p.reshape(rp // 32, 32, k // 32, 2, 16).transpose(0, 2, 3, 1, 4)).reshape(rp, k)


def from_blocked(b, rows):
    if b.ndim == 3:                     # the binding's [R / 32, k / 32, 1024] form
        b = b.reshape(b.shape[0] * 32, b.shape[1] * 32)
    rp, k = b.shape
    a = b.reshape(rp // 32, k // 32, 2, 32, 16).transpose(0, 3, 1, 2, 4).reshape(rp, k)
    return np.ascontiguousarray(a[:rows])


_cache = {}


def inputs(name):
    if name not in _cache:
        w = W.WORKLOADS[name]
        _cache[name] = W.mlp_inputs(w) if w.kind == "mlp" else W.linear_inputs(w)
    return _cache[name]


def prepped(orc, name, key="w"):
    ck_key = (name, key)
    if ck_key not in _cache:
        _cache[ck_key] = orc.weight_prep(inputs(name)[key], W.WORKLOADS[name].group)
    return _cache[ck_key]


def full_ref(orc, name):
    """The oracle on the whole workload, with every intermediate (cached)."""
    key = ("ref", name)
    if key not in _cache:
        wl = W.WORKLOADS[name]
        d = inputs(name)
        if wl.kind == "mlp":
            (gq, gs), (dq, ds) = prepped(orc, name, "w_gu"), prepped(orc, name, "w_down")
            _cache[key] = orc.swiglu_mlp(d["x"], gq, gs, dq, ds, wl.group, return_all=True)
        else:
            wq_o, sw_o = prepped(orc, name)
            _cache[key] = orc.int8_linear(d["x"], wl.act, wq_o, sw_o, wl.group, return_all=True)
    return _cache[key]


def ref_f64(orc, name):
    """The float64 reference (unrotated, unquantized weights) of the whole workload."""
    key = ("f64", name)
    if key not in _cache:
        wl = W.WORKLOADS[name]
        d = inputs(name)
        _cache[key] = (orc.reference_mlp_f64(d["x"], d["w_gu"], d["w_down"]) if wl.kind == "mlp"
                       else orc.reference_linear_f64(d["x"], wl.act, d["w"]))
    return _cache[key]


def check_codes(q_gpu, s_gpu, ref, m, what, blocked):
    """Activation codes and scales of every row against the oracle's, bit for bit."""
    q = from_blocked(host(q_gpu), m) if blocked else host(q_gpu)
    np.testing.assert_array_equal(host(s_gpu).reshape(-1).view(np.uint32), ref["sx"].view(np.uint32),
                                  err_msg=what + " scales")
    np.testing.assert_array_equal(q, ref["xq"], err_msg=what + " codes")


# ---------------------------------------------------------------------------
def test_silu_exhaustive_bf16(orc):
    say("silu: all 65536 BF16 patterns")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    fin = np.isfinite(f)
    got = host(ck.ck_silu_f32(bf16_dev(bits)))
    want = orc.silu_bf16(bits)
    np.testing.assert_array_equal(got[fin].view(np.uint32), want[fin].view(np.uint32))


@pytest.mark.parametrize("name,key", [("c1", "w"), ("c2", "w"), ("c3", "w"), ("c4", "w"),
                                      ("c5", "w_gu"), ("c5", "w_down")])
def test_weight_prep_bit_exact(orc, name, key):
    w = inputs(name)[key]
    say(f"weight_prep {name}.{key} {w.shape}")
    q, s = prep_rows(dev(w), W.WORKLOADS[name].group)
    torch.cuda.synchronize()
    q_o, s_o = prepped(orc, name, key)
    np.testing.assert_array_equal(host(q), q_o)
    np.testing.assert_array_equal(host(s)[:, 0].view(np.uint32), s_o.view(np.uint32))


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_act_quant_bit_exact(orc, name):
    wl = W.WORKLOADS[name]
    x = inputs(name)["x"]
    act = 0 if wl.kind == "mlp" else wl.act
    say(f"act_quant {name} act={act} x{x.shape}")
    q, s = act_quant(bf16_dev(x), act, wl.group)
    torch.cuda.synchronize()
    q_o, s_o = orc.act_quant(x, act, wl.group)
    np.testing.assert_array_equal(host(s)[:, 0].view(np.uint32), s_o.view(np.uint32))
    np.testing.assert_array_equal(host(q), q_o)


def plant_zero_rows(x, k, act):
    """Rows whose rotation is all zeros, which IEEE sums would leave as -0 in
    places (the rotation writes +0): row 0 all -0 (act 0) or up = +0 under
    gates of both signs (act 1, silu(gate) * 0 = +-0), the last row all +0."""
    x = x.copy()
    if act == 1:
        x[0, k:2 * k] = 0
    else:
        x[0, :k] = 0x8000
    x[-1, :] = 0
    return x


@pytest.mark.parametrize("m,k,act,g", [(37, 384, 1, 128), (64, 1024, 0, 256), (9, 512, 1, 64),
                                       (5, 256, 0, 1), (3, 32768, 1, 128)])
def test_act_rotate_bit_exact(orc, m, k, act, g):
    say(f"act_rotate m={m} k={k} act={act} g={g}")
    d = W.case(m, k, 16, act, seed=m + k)
    d["x"] = plant_zero_rows(d["x"], k, act)
    u = host(ck.ck_act_rotate_f32(bf16_dev(d["x"]), act, g))
    np.testing.assert_array_equal(u.view(np.uint32), orc.act_rotate(d["x"], act, g).view(np.uint32))


GEMM_SHAPES = [  # (m, n, k): every tile shape and k-step size, ragged m and n; the few-tile
    # shapes: 64 x 64 tiles with four k-slices per half stage (300, 272, 1024), (48, 4112, 256)
    # or two (600, 1200, 384), (100, 8192, 128); 64 x 128 with two (1000, 1040, 640),
    # (2048, 1024, 3072); 128 x 128 with two (513, 4112, 128)
    (1, 16, 64), (64, 128, 256), (77, 144, 192), (300, 272, 1024), (1000, 1040, 640),
    (600, 1200, 384), (2048, 1024, 3072), (513, 4112, 128),
    # few rows on tiles (n > 16 * CUs): 64 x 128 and 128 x 128 tiles at m <= 128
    (48, 4112, 256), (100, 8192, 128),
    # 64 x 128 and 128 x 128 tiles with one k-slice per half stage: k % 128 == 64
    # with at most one tile per CU, and more tiles than CUs (several per CU)
    (300, 272, 192), (600, 1200, 448), (320, 11008, 256), (1500, 4000, 320),
    # two k-slices per half stage on 128 x 128 tiles (at most one per CU)
    (1024, 4096, 1024), (700, 5008, 256),
    # persistent large-tile kernels: 256x256 and 256x192 tiles, ragged m and n,
    # k % 128 == 64, two rounds of tiles, a partial last round
    (4000, 4080, 192), (4000, 3056, 320), (4096, 8192, 128), (3968, 5120, 64), (2560, 6144, 256),
]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_i32_bit_exact(orc, m, n, k):
    say(f"gemm_i32 m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 7 + n)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    acc = host(ck.ck_int8_gemm_i32(dev(xq), dev(wq)))
    np.testing.assert_array_equal(acc, orc.gemm_i32(xq, wq))


@pytest.mark.parametrize("m,n", [(4, 32), (300, 4112)])
def test_gemm_i32_extreme_codes(orc, m, n):
    """The largest accumulators CK_MAX_K allows (127 * 127 * 32768 = 5.3e8),
    through the row-major kernel and both blocked kernels."""
    say(f"gemm_i32 extreme codes m={m} n={n} k=32768")
    k = 32768
    xq = np.full((m, k), -127, np.int8)
    xq[1::3] = 127
    wq = np.full((n, k), 127, np.int8)
    wq[::2] = -127
    want = orc.gemm_i32(xq, wq)
    assert np.abs(want).max() == 127 * 127 * k
    np.testing.assert_array_equal(host(ck.ck_int8_gemm_i32(dev(xq), dev(wq))), want)
    acc = host(ck.ck_int8_gemm_i32(dev(to_blocked(xq)), dev(to_blocked(wq)), "blocked", m=m, n=n))
    np.testing.assert_array_equal(acc, want)


LINEAR_CASES = [  # (m, k, n, act, g)
    (1, 256, 16, 0, 128), (7, 384, 48, 1, 128), (64, 256, 128, 0, 128), (300, 1024, 272, 1, 128),
    (129, 512, 320, 0, 64), (200, 768, 96, 1, 256), (33, 128, 64, 0, 1), (1000, 640, 1040, 0, 128),
    (4000, 256, 4080, 1, 128), (3968, 384, 5120, 0, 64), (5, 64, 32, 1, 64), (70, 64, 4112, 0, 32),
]


@pytest.mark.parametrize("m,k,n,act,g", LINEAR_CASES)
def test_int8_linear_bit_exact(orc, m, k, n, act, g):
    say(f"int8_linear m={m} k={k} n={n} act={act} g={g}")
    d = W.case(m, k, n, act, seed=1000 + m, zero_rows=(m // 2,) if m > 2 else ())
    wq_o, sw_o = orc.weight_prep(d["w"], g)
    wq, sw = prep_rows(dev(d["w"]), g)
    y = bf16_host(ck.ck_int8_linear(bf16_dev(d["x"]), wq, sw, g, act))
    ref = orc.int8_linear(d["x"], act, wq_o, sw_o, g, return_all=True)
    np.testing.assert_array_equal(host(wq), wq_o)
    assert_bf16_close(y, ref["y"], "y")
    if m > 2:
        assert not y[m // 2].any()           # an all-zero input row gives a zero output row


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_full_workload_all_elements(orc, name):
    """Row-major path at full size: codes, scales, int32 accumulators and BF16
    outputs of every row."""
    wl = W.WORKLOADS[name]
    d = inputs(name)
    say(f"int8_linear full {name}: {wl.desc}")
    wq, sw = prep_rows(dev(d["w"]), wl.group)
    x_dev = bf16_dev(d["x"])
    y = ck.ck_int8_linear(x_dev, wq, sw, wl.group, wl.act)
    xq_dev, sx_dev = act_quant(x_dev, wl.act, wl.group)
    acc = ck.ck_int8_gemm_i32(xq_dev, wq)
    torch.cuda.synchronize()
    ref = full_ref(orc, name)
    check_codes(xq_dev, sx_dev, ref, wl.m, name, False)
    np.testing.assert_array_equal(host(acc), ref["acc"])
    y_h = bf16_host(y)
    assert_bf16_close(y_h, ref["y"], f"{name} all rows")
    y64 = ref_f64(orc, name)
    e_gpu, e_orc = orc.rel_l2(y_h, y64), orc.rel_l2(ref["y"], y64)
    say(f"{name}: relL2 gpu={e_gpu:.5f} oracle={e_orc:.5f}")
    assert e_gpu <= e_orc + 1e-4


def test_swiglu_mlp_full_c5_all_elements(orc):
    wl = W.WORKLOADS["c5"]
    d = inputs("c5")
    say(f"swiglu_mlp full c5: {wl.desc}")
    wgu, sgu = prep_rows(dev(d["w_gu"]), wl.group)
    wd, sd = prep_rows(dev(d["w_down"]), wl.group)
    y = ck.ck_swiglu_mlp(bf16_dev(d["x"]), wgu, sgu, wd, sd, wl.group)
    torch.cuda.synchronize()
    ref = full_ref(orc, "c5")
    y_h = bf16_host(y)
    assert_bf16_close(y_h, ref["y"], "c5 all rows")
    y64 = ref_f64(orc, "c5")
    e_gpu, e_orc = orc.rel_l2(y_h, y64), orc.rel_l2(ref["y"], y64)
    say(f"c5: relL2 gpu={e_gpu:.5f} oracle={e_orc:.5f}")
    assert e_gpu <= e_orc + 1e-4


def test_swiglu_mlp_equals_its_stages():
    """ck_swiglu_mlp is the composition of its stage entry points, bit for bit,
    and repeated calls give identical bits."""
    say("swiglu_mlp composition + determinism (m=512, h=1024, i=2048)")
    m, h, i, g = 512, 1024, 2048, 128
    rng = np.random.default_rng(21)
    x = bf16_dev(W.to_bf16_bits(rng.standard_normal((m, h)).astype(np.float32)))
    wgu, sgu = prep_rows(dev((0.02 * rng.standard_normal((2 * i, h))).astype(np.float32)), g)
    wd, sd = prep_rows(dev((0.01 * rng.standard_normal((h, i))).astype(np.float32)), g)
    y1 = ck.ck_swiglu_mlp(x, wgu, sgu, wd, sd, g)
    y2 = ck.ck_swiglu_mlp(x, wgu, sgu, wd, sd, g)
    xq, sx = act_quant(x, 0, g)
    t = ck.ck_int8_gemm_bf16(xq, sx, wgu, sgu)
    hq, sh = act_quant(t, 1, g)
    y3 = ck.ck_int8_gemm_bf16(hq, sh, wd, sd)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))


def test_packed_gate_up_equals_separate():
    """sglang PR #44196, "Accuracy Tests": packed [gate | up] GEMM columns equal
    the two separate projections bit for bit."""
    say("packed gate|up vs separate")
    rng = np.random.default_rng(22)
    m, h, i, g = 300, 512, 384, 128
    x = bf16_dev(W.to_bf16_bits(rng.standard_normal((m, h)).astype(np.float32)))
    wg = (0.02 * rng.standard_normal((i, h))).astype(np.float32)
    wu = (0.02 * rng.standard_normal((i, h))).astype(np.float32)
    q, s = prep_rows(dev(np.concatenate([wg, wu])), g)
    qg, sg = prep_rows(dev(wg), g)
    qu, su = prep_rows(dev(wu), g)
    y = ck.ck_int8_linear(x, q, s, g)
    yg = ck.ck_int8_linear(x, qg, sg, g)
    yu = ck.ck_int8_linear(x, qu, su, g)
    torch.cuda.synchronize()
    assert torch.equal(y[:, :i].contiguous().view(torch.int16), yg.view(torch.int16))
    assert torch.equal(y[:, i:].contiguous().view(torch.int16), yu.view(torch.int16))


def test_empty_and_degenerate_calls(orc):
    say("empty and degenerate calls")
    g = 128
    x0 = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    wq, sw = prep_rows(torch.zeros((32, 256), dtype=torch.float32, device=DEV), g)
    torch.cuda.synchronize()
    assert not wq.any() and not sw.any()                  # all-zero weight rows
    assert ck.ck_int8_linear(x0, wq, sw, g).shape == (0, 32)
    xz = torch.zeros((4, 256), dtype=torch.bfloat16, device=DEV)
    y = ck.ck_int8_linear(xz, wq, sw, g)
    torch.cuda.synchronize()
    assert not y.any()


# ---------------------------------------------------------------------------
# Blocked operand layout (the product path)
# ---------------------------------------------------------------------------
def test_blocked_helpers_round_trip():
    rng = np.random.default_rng(30)
    a = rng.integers(-127, 128, size=(300, 128), dtype=np.int8)
    b = to_blocked(a)
    assert b.shape == (512, 128)
    np.testing.assert_array_equal(from_blocked(b, 300), a)
    # spot-check the documented offset formula
    flat = b.reshape(-1)
    for r, k in [(0, 0), (31, 17), (33, 95), (299, 127), (64, 32)]:
        off = ((r // 32) * (128 // 32) + k // 32) * 1024 + ((k % 32) // 16) * 512 + (r % 32) * 16 + k % 16
        assert flat[off] == a[r, k]


@pytest.mark.parametrize("n,k", [(128, 256), (300, 384), (1040, 640), (24576, 3072)])
def test_weight_pack_layout(orc, n, k):
    say(f"weight_pack n={n} k={k}")
    rng = np.random.default_rng(n + k)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    got = host(ck.ck_weight_pack(dev(wq)))
    assert got.shape == (-(-n // 256) * 8, k // 32, 1024)
    np.testing.assert_array_equal(got.reshape(-1, k), to_blocked(wq))      # padding rows are zero too


@pytest.mark.parametrize("name", ["c1", "c2", "c4"])
def test_act_quant_blocked(orc, name):
    wl = W.WORKLOADS[name]
    x = inputs(name)["x"]
    say(f"act_quant blocked {name}")
    q, s = act_quant(bf16_dev(x), wl.act, wl.group, layout="blocked")
    q_o, s_o = orc.act_quant(x, wl.act, wl.group)
    np.testing.assert_array_equal(from_blocked(host(q), wl.m), q_o)
    np.testing.assert_array_equal(host(s)[:, 0].view(np.uint32), s_o.view(np.uint32))


@pytest.mark.parametrize("m,k,g,layout", [
    (2731, 6144, 64, "blocked"), (2049, 8192, 256, "rows"), (1500, 12288, 128, "blocked"),
    (5600, 3072, 128, "rows"), (4097, 4096, 128, "blocked"),
    # staged blocked codes with 8, 4, 2 and 1 rows per pass (teams of 128 to
    # 1024 lanes), the largest staged k, the unstaged blocked slot order past it
    (5601, 3072, 64, "blocked"), (2051, 8192, 256, "blocked"), (1201, 14336, 128, "blocked"),
    (1025, 16384, 64, "blocked"),
    # k < 1024: the per-row kernel with staged blocked codes
    (32769, 512, 64, "blocked"),
    # m * k in [2^23, 2^24) with at least 8 rows per CU: the table kernel too
    (4097, 2048, 64, "blocked"), (2048, 4096, 128, "rows"), (3001, 4096, 256, "blocked"),
    # k in (6144, 8192]: two rows of two chunks per lane instead of one-row
    # passes, with idle chunk slots (k = 7168)
    (2048, 7168, 64, "rows"), (2313, 7168, 128, "blocked"),
    # table sizes with rows past the table kernel's team (k > 24576, up to
    # CK_MAX_K): the per-row kernel
    (512, 32768, 128, "blocked"), (700, 26624, 256, "rows")])
def test_swiglu_quant_large_calls_bit_exact(orc, m, k, g, layout):
    """Large SwiGLU quantizer calls: codes and scales bit-exact against the
    oracle.  From k = 1024 the persistent kernel whose silu is a table lookup
    takes them (m * k >= 2^24, or 2^23 with 8 rows per CU; teams of 128 to
    1024 lanes, 1 to 3 chunks per lane); blocked
    codes up to k = 14336 are staged in LDS per aligned 8-row group, ragged
    row counts end in partial groups."""
    say(f"swiglu quant large m={m} k={k} g={g} {layout}")
    rng = np.random.default_rng(m + k)
    x = W.to_bf16_bits((rng.standard_normal((m, 2 * k)) * 2.0).astype(np.float32))
    # every BF16 gate pattern of magnitude below 1000 appears in the first rows
    # (the table's whole range, denormals, both clamps; larger gates would only
    # overflow the products), and one all-zero row
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (pats.astype(np.uint32) << 16).view(np.float32)
    pats = pats[np.isfinite(f) & (np.abs(f) < 1000.0)]
    flat = x[:, :k].reshape(-1)
    flat[:pats.size] = pats
    x[:, :k] = flat.reshape(m, k)
    x[m // 2] = 0
    q, sc = act_quant(bf16_dev(x), 1, g, layout=layout)
    torch.cuda.synchronize()
    q_o, s_o = orc.act_quant(x, 1, g)
    np.testing.assert_array_equal(host(sc)[:, 0].view(np.uint32), s_o.view(np.uint32))
    np.testing.assert_array_equal(from_blocked(host(q), m) if layout == "blocked" else host(q), q_o)


@pytest.mark.parametrize("m,k,g,layout", [
    (3001, 2048, 128, "rows"), (2050, 4096, 256, "rows"), (2051, 12288, 64, "rows"),
    # blocked codes from the per-row kernel: shapes that would leave group
    # slots of the line kernel idle (k = 5120 at g = 128, k = 1536 at g = 256),
    # fewer than 8 rows per CU
    (2560, 5120, 128, "blocked"), (2304, 1536, 256, "blocked"), (1500, 4096, 128, "blocked"),
    # the line kernel (8 rows per workgroup, 4 to 16 waves, 1 to 8 loads per
    # lane; ragged last 8-row group)
    (2049, 1024, 64, "blocked"), (4096, 3072, 128, "blocked"), (2050, 8192, 128, "blocked"),
    (3000, 6144, 256, "blocked"), (2500, 2048, 64, "blocked"), (4095, 2560, 64, "blocked"),
    (2100, 1280, 64, "blocked"),
    # m * k >= 2^24, k <= 4096: blocked codes staged in LDS, 1 to 4 chunks per
    # lane (k = 4032: idle chunk slots), ragged last 8-row group; at
    # m * k = 2^24 the line writes are non-temporal
    (16385, 1024, 64, "blocked"), (8193, 2048, 128, "blocked"), (5462, 3072, 256, "blocked"),
    (4097, 4096, 128, "blocked"), (4200, 4032, 64, "blocked"), (8192, 2048, 64, "blocked"),
    (16384, 1024, 256, "blocked")])
def test_x_quant_large_calls_bit_exact(orc, m, k, g, layout):
    """Large x quantizer calls: codes and scales bit-exact against the oracle,
    ragged row counts, row-major and blocked codes (the line kernel, or staged
    in LDS per 8-row group from m * k = 2^24), outlier channels, an all-zero
    row and a row with a single nonzero value."""
    say(f"x quant large m={m} k={k} g={g} {layout}")
    rng = np.random.default_rng(3 * m + k)
    xf = rng.standard_normal((m, k)).astype(np.float32)
    xf[:, rng.choice(k, size=max(1, k // 100), replace=False)] *= 20.0
    x = W.to_bf16_bits(xf)
    x[m // 3] = 0
    x[m // 2] = 0
    x[m // 2, k - 1] = W.to_bf16_bits(np.array([-3.0], dtype=np.float32))[0]
    q, sc = act_quant(bf16_dev(x), 0, g, layout=layout)
    torch.cuda.synchronize()
    q_o, s_o = orc.act_quant(x, 0, g)
    np.testing.assert_array_equal(host(sc)[:, 0].view(np.uint32), s_o.view(np.uint32))
    np.testing.assert_array_equal(from_blocked(host(q), m) if layout == "blocked" else host(q), q_o)


def _random_x_quant_shapes(count=48, seed=2026):
    """Seeded random x-quantizer calls with blocked codes around the kernels'
    domain borders: 1900..9000 rows (under and over 8 rows per CU, under and
    over m * k = 2^24), k either a common model width or a random multiple of
    the group in 768..8448 (both sides of the line kernel's 1024 and 8192 and
    of the staged kernel's 4096; group counts that do and do not divide among
    16, 12, 8 or 4 waves), g in {64, 128, 256}."""
    rng = np.random.default_rng(seed)
    widths = [1024, 1536, 2048, 2560, 3072, 4096, 5120, 6144, 7168, 8192]
    shapes = []
    for _ in range(count):
        g = int(rng.choice([64, 128, 256]))
        if rng.random() < 0.6:
            k = int(rng.choice(widths))
        else:
            k = int(rng.integers(768 // g, 8448 // g + 1)) * g
        m = int(rng.integers(1900, 9001))
        shapes.append((m, k, g))
    return shapes


@pytest.mark.parametrize("m,k,g", _random_x_quant_shapes())
def test_x_quant_random_blocked_bit_exact(orc, m, k, g):
    """x quantizer, blocked codes, seeded random shapes (line kernel, staged
    kernel with and without non-temporal line writes, per-row kernel): codes
    and scales bit-exact against the oracle."""
    say(f"x quant random m={m} k={k} g={g}")
    rng = np.random.default_rng(m * 7 + k)
    xf = rng.standard_normal((m, k)).astype(np.float32)
    xf[:, rng.choice(k, size=max(1, k // 100), replace=False)] *= 20.0
    x = W.to_bf16_bits(xf)
    x[m // 5] = 0
    q, sc = ck.ck_act_quant(bf16_dev(x), 0, g, layout="blocked")
    torch.cuda.synchronize()
    q_o, s_o = orc.act_quant(x, 0, g)
    np.testing.assert_array_equal(host(sc)[:, 0].view(np.uint32), s_o.view(np.uint32))
    np.testing.assert_array_equal(from_blocked(host(q), m), q_o)


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
def test_gemm_i32_blocked_bit_exact(orc, m, n, k):
    say(f"gemm_i32 blocked m={m} n={n} k={k}")
    rng = np.random.default_rng(m * 11 + n)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    acc = host(ck.ck_int8_gemm_i32(dev(to_blocked(xq)), dev(to_blocked(wq)), "blocked", m=m, n=n))
    np.testing.assert_array_equal(acc, orc.gemm_i32(xq, wq))


SMALL_M_SHAPES = [  # (m, n, k): the few-row kernel: 1, 2, 4 and 8 row fragments (m up to 128
    # when n <= 16 * CUs), k-chunk counts below, at and above one batch of the 8 waves,
    # ragged m
    (1, 4096, 4096), (2, 48, 1024), (16, 1024, 3072), (17, 2048, 128), (32, 160, 12288),
    (33, 4096, 4096), (48, 3072, 1536), (64, 4096, 12288), (64, 16, 64),
    (65, 4096, 4096), (96, 1040, 3072), (128, 4096, 12288), (100, 16, 64),
    # two or four 16-row weight groups per workgroup (m >= 16, n % 32 == 0, n / 32 >= CUs;
    # four: n % 64 == 0, n / 64 >= CUs, 17..32 rows), and n % 32 != 0 (one group)
    (16, 16384, 256), (32, 16416, 320), (31, 24576, 192), (20, 16400, 128), (16, 8192, 192),
    (25, 12288, 128), (17, 16384, 128),
]


@pytest.mark.parametrize("m,n,k", SMALL_M_SHAPES)
def test_small_m_gemm_bit_exact(orc, m, n, k):
    say(f"small-m gemm i32 + bf16 blocked m={m} n={n} k={k}")
    rng = np.random.default_rng(7 * m + n + k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    sx = (rng.random(m, dtype=np.float32) * 1e-3).astype(np.float32)
    sw = (rng.random(n, dtype=np.float32) * 1e-3).astype(np.float32)
    xb, wb = dev(to_blocked(xq)), dev(to_blocked(wq))
    acc_o = orc.gemm_i32(xq, wq)
    acc = host(ck.ck_int8_gemm_i32(xb, wb, "blocked", m=m, n=n))
    np.testing.assert_array_equal(acc, acc_o)
    y = bf16_host(ck.ck_int8_gemm_bf16(xb, dev(sx.reshape(m, 1)), wb, dev(sw.reshape(n, 1)),
                                       layout="blocked"))
    np.testing.assert_array_equal(y, orc.dequant(acc_o, sx, sw))


EXTRA_CASES = [  # (m, k, n, layout): few-row, 64x64 (four and two k-slices per half stage),
    # 64x128 and 128x128 (one and two), 256x256 and 256x192 blocked tiles, ragged m and n,
    # and both row-major kernels
    (5, 256, 48, "blocked"), (64, 512, 1040, "blocked"), (100, 512, 1040, "blocked"),
    (300, 1024, 272, "blocked"), (700, 256, 5008, "blocked"), (320, 256, 11008, "blocked"),
    (1500, 384, 4000, "blocked"), (600, 384, 1200, "blocked"), (2048, 3072, 1024, "blocked"),
    (2000, 256, 8192, "blocked"), (2000, 256, 6144, "blocked"),
    (300, 1024, 272, "rows"), (2000, 256, 8192, "rows"),
]


@pytest.mark.parametrize("m,k,n,layout", EXTRA_CASES)
def test_int8_linear_bias_residual_bit_exact(orc, m, k, n, layout):
    say(f"int8_linear bias/residual m={m} k={k} n={n} layout={layout}")
    g = 128
    d = W.case(m, k, n, 0, seed=2000 + m)
    rng = np.random.default_rng(m + n)
    bias = rng.standard_normal(n).astype(np.float32)
    res = orc.f32_to_bf16(rng.standard_normal((m, n)).astype(np.float32))
    wq_o, sw_o = orc.weight_prep(d["w"], g)
    wq, sw = prep_rows(dev(d["w"]), g)
    if layout == "blocked":
        wq = ck.ck_weight_pack(wq)
    x = bf16_dev(d["x"])
    for b, r in ((bias, None), (None, res), (bias, res)):
        y = ck.ck_int8_linear(x, wq, sw, g, layout=layout,
                              bias=None if b is None else dev(b),
                              residual=None if r is None else bf16_dev(r))
        want = orc.int8_linear(d["x"], 0, wq_o, sw_o, g, bias=b, residual=r)
        np.testing.assert_array_equal(bf16_host(y), want)
    # the residual may be the output buffer itself
    y = bf16_dev(res)
    ck.ck_int8_linear(x, wq, sw, g, layout=layout, out=y, bias=dev(bias), residual=y)
    np.testing.assert_array_equal(bf16_host(y),
                                  orc.int8_linear(d["x"], 0, wq_o, sw_o, g, bias=bias, residual=res))


@pytest.mark.parametrize("m,k,n,act,g", LINEAR_CASES)
def test_int8_linear_blocked_bit_exact(orc, m, k, n, act, g):
    say(f"int8_linear blocked m={m} k={k} n={n} act={act} g={g}")
    d = W.case(m, k, n, act, seed=1000 + m, zero_rows=(m // 2,) if m > 2 else ())
    wq_o, sw_o = orc.weight_prep(d["w"], g)
    wq, sw = prep_rows(dev(d["w"]), g)
    y = bf16_host(ck.ck_int8_linear(bf16_dev(d["x"]), ck.ck_weight_pack(wq), sw, g, act,
                                    layout="blocked"))
    assert_bf16_close(y, orc.int8_linear(d["x"], act, wq_o, sw_o, g), "y")


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4"])
def test_full_workload_blocked_all_elements(orc, name):
    """The blocked path at full size: blocked codes and scales, int32
    accumulators and the linear's BF16 output, every element."""
    wl = W.WORKLOADS[name]
    d = inputs(name)
    say(f"int8_linear blocked full {name}: {wl.desc}")
    wq, sw = ck.ck_weight_prep(dev(d["w"]), wl.group)          # blocked by default
    x_dev = bf16_dev(d["x"])
    y = ck.ck_int8_linear(x_dev, wq, sw, wl.group, wl.act)
    xq, sx = ck.ck_act_quant(x_dev, wl.act, wl.group)          # blocked by default
    acc = ck.ck_int8_gemm_i32(xq, wq, m=wl.m, n=wl.n)
    torch.cuda.synchronize()
    ref = full_ref(orc, name)
    check_codes(xq, sx, ref, wl.m, name + " blocked", True)
    np.testing.assert_array_equal(host(acc), ref["acc"])
    assert_bf16_close(bf16_host(y), ref["y"], f"{name} blocked all rows")


def test_swiglu_mlp_blocked_full_c5_all_elements(orc):
    """The benchmarked path at full size: ck_swiglu_mlp's output and, through
    the stage calls bench.py times, both stages' codes, scales, int32
    accumulators and the stage-1 BF16 output, every element."""
    wl = W.WORKLOADS["c5"]
    d = inputs("c5")
    g, m = wl.group, wl.m
    say(f"swiglu_mlp blocked full c5: {wl.desc}")
    wgu, sgu = ck.ck_weight_prep(dev(d["w_gu"]), g)
    wd, sd = ck.ck_weight_prep(dev(d["w_down"]), g)
    x = bf16_dev(d["x"])
    y = ck.ck_swiglu_mlp(x, wgu, sgu, wd, sd, g)
    torch.cuda.synchronize()
    ref = full_ref(orc, "c5")
    s1, s2 = ref["stage1"], ref["stage2"]
    y_h = bf16_host(y)
    assert_bf16_close(y_h, ref["y"], "c5 blocked all rows")
    # stage 1: x codes, scales, accumulators, the [m, 2i] BF16 output
    xq, sx = ck.ck_act_quant(x, 0, g)
    acc1 = ck.ck_int8_gemm_i32(xq, wgu, m=m, n=2 * wl.n)
    torch.cuda.synchronize()
    check_codes(xq, sx, s1, m, "c5 stage 1", True)
    np.testing.assert_array_equal(host(acc1), s1["acc"])
    del acc1
    t1 = ck.ck_int8_gemm_bf16(xq, sx, wgu, sgu)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bf16_host(t1), s1["y"])
    # stage 2: the SwiGLU'd codes, scales and accumulators
    hq, sh = ck.ck_act_quant(t1, 1, g)
    acc2 = ck.ck_int8_gemm_i32(hq, wd, m=m, n=wl.k)
    torch.cuda.synchronize()
    check_codes(hq, sh, s2, m, "c5 stage 2", True)
    np.testing.assert_array_equal(host(acc2), s2["acc"])
    y64 = ref_f64(orc, "c5")
    e_gpu, e_orc = orc.rel_l2(y_h, y64), orc.rel_l2(ref["y"], y64)
    say(f"c5 blocked: relL2 gpu={e_gpu:.5f} oracle={e_orc:.5f}")
    assert e_gpu <= e_orc + 1e-4


def test_blocked_stages_equal_swiglu_mlp():
    """The stage calls bench.py times (blocked layout) compose to ck_swiglu_mlp
    bit for bit, and agree with the row-major path."""
    say("blocked stage composition (m=1000, h=1024, i=2048)")
    m, h, i, g = 1000, 1024, 2048, 128
    rng = np.random.default_rng(31)
    x = bf16_dev(W.to_bf16_bits(rng.standard_normal((m, h)).astype(np.float32)))
    wgu, sgu = prep_rows(dev((0.02 * rng.standard_normal((2 * i, h))).astype(np.float32)), g)
    wd, sd = prep_rows(dev((0.01 * rng.standard_normal((h, i))).astype(np.float32)), g)
    pgu, pd = ck.ck_weight_pack(wgu), ck.ck_weight_pack(wd)
    y_rows = ck.ck_swiglu_mlp(x, wgu, sgu, wd, sd, g)
    y_blk = ck.ck_swiglu_mlp(x, pgu, sgu, pd, sd, g, layout="blocked")
    xq, sx = act_quant(x, 0, g, layout="blocked")
    t1 = ck.ck_int8_gemm_bf16(xq, sx, pgu, sgu, layout="blocked")
    hq, sh = act_quant(t1, 1, g, layout="blocked")
    y_st = ck.ck_int8_gemm_bf16(hq, sh, pd, sd, layout="blocked")
    torch.cuda.synchronize()
    assert torch.equal(y_blk.view(torch.int16), y_rows.view(torch.int16))
    assert torch.equal(y_blk.view(torch.int16), y_st.view(torch.int16))


@pytest.mark.parametrize("g,layout,scalar", [(256, "blocked", False), (128, "rows", False),
                                             (256, "blocked", True), (128, "decode", False)])
def test_serialized_layer_bit_exact(orc, g, layout, scalar):
    """Pre-quantized I8 weights + F32 [out, 1] scales, as a serialized
    checkpoint holds them (sglang PR #35994 report), used without re-quantizing."""
    from swiglu_mlp_amd import checkpoint as C
    say(f"serialized layer g={g} layout={layout} scalar_scale={scalar}")
    m, k, n = (64 if layout == "decode" else 200), 1024, 528
    d = W.case(m, k, n, 0, seed=77)
    wq_o, sw_o = orc.weight_prep(d["w"], g)          # what a serialized file holds
    if scalar:
        sw_o = np.full_like(sw_o, sw_o.max())
        scale = torch.tensor(float(sw_o[0]), dtype=torch.float32)
    else:
        scale = dev(sw_o.reshape(n, 1))
    wq, sw = C.serialized_linear_weights(dev(wq_o), scale, group=g, layout=layout)
    y = bf16_host(ck.ck_int8_linear(bf16_dev(d["x"]), wq, sw, g, layout=layout))
    np.testing.assert_array_equal(y, orc.int8_linear(d["x"], 0, wq_o, sw_o, g))


def to_decode(wq, sw):
    """Row-major int8 [n, k] and FP32 scales [n] -> the decode layout of
    include/ck.h: per 16-row group b, the 16 scales (64 bytes), then chunk c of
    1 KB holding W[16 b + r][64 c + 16 q + e] at 256 q + 16 r + e."""
    n, k = wq.shape
    g = n // 16
    body = wq.reshape(g, 16, k // 64, 4, 16).transpose(0, 2, 3, 1, 4).reshape(g, 16 * k)
    head = np.ascontiguousarray(sw.astype(np.float32).reshape(g, 16)).view(np.uint8)
    return np.ascontiguousarray(np.concatenate([head, body.view(np.uint8)], axis=1))


@pytest.mark.parametrize("n,k", [(16, 64), (48, 1024), (4096, 3072)])
def test_weight_pack_decode_layout(orc, n, k):
    say(f"weight_pack_decode n={n} k={k}")
    rng = np.random.default_rng(n + k)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    sw = rng.random(n, dtype=np.float32)
    got = host(ck.ck_weight_pack_decode(dev(wq), dev(sw)))
    np.testing.assert_array_equal(got, to_decode(wq, sw))


DECODE_SHAPES = [  # (m, n, k): 1, 2 and 4 row fragments, ragged m, short and long k
    (1, 4096, 4096), (2, 48, 1024), (16, 1024, 3072), (17, 2048, 128), (33, 4096, 4096),
    (64, 4096, 12288), (64, 16, 64),
    # two weight groups per workgroup (1, 2 and 4 row fragments), and n % 32 != 0
    (16, 16384, 256), (23, 16416, 64), (40, 16384, 192), (64, 24576, 128), (50, 16400, 256),
    (48, 8192, 128), (16, 11008, 256), (30, 16384, 192),
]


@pytest.mark.parametrize("m,n,k", DECODE_SHAPES)
def test_decode_gemm_bit_exact(orc, m, n, k):
    say(f"decode gemm i32 + bf16 m={m} n={n} k={k}")
    rng = np.random.default_rng(5 * m + n + k)
    xq = rng.integers(-127, 128, size=(m, k), dtype=np.int8)
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    sx = (rng.random(m, dtype=np.float32) * 1e-3).astype(np.float32)
    sw = (rng.random(n, dtype=np.float32) * 1e-3).astype(np.float32)
    xb, wd = dev(to_blocked(xq)), dev(to_decode(wq, sw))
    acc_o = orc.gemm_i32(xq, wq)
    np.testing.assert_array_equal(host(ck.ck_int8_gemm_i32(xb, wd, "decode", m=m)), acc_o)
    y = bf16_host(ck.ck_int8_gemm_bf16(xb, dev(sx.reshape(m, 1)), wd, None, layout="decode"))
    np.testing.assert_array_equal(y, orc.dequant(acc_o, sx, sw))


DECODE_LINEAR = [  # (m, k, n, act, g)
    (1, 1024, 4096, 0, 128), (7, 2048, 528, 1, 256), (33, 3072, 1040, 0, 128),
    (64, 12288, 3072, 1, 128), (64, 256, 16, 1, 64),
    # the quantizer fused into the decode GEMM at m <= 2: x (k <= 8192) and SwiGLU
    # (k <= 16384), groups 64, 128, 256; 1 to 4 chunks per lane, a row shorter than
    # the team; then the first shapes past each limit
    (1, 12288, 3072, 1, 128), (2, 3072, 1040, 0, 64), (1, 8192, 48, 0, 256),
    (1, 16384, 32, 1, 256), (1, 64, 16, 0, 64), (2, 4096, 528, 0, 128), (2, 512, 16, 1, 128),
    (2, 12288, 528, 1, 256), (3, 256, 32, 0, 128), (3, 512, 16, 1, 128), (1, 8256, 16, 0, 64),
    (1, 1024, 64, 1, 32),
]


@pytest.mark.parametrize("layout", ["decode", "blocked"])
@pytest.mark.parametrize("m,k,n,act,g", DECODE_LINEAR)
def test_int8_linear_decode_bit_exact(orc, m, k, n, act, g, layout):
    """Few rows on decode or blocked weights, through the fused quantizer at
    m <= 2 and the separate one past its limits."""
    say(f"int8_linear few rows m={m} k={k} n={n} act={act} g={g} layout={layout}")
    d = W.case(m, k, n, act, seed=3000 + m, zero_rows=(m // 2,) if m > 2 else ())
    wq_o, sw_o = orc.weight_prep(d["w"], g)
    wq, sw = prep_rows(dev(d["w"]), g)
    if layout == "decode":
        wd, sl = ck.ck_weight_pack_decode(wq, sw), None
    else:
        wd, sl = ck.ck_weight_pack(wq), sw
    x = bf16_dev(d["x"])
    y = bf16_host(ck.ck_int8_linear(x, wd, sl, g, act, layout=layout))
    np.testing.assert_array_equal(y, orc.int8_linear(d["x"], act, wq_o, sw_o, g))
    rng = np.random.default_rng(m + n)
    bias = rng.standard_normal(n).astype(np.float32)
    res = orc.f32_to_bf16(rng.standard_normal((m, n)).astype(np.float32))
    y = ck.ck_int8_linear(x, wd, sl, g, act, layout=layout, bias=dev(bias),
                          residual=bf16_dev(res))
    np.testing.assert_array_equal(
        bf16_host(y), orc.int8_linear(d["x"], act, wq_o, sw_o, g, bias=bias, residual=res))


@pytest.mark.parametrize("m", [1, 2, 16, 64])
def test_swiglu_mlp_decode_bit_exact(orc, m):
    say(f"swiglu_mlp decode m={m} h=1024 i=2816")
    h, i, g = 1024, 2816, 128
    rng = np.random.default_rng(40 + m)
    xb = W.to_bf16_bits(rng.standard_normal((m, h)).astype(np.float32))
    w_gu = (0.02 * rng.standard_normal((2 * i, h))).astype(np.float32)
    w_dn = (0.01 * rng.standard_normal((h, i))).astype(np.float32)
    gq, gs = prep_rows(dev(w_gu), g)
    dq, ds = prep_rows(dev(w_dn), g)
    y = ck.ck_swiglu_mlp(bf16_dev(xb), ck.ck_weight_pack_decode(gq, gs), None,
                         ck.ck_weight_pack_decode(dq, ds), None, g, layout="decode")
    y_blk = ck.ck_swiglu_mlp(bf16_dev(xb), ck.ck_weight_pack(gq), gs, ck.ck_weight_pack(dq), ds,
                             g, layout="blocked")
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_blk.view(torch.int16))
    (gq_o, gs_o), (dq_o, ds_o) = orc.weight_prep(w_gu, g), orc.weight_prep(w_dn, g)
    np.testing.assert_array_equal(bf16_host(y), orc.swiglu_mlp(xb, gq_o, gs_o, dq_o, ds_o, g))


SPLITK_CASES = [  # (m, k, n, act, g, bias and residual): m >= 48, k >= 8192, few output tiles
    (64, 12288, 4096, 0, 128, False),    # 64 x 64 tiles in four k ranges (the weight-stream regime)
    (48, 12288, 3072, 1, 128, True),     # SwiGLU input, bias and residual
    (128, 12288, 4096, 0, 256, False),
    (100, 8192, 2048, 0, 64, True),      # ragged m
    (53, 8192, 1056, 1, 128, False),     # ragged m and n (16.5 tiles of 64 columns)
    (256, 12288, 3072, 0, 128, False),   # 128 x 128 tiles
    (1024, 12288, 1024, 0, 128, True),
]


@pytest.mark.parametrize("m,k,n,act,g,extra", SPLITK_CASES)
def test_int8_linear_splitk_bit_exact(orc, m, k, n, act, g, extra):
    """Few-tile blocked linears split k over more CUs and add the int32 partial
    sums in a second kernel that applies the epilogue: bit-exact against the
    oracle, and equal to the same call with a workspace that only holds the
    codes (which runs unsplit)."""
    say(f"int8_linear split-k m={m} k={k} n={n} act={act} g={g} extra={extra}")
    L = ck.lib()
    codes = ck._linear_codes_bytes(m, k)
    full = L.ck_int8_linear_workspace_size(m, k, n)
    assert full > codes, "this shape is meant to take split K"
    d = W.case(m, k, n, act, seed=3000 + m, zero_rows=(m // 2,))
    rng = np.random.default_rng(m * 3 + n)
    b = rng.standard_normal(n).astype(np.float32) if extra else None
    r = orc.f32_to_bf16(rng.standard_normal((m, n)).astype(np.float32)) if extra else None
    wq_o, sw_o = orc.weight_prep(d["w"], g)
    wq, sw = ck.ck_weight_prep(dev(d["w"]), g)
    x = bf16_dev(d["x"])
    kw = dict(bias=None if b is None else dev(b), residual=None if r is None else bf16_dev(r))
    y_split = ck.ck_int8_linear(x, wq, sw, g, act, workspace=torch.empty(full, dtype=torch.uint8, device=DEV), **kw)
    y_plain = ck.ck_int8_linear(x, wq, sw, g, act, workspace=torch.empty(codes, dtype=torch.uint8, device=DEV), **kw)
    want = orc.int8_linear(d["x"], act, wq_o, sw_o, g, bias=b, residual=r)
    np.testing.assert_array_equal(bf16_host(y_split), want)
    np.testing.assert_array_equal(bf16_host(y_plain), want)


def test_swiglu_mlp_splitk_bit_exact(orc):
    """The MLP block at 64 rows with c5's dimensions: the down projection (k =
    12288, 3072 columns) takes split K; bit-exact against the oracle."""
    m, h, i, g = 64, 3072, 12288, 128
    say(f"swiglu_mlp split-k m={m} h={h} i={i}")
    L = ck.lib()
    assert L.ck_swiglu_mlp_workspace_size(m, h, i) > L.ck_swiglu_mlp_workspace_size(m, h, 4096)
    rng = np.random.default_rng(4242)
    xb = W.to_bf16_bits(rng.standard_normal((m, h)).astype(np.float32))
    w_gu = (0.02 * rng.standard_normal((2 * i, h))).astype(np.float32)
    w_dn = (0.01 * rng.standard_normal((h, i))).astype(np.float32)
    gq, gs = ck.ck_weight_prep(dev(w_gu), g)
    dq, ds = ck.ck_weight_prep(dev(w_dn), g)
    y = ck.ck_swiglu_mlp(bf16_dev(xb), gq, gs, dq, ds, g)
    (gq_o, gs_o), (dq_o, ds_o) = orc.weight_prep(w_gu, g), orc.weight_prep(w_dn, g)
    np.testing.assert_array_equal(bf16_host(y), orc.swiglu_mlp(xb, gq_o, gs_o, dq_o, ds_o, g))


@pytest.mark.parametrize("layout", ["decode", "blocked"])
@pytest.mark.parametrize("m,k,act,g", [(1, 3072, 0, 128), (2, 3072, 0, 128), (2, 8192, 0, 64),
                                        (1, 12288, 1, 128), (1, 4096, 1, 256), (2, 12288, 1, 128)])
def test_fused_decode_equals_the_stages(m, k, act, g, layout):
    """ck_int8_linear at the fewest rows (one kernel that quantizes the rows
    itself, decode or blocked weights) equals ck_act_quant followed by the
    few-row GEMM, codes, scales and outputs alike, bit for bit, with bias and
    residual."""
    say(f"fused quantizer vs stages m={m} k={k} act={act} g={g} layout={layout}")
    n = 1040
    rng = np.random.default_rng(77 + m + k)
    d = W.case(m, k, n, act, seed=4000 + m)
    wq, sw = prep_rows(dev(d["w"]), g)
    if layout == "decode":
        wl, sl = ck.ck_weight_pack_decode(wq, sw), None
    else:
        wl, sl = ck.ck_weight_pack(wq), sw
    x = bf16_dev(d["x"])
    bias = dev(rng.standard_normal(n).astype(np.float32))
    res = bf16_dev(W.to_bf16_bits(rng.standard_normal((m, n)).astype(np.float32)))
    y = ck.ck_int8_linear(x, wl, sl, g, act, layout=layout, bias=bias, residual=res)
    xq, sx = act_quant(x, act, g, k=k, layout="blocked")
    y_st = ck.ck_int8_gemm_bf16(xq, sx, wl, sl, layout=layout, bias=bias, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_st.view(torch.int16))


@pytest.mark.parametrize("m,k,act,g", [(1, 3072, 0, 128), (2, 3072, 0, 128), (2, 8192, 0, 64),
                                        (1, 12288, 1, 128), (1, 4096, 1, 256), (2, 12288, 1, 128),
                                        (2, 16384, 1, 64), (1, 64, 0, 64)])
def test_w8a16_fused_equals_the_stages(m, k, act, g):
    """ck_int8_linear_w8a16 at the fewest rows (one kernel that rotates the
    rows itself) equals ck_act_rotate_bf16 followed by the W8A16 GEMM, bit for
    bit, with bias and residual."""
    say(f"w8a16 fused vs stages m={m} k={k} act={act} g={g}")
    n = 1040
    rng = np.random.default_rng(79 + m + k)
    d = W.case(m, k, n, act, seed=4100 + m)
    wq, sw = prep_rows(dev(d["w"]), g)
    wb = ck.ck_weight_pack(wq)
    x = bf16_dev(d["x"])
    bias = dev(rng.standard_normal(n).astype(np.float32))
    res = bf16_dev(W.to_bf16_bits(rng.standard_normal((m, n)).astype(np.float32)))
    y = ck.ck_int8_linear_w8a16(x, wb, sw, g, act, bias=bias, residual=res)
    xr = ck.ck_act_rotate_bf16(x, act, g, k=k, layout="blocked")
    y_st = ck.ck_w8a16_gemm_bf16(xr, wb, sw, m, bias=bias, residual=res)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_st.view(torch.int16))


def test_decode_rejects_more_than_64_rows():
    say("decode layout with m=65 -> CK_EUNSUPPORTED")
    wq, sw = prep_rows(torch.zeros((32, 256), dtype=torch.float32, device=DEV), 128)
    wd = ck.ck_weight_pack_decode(wq, sw)
    x = torch.zeros((65, 256), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ck.CKError, match="CK_EUNSUPPORTED"):
        ck.ck_int8_linear(x, wd, None, 128, layout="decode")


# ---------------------------------------------------------------------------
# W8A16: BF16 rotated activations times INT8 weights (comfy-kitchen PR #277,
# "Notes for the reviewer")
# ---------------------------------------------------------------------------
def to_blocked_bf16(a):
    """Row-major BF16 bits [R, K] -> the BF16 blocked layout of include/ck.h:
    rows padded to 256 (zeros), 2 KB per (r / 32, k / 32), inside it
    ((k % 16) / 8, (k % 32) / 16, r % 32, k % 8)."""
    r, k = a.shape
    rp = -(-r // 256) * 256
    p = np.zeros((rp, k), dtype=np.uint16)
    p[:r] = a
    return np.ascontiguousarray(
        p.reshape(rp // 32, 32, k // 32, 2, 2, 8).transpose(0, 2, 4, 3, 1, 5)).reshape(rp, k)


def from_blocked_bf16(b, rows):
    rp, k = b.shape
    a = b.reshape(rp // 32, k // 32, 2, 2, 32, 8).transpose(0, 4, 1, 3, 2, 5).reshape(rp, k)
    return np.ascontiguousarray(a[:rows])


def w8a16_bound(orc, x_rot, wq, sw, y_ref, k, bias=None, residual=None):
    """Elementwise bound of the W8A16 result against the oracle: FP32
    accumulation in any order errs by at most gamma_k * sum|x q| (every product
    is exact), scaled by s_w; the epilogue's FP32 roundings add 2^-23 of their
    operands; the two BF16 roundings differ by at most one BF16 ulp."""
    u = 2.0 ** -24
    gamma = k * u / (1 - k * u)
    s_abs = orc.w8a16_abs_acc(x_rot, wq) * sw.astype(np.float64)[None, :]
    t = np.abs(orc.w8a16_acc(x_rot, wq) * sw.astype(np.float64)[None, :])
    if bias is not None:
        t = t + np.abs(bias.astype(np.float64))[None, :]
    if residual is not None:
        t = t + np.abs(orc.bf16_to_f32(residual).astype(np.float64))
    yr = orc.bf16_to_f32(y_ref).astype(np.float64)
    ulp = np.spacing(np.maximum(np.abs(yr), 1e-38).astype(np.float32)).astype(np.float64) * 65536.0
    return ulp + gamma * s_abs + 2 * 2.0 ** -23 * t


def assert_w8a16_close(orc, got, want, x_rot, wq, sw, k, what, bias=None, residual=None):
    g = orc.bf16_to_f32(got).astype(np.float64)
    w = orc.bf16_to_f32(want).astype(np.float64)
    bound = w8a16_bound(orc, x_rot, wq, sw, want, k, bias, residual)
    bad = np.abs(g - w) > bound
    assert not bad.any(), f"{what}: {np.count_nonzero(bad)} elements beyond the FP32-accumulation bound"
    say(f"{what}: {np.count_nonzero(got != want)} of {got.size} BF16 elements differ by <= bound; "
        f"relL2 vs oracle {orc.rel_l2(got, w):.2e}")


ROTATE_CASES = [  # (m, k, act, g)
    (1, 256, 0, 128), (37, 384, 1, 128), (300, 1024, 0, 64), (257, 512, 1, 256), (64, 3072, 1, 128),
    # from m * k = 2^20 and 512 rows the blocked layout of x comes from the line
    # kernel: one group per lane with idle group slots (k = 640), two per lane
    # (ragged m), four at g = 256, a row in five slices, a ragged last slice of two
    (2049, 640, 0, 64), (1000, 1536, 0, 128), (520, 4096, 0, 256), (600, 5120, 0, 64), (521, 7424, 0, 256),
    # SwiGLU from m * k = 2^22 and 1024 rows, below the silu table's sizes: the
    # line kernel with silu_f32 itself (c2's shape; g = 64 and 256, ragged m)
    (2048, 3072, 1, 128), (1100, 4096, 1, 64), (1501, 5120, 1, 256),
    # short rows on the line kernel: fewer groups than a workgroup has slots
    (2048, 512, 0, 64), (4096, 256, 0, 256), (8192, 512, 1, 128),
]


@pytest.mark.parametrize("m,k,act,g", ROTATE_CASES)
def test_act_rotate_bf16_bit_exact(orc, m, k, act, g):
    say(f"act_rotate_bf16 m={m} k={k} act={act} g={g}")
    d = W.case(m, k, 16, act, seed=500 + m)
    if m > 1:
        d["x"] = plant_zero_rows(d["x"], k, act)
    x = bf16_dev(d["x"])
    want = orc.act_rotate_bf16(d["x"], act, g, k=k)
    np.testing.assert_array_equal(bf16_host(ck.ck_act_rotate_bf16(x, act, g, k=k)), want)
    blk = bf16_host(ck.ck_act_rotate_bf16(x, act, g, k=k, layout="blocked"))
    np.testing.assert_array_equal(from_blocked_bf16(blk, m), want)


# The SwiGLU rotation at sizes where the blocked layout comes from the line
# kernel with its silu table (from m * k = 2^24 with m >= 512, or 2^23 with 8
# rows per CU): two groups per lane in four slices (k = 8192), two in two
# slices (k = 4096, ragged m), one in five slices (k = 5120), three (c5's
# width, ragged m), and a ragged last slice (k = 7424); row-major from the
# row-wise kernel at the same sizes.  With random
# inputs a few rotated values cancel to exactly zero at these sizes (the
# sign-folded butterflies hold them as -0 in half the lanes): they and the
# planted zero rows check that a zero is written as +0.
ROTATE_TAB_CASES = [  # (m, k, g)
    (2048, 8192, 128), (4097, 4096, 64), (2100, 5120, 64), (3001, 12288, 256), (2300, 7424, 256),
    (512, 32768, 128),   # CK_MAX_K
]


@pytest.mark.parametrize("m,k,g", ROTATE_TAB_CASES)
def test_act_rotate_bf16_swiglu_tab_bit_exact(orc, m, k, g):
    say(f"act_rotate_bf16 swiglu (table kernel) m={m} k={k} g={g}")
    d = W.case(m, k, 16, 1, seed=510 + m)
    d["x"] = plant_zero_rows(d["x"], k, 1)
    x = bf16_dev(d["x"])
    want = orc.act_rotate_bf16(d["x"], 1, g, k=k)
    np.testing.assert_array_equal(bf16_host(ck.ck_act_rotate_bf16(x, 1, g, k=k)), want)
    blk = bf16_host(ck.ck_act_rotate_bf16(x, 1, g, k=k, layout="blocked"))
    np.testing.assert_array_equal(from_blocked_bf16(blk, m), want)


@pytest.mark.parametrize("m,k,act,g,pad,layout", [
    (300, 1024, 0, 128, 32, "rows"),          # the per-row kernel
    (2048, 3072, 0, 128, 64, "blocked"),      # the line quantizer
    (4096, 4096, 0, 64, 16, "blocked"),       # staged per-row codes
    (2100, 8192, 1, 128, 128, "blocked"),     # the table kernel, staged
    (2048, 4096, 1, 64, 8, "rows"),           # the table kernel, row-major codes
])
def test_act_quant_padded_rows_bit_exact(orc, m, k, act, g, pad, layout):
    """Rows with a leading dimension past their values (ldx = k or 2k, plus
    pad, NaN in the padding) through each quantizer kernel."""
    say(f"act_quant padded rows m={m} k={k} act={act} g={g} pad={pad} {layout}")
    d = W.case(m, k, 16, act, seed=540 + m)
    width = d["x"].shape[1]
    xp = np.full((m, width + pad), 0x7FC0, dtype=np.uint16)
    xp[:, :width] = d["x"]
    q_o, s_o = orc.act_quant(d["x"], act, g, k=k)
    q, sc = ck.ck_act_quant(bf16_dev(xp), act, g, k=k, layout=layout)
    q = host(q)
    np.testing.assert_array_equal(host(sc).reshape(-1).view(np.uint32), s_o.view(np.uint32))
    np.testing.assert_array_equal(q if layout == "rows" else from_blocked(q, m), q_o)


@pytest.mark.parametrize("m,k,act,g,pad", [(600, 2048, 0, 128, 64), (1100, 4096, 1, 64, 128),
                                           (2100, 4096, 1, 256, 8)])
def test_act_rotate_bf16_padded_rows_bit_exact(orc, m, k, act, g, pad):
    """Rows with a leading dimension past their values (ldx = k or 2k, plus
    pad) on the line kernel: x, and SwiGLU without and with the silu table."""
    say(f"act_rotate_bf16 padded rows m={m} k={k} act={act} g={g} pad={pad}")
    d = W.case(m, k, 16, act, seed=530 + m)
    width = d["x"].shape[1]
    xp = np.full((m, width + pad), 0x7FC0, dtype=np.uint16)     # NaN in the padding
    xp[:, :width] = d["x"]
    want = orc.act_rotate_bf16(xp, act, g, k=k)
    np.testing.assert_array_equal(want, orc.act_rotate_bf16(d["x"], act, g, k=k))
    blk = bf16_host(ck.ck_act_rotate_bf16(bf16_dev(xp), act, g, k=k, layout="blocked"))
    np.testing.assert_array_equal(from_blocked_bf16(blk, m), want)


def _random_rotate_shapes(count=32, seed=2027):
    """Seeded random shapes of the line rotation: x from 512 rows and m * k >=
    2^20; SwiGLU from 1024 rows and m * k >= 2^22 (with and without the silu
    table); k a multiple of the group, up to 8192 (x) or 6144 (SwiGLU)."""
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < count:
        act = int(rng.integers(0, 2))
        g = int(rng.choice([64, 128, 256]))
        k = g * int(rng.integers(max(1, 1024 // g), (8192 if act == 0 else 6144) // g + 1))
        lo = 1024 if act else 512
        m = int(rng.integers(lo, lo + 3000))
        if m * k >= (1 << 22 if act else 1 << 20):
            shapes.append((m, k, act, g))
    return shapes


@pytest.mark.parametrize("m,k,act,g", _random_rotate_shapes())
def test_act_rotate_bf16_random_blocked_bit_exact(orc, m, k, act, g):
    say(f"act_rotate_bf16 random blocked m={m} k={k} act={act} g={g}")
    d = W.case(m, k, 16, act, seed=m * 7 + k)
    x = bf16_dev(d["x"])
    want = orc.act_rotate_bf16(d["x"], act, g, k=k)
    blk = bf16_host(ck.ck_act_rotate_bf16(x, act, g, k=k, layout="blocked"))
    np.testing.assert_array_equal(from_blocked_bf16(blk, m), want)


W8A16_GEMM_SHAPES = [  # (m, n, k): every tile shape, k-stage counts 1, 2, 3 and more,
    # ragged m and n, a partial last round of tiles; the few-tile shapes: 64 x 64 with four
    # k-slices per half stage (300, 272, 1024), (48, 4112, 256) or two (100, 8192, 128)
    (77, 144, 192), (300, 272, 1024), (1000, 1040, 640),
    (513, 4112, 128), (4000, 4080, 192), (4000, 3056, 320), (2560, 6144, 256), (2048, 1024, 3072),
    # the few-row kernel (m <= 64): 1, 2 and 4 row fragments, short and long k
    (1, 16, 64), (1, 4096, 4096), (2, 48, 1024), (16, 1024, 3072), (17, 2048, 128), (33, 4096, 4096),
    (64, 128, 256), (64, 4096, 12288), (65, 272, 1024), (128, 4096, 4096),
    # few rows on tiles (n > 16 * CUs)
    (48, 4112, 256), (100, 8192, 128),
    # 64 x 128 and 128 x 128 tiles with one k-slice per half stage (k % 128 == 64, or
    # more tiles than CUs), and 128 x 128 tiles with two
    (300, 272, 192), (600, 1200, 448), (320, 11008, 256), (1500, 4000, 320),
    (1024, 4096, 1024), (700, 5008, 256),
    # few rows, two weight groups per workgroup, and n % 32 != 0
    (16, 16384, 128), (29, 16416, 320), (32, 24576, 64), (18, 16400, 128), (24, 8192, 192),
    (20, 28672, 128),
]


@pytest.mark.parametrize("m,n,k", W8A16_GEMM_SHAPES)
def test_w8a16_gemm_exact_on_integer_activations(orc, m, n, k):
    """Integer activations with |x| * 127 * k < 2^24 keep every partial sum an
    integer below 2^24, so FP32 accumulation in any order is exact:
    accumulators and BF16 outputs must equal the oracle bit for bit."""
    say(f"w8a16 gemm integer activations m={m} n={n} k={k}")
    rng = np.random.default_rng(3 * m + n + k)
    xmax = min(32, (1 << 24) // (127 * k) - 1)
    xr = orc.f32_to_bf16(rng.integers(-xmax, xmax + 1, size=(m, k)).astype(np.float32))
    wq = rng.integers(-127, 128, size=(n, k), dtype=np.int8)
    sw = (rng.random(n, dtype=np.float32) * 1e-3).astype(np.float32)
    xb, wb = bf16_dev(to_blocked_bf16(xr)), dev(to_blocked(wq))
    acc_o = orc.w8a16_acc(xr, wq)
    np.testing.assert_array_equal(host(ck.ck_w8a16_gemm_f32(xb, wb, m, n)).astype(np.float64), acc_o)
    y = bf16_host(ck.ck_w8a16_gemm_bf16(xb, wb, dev(sw), m))
    np.testing.assert_array_equal(y, orc.w8a16_epilogue(acc_o, sw))
    bias = rng.standard_normal(n).astype(np.float32)
    res = orc.f32_to_bf16(rng.standard_normal((m, n)).astype(np.float32))
    y = bf16_host(ck.ck_w8a16_gemm_bf16(xb, wb, dev(sw), m, bias=dev(bias), residual=bf16_dev(res)))
    np.testing.assert_array_equal(y, orc.w8a16_epilogue(acc_o, sw, bias, res))


W8A16_LINEAR = [  # (m, k, n, act, g)
    (1, 256, 16, 0, 128), (7, 384, 48, 1, 128), (300, 1024, 272, 1, 128), (129, 512, 320, 0, 64),
    (200, 768, 96, 1, 256), (1000, 640, 1040, 0, 128), (4000, 256, 4080, 1, 128), (5, 64, 32, 1, 64),
    (1500, 384, 4000, 0, 128), (700, 256, 5008, 1, 128), (2, 4096, 1040, 1, 256), (2, 3072, 528, 0, 128),
]


@pytest.mark.parametrize("m,k,n,act,g", W8A16_LINEAR)
def test_int8_linear_w8a16_within_bound(orc, m, k, n, act, g):
    say(f"int8_linear_w8a16 m={m} k={k} n={n} act={act} g={g}")
    d = W.case(m, k, n, act, seed=700 + m, zero_rows=(m // 2,) if m > 2 else ())
    wq_o, sw_o = orc.weight_prep(d["w"], g)
    wq, sw = prep_rows(dev(d["w"]), g)
    x = bf16_dev(d["x"])
    y = bf16_host(ck.ck_int8_linear_w8a16(x, ck.ck_weight_pack(wq), sw, g, act))
    ref = orc.w8a16_linear(d["x"], act, wq_o, sw_o, g, return_all=True)
    assert_w8a16_close(orc, y, ref["y"], ref["x_rot"], wq_o, sw_o, k, "w8a16 y")
    if m > 2:
        assert not y[m // 2].any()
    rng = np.random.default_rng(m + n)
    bias = rng.standard_normal(n).astype(np.float32)
    res = orc.f32_to_bf16(rng.standard_normal((m, n)).astype(np.float32))
    y = bf16_host(ck.ck_int8_linear_w8a16(x, ck.ck_weight_pack(wq), sw, g, act, bias=dev(bias),
                                          residual=bf16_dev(res)))
    want = orc.w8a16_epilogue(ref["acc"], sw_o, bias, res)
    assert_w8a16_close(orc, y, want, ref["x_rot"], wq_o, sw_o, k, "w8a16 y + bias + residual",
                       bias=bias, residual=res)


@pytest.mark.parametrize("name", ["c2", "c4"])
def test_w8a16_full_workload_all_elements(orc, name):
    wl = W.WORKLOADS[name]
    d = inputs(name)
    say(f"int8_linear_w8a16 full {name}: {wl.desc}")
    wq, sw = ck.ck_weight_prep(dev(d["w"]), wl.group)
    y = ck.ck_int8_linear_w8a16(bf16_dev(d["x"]), wq, sw, wl.group, wl.act)
    torch.cuda.synchronize()
    wq_o, sw_o = prepped(orc, name)
    ref = orc.w8a16_linear(d["x"], wl.act, wq_o, sw_o, wl.group, return_all=True)
    y_h = bf16_host(y)
    assert_w8a16_close(orc, y_h, ref["y"], ref["x_rot"], wq_o, sw_o, wl.k, f"{name} w8a16 all rows")
    y64 = ref_f64(orc, name)
    e16 = orc.rel_l2(y_h, y64)
    e8 = orc.rel_l2(full_ref(orc, name)["y"], y64)
    say(f"{name}: relL2 vs float64  w8a16 gpu={e16:.5f}  int8 oracle={e8:.5f}")
    assert e16 < e8


def _mlp_w8a16_check(orc, xb, rows, w_gu_o, s_gu_o, w_d_o, s_d_o, g, y, y1, what):
    """Stage 1 against the oracle on the same input; stage 2 against the oracle
    applied to the GPU's own stage-1 output (stage 1 is exact only up to FP32
    accumulation order, so its rounding differences must not be compounded)."""
    h = xb.shape[1]
    i = w_d_o.shape[1]
    r1 = orc.w8a16_linear(xb[rows], 0, w_gu_o, s_gu_o, g, return_all=True)
    assert_w8a16_close(orc, y1[rows], r1["y"], r1["x_rot"], w_gu_o, s_gu_o, h, what + " stage 1")
    r2 = orc.w8a16_linear(y1[rows], 1, w_d_o, s_d_o, g, return_all=True)
    assert_w8a16_close(orc, y[rows], r2["y"], r2["x_rot"], w_d_o, s_d_o, i, what + " stage 2")


@pytest.mark.parametrize("m", [300, 1, 2, 3])
def test_swiglu_mlp_w8a16(orc, m):
    """At m <= 2 each stage is one launch (the rotation inside the GEMM); at
    m = 3 the rotations are launches of their own."""
    h, i, g = 1024, 2816, 128
    say(f"swiglu_mlp_w8a16 m={m} h={h} i={i}")
    rng = np.random.default_rng(91)
    xb = W.to_bf16_bits(rng.standard_normal((m, h)).astype(np.float32))
    w_gu = (0.02 * rng.standard_normal((2 * i, h))).astype(np.float32)
    w_dn = (0.01 * rng.standard_normal((h, i))).astype(np.float32)
    gq, gs = prep_rows(dev(w_gu), g)
    dq, ds = prep_rows(dev(w_dn), g)
    pgu, pd = ck.ck_weight_pack(gq), ck.ck_weight_pack(dq)
    x = bf16_dev(xb)
    y = ck.ck_swiglu_mlp_w8a16(x, pgu, gs, pd, ds, g)
    # the same stages called one by one compose to the block bit for bit
    y1 = ck.ck_w8a16_gemm_bf16(ck.ck_act_rotate_bf16(x, 0, g, layout="blocked"), pgu, gs, m)
    y_st = ck.ck_w8a16_gemm_bf16(ck.ck_act_rotate_bf16(y1, 1, g, layout="blocked"), pd, ds, m)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_st.view(torch.int16))
    (gq_o, gs_o), (dq_o, ds_o) = orc.weight_prep(w_gu, g), orc.weight_prep(w_dn, g)
    _mlp_w8a16_check(orc, xb, np.arange(m), gq_o, gs_o, dq_o, ds_o, g, bf16_host(y), bf16_host(y1),
                     "mlp w8a16")
    y64 = orc.reference_mlp_f64(xb, w_gu, w_dn)
    e16 = orc.rel_l2(bf16_host(y), y64)
    e8 = orc.rel_l2(orc.swiglu_mlp(xb, gq_o, gs_o, dq_o, ds_o, g), y64)
    say(f"mlp: relL2 vs float64  w8a16 gpu={e16:.5f}  int8 oracle={e8:.5f}")
    assert e16 < e8


def test_swiglu_mlp_w8a16_full_c5_all_elements(orc):
    wl = W.WORKLOADS["c5"]
    d = inputs("c5")
    say(f"swiglu_mlp_w8a16 full c5: {wl.desc}")
    g = wl.group
    pgu, gs = ck.ck_weight_prep(dev(d["w_gu"]), g)
    pd, ds = ck.ck_weight_prep(dev(d["w_down"]), g)
    x = bf16_dev(d["x"])
    y = ck.ck_swiglu_mlp_w8a16(x, pgu, gs, pd, ds, g)
    y1 = ck.ck_w8a16_gemm_bf16(ck.ck_act_rotate_bf16(x, 0, g, layout="blocked"), pgu, gs, wl.m)
    torch.cuda.synchronize()
    (gq_o, gs_o), (dq_o, ds_o) = prepped(orc, "c5", "w_gu"), prepped(orc, "c5", "w_down")
    y_h = bf16_host(y)
    _mlp_w8a16_check(orc, d["x"], np.arange(wl.m), gq_o, gs_o, dq_o, ds_o, g, y_h, bf16_host(y1),
                     "c5 w8a16")
    say(f"c5 w8a16: relL2 vs float64 {orc.rel_l2(y_h, ref_f64(orc, 'c5')):.5f}")


@pytest.mark.parametrize("m", [1, 16, 64])
def test_swiglu_mlp_decode_c5_dims_bit_exact(orc, m):
    """c5's block dimensions at decode sizes, both weights in the decode layout,
    in the configuration `bench.py --decode-mlp` times: bit-exact against the
    oracle on the first m tokens of c5's input."""
    wl = W.WORKLOADS["c5"]
    d = inputs("c5")
    say(f"swiglu_mlp decode c5 dims m={m}")
    g = wl.group
    key = ("c5", "decode_weights")
    if key not in _cache:
        gq, gs = prep_rows(dev(d["w_gu"]), g)
        dq, ds = prep_rows(dev(d["w_down"]), g)
        _cache[key] = (ck.ck_weight_pack_decode(gq, gs), ck.ck_weight_pack_decode(dq, ds))
    dgu, dd = _cache[key]
    xb = np.ascontiguousarray(d["x"][:m])
    y = ck.ck_swiglu_mlp(bf16_dev(xb), dgu, None, dd, None, g, layout="decode")
    (gq_o, gs_o), (dq_o, ds_o) = prepped(orc, "c5", "w_gu"), prepped(orc, "c5", "w_down")
    np.testing.assert_array_equal(bf16_host(y), orc.swiglu_mlp(xb, gq_o, gs_o, dq_o, ds_o, g))


def test_calls_replay_bit_exact_from_a_hip_graph():
    """Every entry point only enqueues kernels (no allocation, memset or
    synchronisation), so a call sequence can be captured into a HIP graph.
    Each replay, with new inputs copied in eagerly between replays, must match
    the eager calls bit for bit."""
    say("graph capture: ck_swiglu_mlp (decode, m=1; blocked, m=2 and 2048) + ck_swiglu_mlp_w8a16 (m=1 and "
        "2048) + ck_int8_linear (blocked, m=300)")
    g = 128
    rng = np.random.default_rng(17)
    h, i = 1024, 2816
    gq, gs = prep_rows(dev((0.02 * rng.standard_normal((2 * i, h))).astype(np.float32)), g)
    dq, ds = prep_rows(dev((0.01 * rng.standard_normal((h, i))).astype(np.float32)), g)
    dgu, dd = ck.ck_weight_pack_decode(gq, gs), ck.ck_weight_pack_decode(dq, ds)
    wl, sl = prep_rows(dev((0.02 * rng.standard_normal((528, 768))).astype(np.float32)), g)
    wlb = ck.ck_weight_pack(wl)
    x1 = torch.zeros((1, h), dtype=torch.bfloat16, device=DEV)
    x2 = torch.zeros((300, 768), dtype=torch.bfloat16, device=DEV)
    y1 = torch.empty((1, h), dtype=torch.bfloat16, device=DEV)
    y2 = torch.empty((300, 528), dtype=torch.bfloat16, device=DEV)
    ws1 = torch.empty(ck.lib().ck_swiglu_mlp_workspace_size(1, h, i), dtype=torch.uint8, device=DEV)
    ws2 = torch.empty(ck.lib().ck_int8_linear_workspace_size(300, 768, 528), dtype=torch.uint8, device=DEV)
    bgu, bd = ck.ck_weight_pack(gq), ck.ck_weight_pack(dq)
    x3 = torch.zeros((2, h), dtype=torch.bfloat16, device=DEV)
    y3 = torch.empty((2, h), dtype=torch.bfloat16, device=DEV)
    y4 = torch.empty((1, h), dtype=torch.bfloat16, device=DEV)
    ws3 = torch.empty(ck.lib().ck_swiglu_mlp_workspace_size(2, h, i), dtype=torch.uint8, device=DEV)
    ws4 = torch.empty(ck.lib().ck_swiglu_mlp_w8a16_workspace_size(1, h, i), dtype=torch.uint8, device=DEV)
    # m = 2048 with i = 8192: the line x quantizer, the staged table quantizer
    # and the large-tile GEMMs; in W8A16 both line rotations (x, SwiGLU with
    # the silu table)
    i5 = 8192
    gq5, gs5 = prep_rows(dev((0.02 * rng.standard_normal((2 * i5, h))).astype(np.float32)), g)
    dq5, ds5 = prep_rows(dev((0.01 * rng.standard_normal((h, i5))).astype(np.float32)), g)
    bgu5, bd5 = ck.ck_weight_pack(gq5), ck.ck_weight_pack(dq5)
    x5 = torch.zeros((2048, h), dtype=torch.bfloat16, device=DEV)
    y5 = torch.empty((2048, h), dtype=torch.bfloat16, device=DEV)
    y6 = torch.empty((2048, h), dtype=torch.bfloat16, device=DEV)
    ws5 = torch.empty(ck.lib().ck_swiglu_mlp_workspace_size(2048, h, i5), dtype=torch.uint8, device=DEV)
    ws6 = torch.empty(ck.lib().ck_swiglu_mlp_w8a16_workspace_size(2048, h, i5), dtype=torch.uint8, device=DEV)

    def calls():
        ck.ck_swiglu_mlp(x1, dgu, None, dd, None, g, out=y1, workspace=ws1, layout="decode")
        ck.ck_int8_linear(x2, wlb, sl, g, out=y2, workspace=ws2, layout="blocked")
        ck.ck_swiglu_mlp(x3, bgu, gs, bd, ds, g, out=y3, workspace=ws3, layout="blocked")
        ck.ck_swiglu_mlp_w8a16(x1, bgu, gs, bd, ds, g, out=y4, workspace=ws4)
        ck.ck_swiglu_mlp(x5, bgu5, gs5, bd5, ds5, g, out=y5, workspace=ws5, layout="blocked")
        ck.ck_swiglu_mlp_w8a16(x5, bgu5, gs5, bd5, ds5, g, out=y6, workspace=ws6)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(3):
        a1 = rng.standard_normal((1, h)).astype(np.float32)
        a2 = rng.standard_normal((300, 768)).astype(np.float32)
        x1.copy_(torch.from_numpy(a1).to(DEV).to(torch.bfloat16))
        x2.copy_(torch.from_numpy(a2).to(DEV).to(torch.bfloat16))
        x3.copy_(torch.from_numpy(rng.standard_normal((2, h)).astype(np.float32)).to(DEV).to(torch.bfloat16))
        x5.copy_(torch.from_numpy(rng.standard_normal((2048, h)).astype(np.float32)).to(DEV).to(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (y1, y2, y3, y4, y5, y6)]
        calls()                                   # eager reference on the same inputs
        torch.cuda.synchronize()
        for what, gt, want in zip(("mlp decode", "linear", "mlp blocked", "mlp w8a16", "mlp blocked m=2048",
                                   "mlp w8a16 m=2048"), got, (y1, y2, y3, y4, y5, y6)):
            assert torch.equal(gt.view(torch.int16), want.view(torch.int16)), f"replay {rep}: {what} differs"
            assert gt.abs().sum() > 0, f"replay {rep}: {what} is all zeros"


def test_concurrent_calls_on_separate_streams():
    """The library keeps no per-call state of its own (scratch is the caller's
    workspace), so host threads calling it on separate streams with separate
    buffers get the results of sequential calls, bit for bit."""
    import threading
    say("4 host threads x 5 ck_int8_linear calls on separate streams")
    g = 128
    rng = np.random.default_rng(23)
    wq, sw = prep_rows(dev((0.02 * rng.standard_normal((1040, 1024))).astype(np.float32)), g)
    wb = ck.ck_weight_pack(wq)
    xs = [bf16_dev(W.to_bf16_bits(rng.standard_normal((300 + 37 * t, 2048)).astype(np.float32)))
          for t in range(4)]
    want = [ck.ck_int8_linear(x, wb, sw, g, "swiglu", layout="blocked") for x in xs]
    torch.cuda.synchronize()
    got = [[None] * 5 for _ in range(4)]
    errors = []

    def worker(t):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for r in range(5):
                    got[t][r] = ck.ck_int8_linear(xs[t], wb, sw, g, "swiglu", layout="blocked")
            st.synchronize()
        except Exception as e:   # surfaced below
            errors.append(e)
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=60)
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(4):
        for r in range(5):
            assert torch.equal(got[t][r].view(torch.int16), want[t].view(torch.int16)), (t, r)


def _random_cases(count, seed):
    """Random (m, k, n, act, group, layout, epilogue): m drawn from 1..3 (the
    fused decode kernel), 1..64 and 65..799; k either a few groups or a multiple
    of 128 up to 4096 (the few-tile kernels' two and four k-slices)."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        g = int(rng.choice([32, 64, 128, 256]))
        k = int(rng.choice([g * int(rng.integers(1, 9)), 128 * int(rng.integers(1, 33))]))
        step = max(g, 64)
        k = max(step, (k + step - 1) // step * step)
        n = 16 * int(rng.integers(1, 300))
        m = int(rng.choice([int(rng.integers(1, 4)), int(rng.integers(1, 65)), int(rng.integers(65, 800))]))
        layout = str(rng.choice(["rows", "blocked", "decode"] if m <= 64 else ["rows", "blocked"]))
        act = int(rng.integers(0, 2))
        extra = bool(rng.integers(0, 2))
        cases.append((m, k, n, act, g, layout, extra))
    return cases


@pytest.mark.parametrize("m,k,n,act,g,layout,extra", _random_cases(96, 2024))
def test_random_shapes_bit_exact(orc, m, k, n, act, g, layout, extra):
    """Seeded random shapes over every layout, activation, group and epilogue:
    bit-exact against the oracle."""
    say(f"random m={m} k={k} n={n} act={act} g={g} layout={layout} extra={extra}")
    d = W.case(m, k, n, act, seed=m * 7 + n)
    wq_o, sw_o = orc.weight_prep(d["w"], g)
    wq, sw = prep_rows(dev(d["w"]), g)
    if layout == "blocked":
        wq = ck.ck_weight_pack(wq)
    elif layout == "decode":
        wq, sw = ck.ck_weight_pack_decode(wq, sw), None
    bias = res = None
    if extra:
        rng = np.random.default_rng(m + n + k)
        bias = rng.standard_normal(n).astype(np.float32)
        res = orc.f32_to_bf16(rng.standard_normal((m, n)).astype(np.float32))
    y = ck.ck_int8_linear(bf16_dev(d["x"]), wq, sw, g, act, layout=layout,
                          bias=None if bias is None else dev(bias),
                          residual=None if res is None else bf16_dev(res))
    np.testing.assert_array_equal(bf16_host(y), orc.int8_linear(d["x"], act, wq_o, sw_o, g, bias=bias,
                                                                residual=res))


def _random_w8a16_shapes(count, seed):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 800)), 16 * int(rng.integers(1, 300)), 64 * int(rng.integers(1, 64)))
            for _ in range(count)]


@pytest.mark.parametrize("m,n,k", _random_w8a16_shapes(32, 2025))
def test_random_w8a16_gemm_exact(orc, m, n, k):
    """Seeded random W8A16 GEMM shapes on integer activations (exact in any
    summation order): accumulators and outputs bit-exact."""
    test_w8a16_gemm_exact_on_integer_activations(orc, m, n, k)
