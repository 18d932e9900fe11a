"""C ABI checks that need no GPU: the library loads, exports every entry point
include/ck.h declares, and rejects bad arguments on the host (returning the
documented status, enqueueing nothing) before any device is touched."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

import swiglu_mlp_amd as ck

HEADER = os.path.join(ROOT, "include", "ck.h")
OK, EINVAL, ESHAPE, EUNSUP, EWS = 0, 1, 2, 3, 4
FAKE = 1 << 20          # an aligned non-null address that is never dereferenced


@pytest.fixture(scope="module")
def L():
    return ck.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ck_\w+)\s*\(", text)))


def test_header_declares_the_four_path_calls():
    names = declared_functions()
    for n in ("ck_weight_prep", "ck_act_quant", "ck_int8_linear", "ck_swiglu_mlp"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_every_declared_symbol_has_a_c_signature(L):
    # ctypes passes undeclared int arguments as C int, masking pointers to 32 bits
    for name in declared_functions():
        assert getattr(L, name).argtypes is not None, name
        assert getattr(L, name).restype is not None, name


def test_status_strings_and_version(L):
    assert L.ck_version().decode().startswith("ck-convrot")
    for s in range(6):
        assert L.ck_status_str(s)
    assert b"unknown" in L.ck_status_str(99)


def test_workspace_sizes(L):
    assert L.ck_int8_linear_workspace_size(0, 256, 32) == 0
    assert L.ck_int8_linear_workspace_size(3, 256, 32) == 256 * 256 + 256   # blocked codes: 256 rows
    # 64 x 4096 x 12288 takes split K on 256 CUs (four k ranges of 64 x 64 tiles): the int32 partials follow
    # the codes and scales
    assert L.ck_int8_linear_workspace_size(64, 12288, 4096) == 256 * 12288 + 256 + 4 * 64 * 4096 * 4
    assert L.ck_int8_linear_workspace_size(64, 4096, 4096) == 256 * 4096 + 256            # k too small to split
    assert L.ck_int8_linear_workspace_size(47, 12288, 4096) == 256 * 12288 + 256          # m too small
    assert L.ck_swiglu_mlp_workspace_size(64, 3072, 12288) > L.ck_swiglu_mlp_workspace_size(64, 3072, 4096)
    assert L.ck_blocked_rows(1) == 256 and L.ck_blocked_rows(256) == 256 and L.ck_blocked_rows(257) == 512
    assert L.ck_blocked_size(300, 128) == 512 * 128 and L.ck_blocked_size(0, 128) == 0
    ws = L.ck_swiglu_mlp_workspace_size(4096, 3072, 12288)
    assert ws >= 4096 * 3072 + 4096 * 4 + 4096 * 2 * 12288 * 2 + 4096 * 12288 + 4096 * 4
    assert ws % 256 == 0


@pytest.mark.parametrize("k,group,want", [
    (256, 128, OK), (192, 128, ESHAPE), (96, 32, ESHAPE), (256, 96, EUNSUP),
    (256, 512, EUNSUP), (0, 128, ESHAPE), (65536, 128, EUNSUP), (256, 0, EUNSUP),
])
def test_weight_prep_shape_checks(L, k, group, want):
    # n == 0 makes a valid call a no-op, so nothing is launched on success
    assert L.ck_weight_prep(FAKE, 0, k, group, FAKE, FAKE, None) == want


def test_weight_prep_null_and_alignment(L):
    assert L.ck_weight_prep(None, 4, 256, 128, FAKE, FAKE, None) == EINVAL
    assert L.ck_weight_prep(FAKE + 4, 4, 256, 128, FAKE, FAKE, None) == EINVAL
    assert L.ck_weight_prep(FAKE, -1, 256, 128, FAKE, FAKE, None) == ESHAPE


def test_act_quant_checks(L):
    f = L.ck_act_quant
    assert f(FAKE, 256, 0, 256, 0, 128, 0, FAKE, FAKE, None) == OK          # m == 0: no-op
    assert f(FAKE, 256, -2, 256, 0, 128, 0, FAKE, FAKE, None) == ESHAPE
    assert f(FAKE, 256, 4, 256, 1, 128, 0, FAKE, FAKE, None) == ESHAPE      # swiglu needs ld >= 2k
    assert f(FAKE, 260, 4, 256, 0, 128, 0, FAKE, FAKE, None) == ESHAPE      # ld % 8
    assert f(FAKE, 256, 4, 256, 7, 128, 0, FAKE, FAKE, None) == EINVAL      # unknown act
    assert f(FAKE, 256, 4, 256, 0, 128, 5, FAKE, FAKE, None) == EINVAL      # unknown layout
    assert f(None, 256, 4, 256, 0, 128, 1, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 256, 4, 256, 0, 128, 0, FAKE, None, None) == EINVAL


@pytest.mark.parametrize("layout", [0, 1])
def test_int8_linear_checks(L, layout):
    f = L.ck_int8_linear
    ws = L.ck_int8_linear_workspace_size(4, 256, 32)
    lay = layout
    assert f(FAKE, 256, 0, FAKE, FAKE, None, None, lay, 4, 40, 256, 128, FAKE, FAKE, ws, None) == ESHAPE  # n % 16
    assert f(FAKE, 256, 0, FAKE, FAKE, None, None, lay, 4, 32, 256, 128, FAKE, FAKE, ws - 1, None) == EWS
    assert f(FAKE, 256, 0, FAKE, FAKE, None, None, lay, 4, 32, 256, 128, FAKE, None, ws, None) == EWS
    assert f(FAKE, 256, 0, FAKE, FAKE, None, None, lay, 4, 32, 256, 128, FAKE, FAKE + 16, ws, None) == EWS
    assert f(FAKE, 256, 0, None, FAKE, None, None, lay, 4, 32, 256, 128, FAKE, FAKE, ws, None) == EINVAL
    assert f(FAKE, 256, 0, FAKE, FAKE, None, None, lay, 0, 32, 256, 128, FAKE, FAKE, 0, None) == OK
    assert f(FAKE, 256, 0, FAKE, FAKE, None, None, 9, 4, 32, 256, 128, FAKE, FAKE, ws, None) == EINVAL
    # optional bias (float4 reads) and residual (8-byte reads) must be aligned
    assert f(FAKE, 256, 0, FAKE, FAKE, FAKE + 4, None, lay, 4, 32, 256, 128, FAKE, FAKE, ws, None) == EINVAL
    assert f(FAKE, 256, 0, FAKE, FAKE, None, FAKE + 2, lay, 4, 32, 256, 128, FAKE, FAKE, ws, None) == EINVAL
    # operands addressed with 32-bit offsets: refuse what would overflow them
    assert f(FAKE, 32768, 0, FAKE, FAKE, None, None, lay, 70000, 32, 32768, 128, FAKE, FAKE, ws, None) == EUNSUP


def test_swiglu_mlp_checks(L):
    f = L.ck_swiglu_mlp
    ws = L.ck_swiglu_mlp_workspace_size(8, 256, 512)
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 256, 500, 128, FAKE, FAKE, ws, None) == ESHAPE
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 256, 512, 128, FAKE, FAKE, ws - 256, None) == EWS
    assert f(FAKE, None, FAKE, FAKE, FAKE, 1, 8, 256, 512, 128, FAKE, FAKE, ws, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 3, 8, 256, 512, 128, FAKE, FAKE, ws, None) == EINVAL
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 256, 512, 128, FAKE, FAKE, 0, None) == OK
    # decode layout: m <= 64 only; the weights carry their scales (NULL accepted)
    ws65 = L.ck_swiglu_mlp_workspace_size(65, 256, 512)
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, 2, 65, 256, 512, 128, FAKE, FAKE, ws65, None) == EUNSUP
    assert f(FAKE, FAKE, None, FAKE, None, 2, 8, 256, 512, 128, FAKE, FAKE, ws - 256, None) == EWS
    assert f(FAKE, FAKE, None, FAKE, None, 1, 8, 256, 512, 128, FAKE, FAKE, ws, None) == EINVAL


def test_decode_layout_checks(L):
    """Decode layout (include/ck.h): size, packing and GEMM argument checks.
    No call here reaches a kernel launch."""
    assert L.ck_decode_size(32, 256) == 2 * (64 + 16 * 256)
    assert L.ck_decode_size(0, 256) == 0 and L.ck_decode_size(16, 0) == 0
    assert L.ck_decode_size(17, 64) == 2 * (64 + 16 * 64)
    pk = L.ck_weight_pack_decode
    assert pk(FAKE, FAKE, 20, 256, FAKE, None) == ESHAPE       # n % 16
    assert pk(FAKE, FAKE, 32, 100, FAKE, None) == ESHAPE       # k % 64
    assert pk(FAKE, None, 32, 256, FAKE, None) == EINVAL       # scales needed
    assert pk(FAKE, FAKE + 4, 32, 256, FAKE, None) == EINVAL   # scales read as float4
    assert pk(FAKE, FAKE, 0, 256, FAKE, None) == OK
    assert pk(FAKE, FAKE, 32, 65536, FAKE, None) == EUNSUP
    assert pk(FAKE, FAKE, 16 * 8192, 32768, FAKE, None) == EUNSUP   # > 2^31 bytes
    assert L.ck_int8_gemm_i32(FAKE, FAKE, 2, 65, 32, 256, FAKE, None) == EUNSUP
    assert L.ck_int8_gemm_i32(FAKE, FAKE, 2, 4, 20, 256, FAKE, None) == ESHAPE
    g = L.ck_int8_gemm_bf16
    assert g(FAKE, FAKE, FAKE, None, None, None, 2, 65, 32, 256, FAKE, None) == EUNSUP
    assert g(FAKE, None, FAKE, None, None, None, 2, 4, 32, 256, FAKE, None) == EINVAL
    lin = L.ck_int8_linear
    ws = L.ck_int8_linear_workspace_size(8, 256, 32)
    assert lin(FAKE, 256, 0, FAKE, None, None, None, 2, 65, 32, 256, 128, FAKE, FAKE,
               L.ck_int8_linear_workspace_size(65, 256, 32), None) == EUNSUP
    assert lin(FAKE, 256, 0, FAKE, None, None, None, 2, 8, 32, 256, 128, FAKE, FAKE,
               ws - 1, None) == EWS
    assert lin(FAKE, 256, 0, FAKE, None, None, None, 1, 8, 32, 256, 128, FAKE, FAKE,
               ws, None) == EINVAL
    # activation codes are never in the decode layout
    assert L.ck_act_quant(FAKE, 256, 4, 256, 0, 128, 2, FAKE, FAKE, None) == EINVAL


def test_weight_pack_checks(L):
    assert L.ck_weight_pack(FAKE, 4, 100, FAKE, None) == ESHAPE
    assert L.ck_weight_pack(None, 4, 128, FAKE, None) == EINVAL
    assert L.ck_weight_pack(FAKE, 0, 128, FAKE, None) == OK
    assert L.ck_weight_pack(FAKE, 4, 65536, FAKE, None) == EUNSUP


def test_gemm_hook_checks(L):
    assert L.ck_int8_gemm_i32(FAKE, FAKE, 0, 4, 20, 256, FAKE, None) == ESHAPE
    assert L.ck_int8_gemm_i32(FAKE, FAKE, 1, 4, 32, 100, FAKE, None) == ESHAPE
    assert L.ck_int8_gemm_i32(None, FAKE, 0, 4, 32, 256, FAKE, None) == EINVAL
    assert L.ck_int8_gemm_i32(FAKE, FAKE, 3, 4, 32, 256, FAKE, None) == EINVAL
    assert L.ck_int8_gemm_bf16(FAKE, None, FAKE, FAKE, None, None, 1, 4, 32, 256, FAKE, None) == EINVAL
    assert L.ck_int8_gemm_bf16(FAKE, FAKE, FAKE, FAKE, FAKE + 8, None, 1, 4, 32, 256, FAKE, None) == EINVAL
    assert L.ck_int8_gemm_bf16(FAKE, FAKE, FAKE, FAKE, None, FAKE + 4, 1, 4, 32, 256, FAKE, None) == EINVAL
    assert L.ck_silu_f32(FAKE, -1, FAKE, None) == ESHAPE
    assert L.ck_act_rotate_f32(FAKE, 256, 4, 256, 0, 100, FAKE, None) == EUNSUP


def test_binding_rejects_bad_tensors():
    import torch
    with pytest.raises(ValueError, match="GPU"):
        ck.ck_weight_prep(torch.zeros(4, 256))
    with pytest.raises(ValueError):
        ck.ck_act_quant(torch.zeros(4, 256, dtype=torch.float32))


def test_binding_is_not_backed_by_the_oracle():
    """The product package must not reach the CPU oracle."""
    import glob
    for path in glob.glob(os.path.join(ROOT, "swiglu_mlp_amd", "**", "*.py"), recursive=True):
        src = open(path).read()
        assert "import oracle" not in src and "from oracle" not in src, path


def test_w8a16_checks(L):
    """W8A16 entry points: shape, null, alignment and workspace checks on the
    host; nothing here reaches a launch."""
    r = L.ck_act_rotate_bf16
    assert r(FAKE, 256, 0, 256, 0, 128, 1, FAKE, None) == OK                 # m == 0
    assert r(FAKE, 256, 4, 192, 0, 128, 1, FAKE, None) == ESHAPE            # k % group
    assert r(FAKE, 256, 4, 256, 0, 128, 2, FAKE, None) == EINVAL            # no decode layout
    assert r(None, 256, 4, 256, 0, 128, 1, FAKE, None) == EINVAL
    assert r(FAKE, 32768, 70000, 32768, 0, 128, 1, FAKE, None) == EUNSUP    # > 2^31 bytes
    g = L.ck_w8a16_gemm_bf16
    assert g(FAKE, FAKE, FAKE, None, None, 4, 20, 256, FAKE, None) == ESHAPE    # n % 16
    assert g(FAKE, FAKE, FAKE, None, None, 4, 32, 100, FAKE, None) == ESHAPE    # k % 64
    assert g(FAKE, FAKE, None, None, None, 4, 32, 256, FAKE, None) == EINVAL    # scale
    assert g(FAKE, FAKE, FAKE, FAKE + 4, None, 4, 32, 256, FAKE, None) == EINVAL
    assert g(FAKE, FAKE, FAKE, None, FAKE + 2, 4, 32, 256, FAKE, None) == EINVAL
    assert g(FAKE, FAKE, FAKE, None, None, 0, 32, 256, FAKE, None) == OK
    assert L.ck_w8a16_gemm_f32(FAKE, None, 4, 32, 256, FAKE, None) == EINVAL
    assert L.ck_int8_linear_w8a16_workspace_size(3, 256) == 256 * 256 * 2
    lin = L.ck_int8_linear_w8a16
    ws = L.ck_int8_linear_w8a16_workspace_size(8, 256)
    assert lin(FAKE, 256, 0, FAKE, FAKE, None, None, 8, 32, 256, 128, FAKE, FAKE, ws - 1, None) == EWS
    assert lin(FAKE, 256, 0, FAKE, None, None, None, 8, 32, 256, 128, FAKE, FAKE, ws, None) == EINVAL
    assert lin(FAKE, 256, 1, FAKE, FAKE, None, None, 8, 32, 256, 128, FAKE, FAKE, ws, None) == ESHAPE
    mlp = L.ck_swiglu_mlp_w8a16
    ws = L.ck_swiglu_mlp_w8a16_workspace_size(8, 256, 512)
    assert ws >= 256 * 256 * 2 + 8 * 1024 * 2 + 256 * 512 * 2
    assert mlp(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 256, 512, 128, FAKE, FAKE, ws - 256, None) == EWS
    assert mlp(FAKE, FAKE, None, FAKE, FAKE, 8, 256, 512, 128, FAKE, FAKE, ws, None) == EINVAL
    assert mlp(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 256, 500, 128, FAKE, FAKE, ws, None) == ESHAPE


def test_header_compiles_as_c_and_links(tmp_path):
    """include/ck.h is plain C: a C99 program compiled with gcc against it
    links to the library and gets the documented status codes."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "abi_check"
    libdir = os.path.join(ROOT, "swiglu_mlp_amd")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    os.path.join(ROOT, "tests", "abi_check.c"), "-I", os.path.join(ROOT, "include"),
                    "-L", libdir, "-lck_convrot", f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_binding_layout_inference_and_overlap_on_host_tensors():
    """Host-side helpers of the binding (no GPU): the layout is read off the
    weight tensor's form, and output/input overlap is detected by byte range."""
    torch = pytest.importorskip("torch")
    assert ck._weight_layout(None, torch.zeros((8, 2, 1024), dtype=torch.int8)) == ck.CK_LAYOUT_BLOCKED
    assert ck._weight_layout(None, torch.zeros((256, 64), dtype=torch.int8)) == ck.CK_LAYOUT_ROWS
    assert ck._weight_layout(None, torch.zeros((4, 1088), dtype=torch.uint8)) == ck.CK_LAYOUT_DECODE
    assert ck._weight_layout("rows", torch.zeros((8, 2, 1024), dtype=torch.int8)) == ck.CK_LAYOUT_ROWS
    with pytest.raises(ValueError):
        ck._weight_layout("tiled", torch.zeros((8, 2), dtype=torch.int8))
    buf = torch.zeros(64, dtype=torch.bfloat16)
    assert ck._overlaps(buf[:32], buf[16:48])
    assert not ck._overlaps(buf[:32], buf[32:])
    assert ck._overlaps(buf, buf)


def test_noalloc_linear_checks_before_the_gpu(L):
    """The allocation-free linear checks its arguments, and its scratch limit,
    before it touches the device (no GPU needed for these returns)."""
    cap = L.ck_noalloc_scratch_bytes()
    assert cap == 64 << 20
    k = 16384
    m = cap // k + 1
    assert L.ck_int8_linear_workspace_size(m, k, 16) > cap
    args = (FAKE, k, 0, FAKE, FAKE, None, None, 0)
    assert L.ck_int8_linear_noalloc(*args, m, 16, k, 128, FAKE, None) == EWS
    assert L.ck_int8_linear_noalloc(*args, 4, 16, k, 100, FAKE, None) == EUNSUP
    assert L.ck_int8_linear_noalloc(FAKE, k, 0, None, FAKE, None, None, 0, 4, 16, k, 128, FAKE, None) == EINVAL
    assert L.ck_int8_linear_noalloc(*args, 0, 16, k, 128, FAKE, None) == OK


def test_probe_hooks_check_arguments(L):
    """The measurement hooks refuse bad sizes and pointers before launching."""
    assert L.ck_probe_mfma_workgroups() >= 0
    assert L.ck_probe_mfma_i8(FAKE, -1, 0, FAKE, None) == ESHAPE
    assert L.ck_probe_mfma_i8(FAKE, 11, 0, FAKE, None) == ESHAPE
    assert L.ck_probe_mfma_i8(None, 10, 0, FAKE, None) == EINVAL
    assert L.ck_probe_mfma_i8(FAKE + 4, 10, 0, FAKE, None) == EINVAL
    assert L.ck_probe_mfma_i8(FAKE, 0, 1, FAKE, None) == OK
    assert L.ck_probe_stream_rows(FAKE, 64, 4, 60, 16, FAKE, None) == ESHAPE      # read bytes % 16
    assert L.ck_probe_stream_rows(FAKE, 64, 4, 64, 40, FAKE, None) == ESHAPE      # writes more chunks than it reads
    assert L.ck_probe_stream_rows(FAKE, 32, 4, 64, 16, FAKE, None) == ESHAPE      # ld < read bytes
    assert L.ck_probe_stream_rows(FAKE, 1 << 20, 4, 1 << 17, 16, FAKE, None) == ESHAPE
    assert L.ck_probe_stream_rows(None, 64, 4, 64, 16, FAKE, None) == EINVAL
    assert L.ck_probe_stream_rows(FAKE, 64, 0, 64, 16, FAKE, None) == OK
