"""Host-side checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

from block_scaled_fp8_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w8a16.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(moe_[a-z0-9_]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("moe_route", "moe_route_sigmoid", "moe_route_proj", "moe_sort", "moe_fused_w8a16", "moe_last_error",
              "moe_sort_workspace_bytes", "moe_fused_workspace_bytes", "moe_fused_w8a16_ex",
              "moe_decode_e4m3fn",
              "moe_pack_w8"):
        assert n in names
    assert set(names) == set(binding.EXPORTED)


def test_library_loads_and_exports_every_symbol():
    lib = binding.load_library()
    for n in _declared_functions():
        assert hasattr(lib, n), n
    assert lib.moe_last_error() == b""


def _null():
    return ctypes.c_void_p(0)


def test_route_argument_checks():
    lib = binding.load_library()
    fake = ctypes.c_void_p(0x1000)
    # k > E, k > MAX_K, E > MAX_E, T < 0 are rejected without a launch
    assert lib.moe_route(fake, 4, 8, 9, fake, fake, None, None) == binding.MOE_EINVAL
    assert b"k must be" in lib.moe_last_error()
    assert lib.moe_route(fake, 4, 64, 17, fake, fake, None, None) == binding.MOE_EINVAL
    assert lib.moe_route(fake, 4, 2000, 2, fake, fake, None, None) == binding.MOE_EINVAL
    assert lib.moe_route(fake, -1, 8, 2, fake, fake, None, None) == binding.MOE_EINVAL
    assert lib.moe_route(fake, 4, 8, 0, fake, fake, None, None) == binding.MOE_EINVAL
    # NULL outputs
    assert lib.moe_route(fake, 4, 8, 2, None, fake, None, None) == binding.MOE_EINVAL
    # T == 0 is a no-op that never touches the device
    assert lib.moe_route(None, 0, 8, 2, None, None, None, None) == binding.MOE_OK
    assert lib.moe_last_error() == b""


def test_route_sigmoid_argument_checks():
    lib = binding.load_library()
    f = ctypes.c_void_p(0x1000)
    assert lib.moe_route_sigmoid(f, 4, 8, 9, 0, 1.0, f, f, None, None) == binding.MOE_EINVAL
    assert lib.moe_route_sigmoid(f, 4, 8, 2, 2, 1.0, f, f, None, None) == binding.MOE_EINVAL
    assert b"normalize" in lib.moe_last_error()
    assert lib.moe_route_sigmoid(f, 4, 8, 2, 0, float("inf"), f, f, None, None) == binding.MOE_EINVAL
    assert lib.moe_route_sigmoid(f, 4, 8, 2, 1, float("nan"), f, f, None, None) == binding.MOE_EINVAL
    assert b"scale" in lib.moe_last_error()
    assert lib.moe_route_sigmoid(f, 4, 8, 2, 0, 1.0, None, f, None, None) == binding.MOE_EINVAL
    assert lib.moe_route_sigmoid(None, 0, 8, 2, 0, 1.0, None, None, None, None) == binding.MOE_OK
    assert lib.moe_last_error() == b""


def test_route_proj_argument_checks():
    lib = binding.load_library()
    f = ctypes.c_void_p(0x1000)
    T, H, E, k = 64, 2048, 256, 8
    need = lib.moe_route_proj_workspace_bytes(T, H, E)
    # decode shape: four 64x64 tiles, so K is split into 8 slices of partial logits
    assert need == 8 * T * E * 4
    # a prefill shape fills the chip without a split: one [T, E] slab
    assert lib.moe_route_proj_workspace_bytes(8192, 2048, 256) == 8192 * 256 * 4
    assert lib.moe_route_proj_workspace_bytes(8, 100, 4) == 0      # H % 64 != 0
    call = lambda T=T, H=H, E=E, k=k, x=f, wg=f, lg=f, ids=f, aff=f, ws=f, wsb=need: (  # noqa: E731
        lib.moe_route_proj(x, wg, T, H, E, k, lg, ids, aff, None, ws, wsb, None))
    assert call(H=96) == binding.MOE_EUNSUPPORTED
    assert b"multiple of 64" in lib.moe_last_error()
    assert call(k=E + 1, E=8) == binding.MOE_EINVAL
    assert call(E=2000) == binding.MOE_EINVAL
    assert call(x=None) == binding.MOE_EINVAL
    assert call(aff=None) == binding.MOE_EINVAL
    assert call(x=ctypes.c_void_p(0x1008)) == binding.MOE_EINVAL
    assert b"aligned" in lib.moe_last_error()
    assert call(wsb=need - 1) == binding.MOE_EINVAL
    assert b"workspace" in lib.moe_last_error()
    assert call(lg=None, ws=None, wsb=0) == binding.MOE_EINVAL
    # T == 0 is a no-op that never touches the device
    assert call(T=0, x=None, wg=None, lg=None, ids=None, aff=None, ws=None, wsb=0) == binding.MOE_OK
    assert lib.moe_last_error() == b""


def test_sort_argument_checks():
    lib = binding.load_library()
    fake = ctypes.c_void_p(0x1000)
    assert lib.moe_sort(fake, 4, 3, 2, fake, fake, fake, fake, None, None, 0, None) == binding.MOE_EINVAL
    assert lib.moe_sort(fake, 4, 2, 8, None, fake, fake, fake, None, None, 0, None) == binding.MOE_EINVAL
    # the large-R path needs scratch: too small a workspace is rejected
    T, k, E = 8192, 8, 256
    need = lib.moe_sort_workspace_bytes(T, k, E)
    assert need >= E * 4
    assert lib.moe_sort(fake, T, k, E, fake, fake, fake, fake, None, fake, need - 1, None) == binding.MOE_EINVAL
    assert b"workspace" in lib.moe_last_error()
    assert lib.moe_sort_workspace_bytes(64, 8, 256) == 0   # single-workgroup path needs none


def test_fused_activation_checks():
    lib = binding.load_library()
    f = ctypes.c_void_p(0x1000)
    o = ctypes.c_void_p(0x3000)
    ws = lib.moe_fused_workspace_bytes(64, 2048, 512, 256, 8, 0, 0)
    base = (f, f, f, f, f, f, f, 64, 2048, 512, 256, 8, None, o, None, f, ws, 0)
    assert lib.moe_fused_w8a16_ex(*base, 0, 2, None) == binding.MOE_EINVAL
    assert b"activation" in lib.moe_last_error()
    # prefill down tiles take 256 output columns: relu^2 with H = 384 is
    # rejected before any launch
    ws384 = lib.moe_fused_workspace_bytes(8192, 384, 512, 256, 8, 0, 2)
    args = (f, f, f, f, f, f, f, 8192, 384, 512, 256, 8, None, o, None, f, ws384, 0, 2)
    assert lib.moe_fused_w8a16_ex(*args, 1, None) == binding.MOE_EUNSUPPORTED
    assert b"H % 256" in lib.moe_last_error()


def test_quant_mxfp4_rows_argument_checks():
    lib = binding.load_library()
    f = ctypes.c_void_p(0x1000)
    assert lib.moe_quant_mxfp4_rows(f, 4, 48, f, f, None) == binding.MOE_EINVAL     # H % 32
    assert b"multiple of 32" in lib.moe_last_error()
    assert lib.moe_quant_mxfp4_rows(ctypes.c_void_p(0x1008), 4, 64, f, f, None) == binding.MOE_EINVAL
    assert lib.moe_quant_mxfp4_rows(f, 4, 64, ctypes.c_void_p(0x1008), f, None) == binding.MOE_EINVAL
    assert b"aligned" in lib.moe_last_error()
    assert lib.moe_quant_mxfp4_rows(f, 4, 64, f, None, None) == binding.MOE_EINVAL
    assert lib.moe_quant_mxfp4_rows(None, 0, 64, None, None, None) == binding.MOE_OK


def test_mxfp4_activation_variant_needs_mxfp4_weights():
    """MOE_VARIANT_PREFILL_A4 and MOE_VARIANT_PREFILL_FP4 are refused for
    E4M3FN weights (both entry points) before any launch; 6 is no variant."""
    lib = binding.load_library()
    f, o = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x3000)
    ws = lib.moe_fused_workspace_bytes(64, 2048, 512, 256, 8, 0, 4)
    assert ws > lib.moe_fused_workspace_bytes(64, 2048, 512, 256, 8, 0, 2)   # + codes and scales of x
    # the MXFP4 hidden activation lives inside the bf16 hidden buffer
    assert lib.moe_fused_workspace_bytes(64, 2048, 512, 256, 8, 0, 5) == ws
    assert lib.moe_fused_workspace_bytes(64, 2048, 512, 256, 8, 0, 6) == 0
    head = (f, f, f, f, f, f, f, 64, 2048, 512, 256, 8, None, o, None)
    for v in (4, 5):
        assert lib.moe_fused_w8a16_ex(*head, f, ws, 0, v, 0, None) == binding.MOE_EUNSUPPORTED
        assert b"MXFP4 weights" in lib.moe_last_error()
        assert lib.moe_fused_w8a16_noalloc(*head, 0, v, 0, None) == binding.MOE_EUNSUPPORTED
    assert lib.moe_fused_w8a16_ex(*head, f, ws, 0, 6, 0, None) == binding.MOE_EINVAL


def test_quant_e4m3_rows_argument_checks():
    lib = binding.load_library()
    f = ctypes.c_void_p(0x1000)
    assert lib.moe_quant_e4m3_rows(f, 4, 12, f, f, None) == binding.MOE_EINVAL
    assert lib.moe_quant_e4m3_rows(ctypes.c_void_p(0x1008), 4, 16, f, f, None) == binding.MOE_EINVAL
    assert b"aligned" in lib.moe_last_error()
    assert lib.moe_quant_e4m3_rows(f, 4, 16, None, f, None) == binding.MOE_EINVAL
    assert lib.moe_quant_e4m3_rows(None, 0, 16, None, None, None) == binding.MOE_OK
    # the fp8-activation variant's workspace also holds the codes and scales
    a8 = lib.moe_fused_workspace_bytes(8192, 2048, 512, 256, 8, 0, 3)
    pf = lib.moe_fused_workspace_bytes(8192, 2048, 512, 256, 8, 0, 2)
    assert a8 >= pf + 8192 * 2048 + 8192 * 4


def test_fused_argument_checks():
    lib = binding.load_library()
    f = ctypes.c_void_p(0x1000)
    o = ctypes.c_void_p(0x3000)
    ws = lib.moe_fused_workspace_bytes(64, 2048, 512, 256, 8, 0, 0)
    assert ws > 64 * 8 * (512 * 2 + 2048 * 4)
    args = lambda T, H, I, E, k, ws_bytes, variant=0, out=o, layout=0: (  # noqa: E731
        f, f, f, f, f, f, f, T, H, I, E, k, None, out, None, f, ws_bytes, layout, variant, None)
    assert lib.moe_fused_w8a16(*args(64, 2000, 512, 256, 8, ws)) == binding.MOE_EUNSUPPORTED
    assert lib.moe_fused_w8a16(*args(64, 2048, 500, 256, 8, ws)) == binding.MOE_EUNSUPPORTED
    assert b"multiples of 128" in lib.moe_last_error()
    assert lib.moe_fused_w8a16(*args(64, 2048, 512, 256, 8, ws - 1)) == binding.MOE_EINVAL
    assert b"workspace" in lib.moe_last_error()
    assert lib.moe_fused_w8a16(*args(64, 2048, 512, 256, 8, ws, 7)) == binding.MOE_EINVAL
    assert lib.moe_fused_w8a16(*args(64, 2048, 512, 256, 8, ws, 0, o, 5)) == binding.MOE_EINVAL
    assert b"layout" in lib.moe_last_error()
    assert lib.moe_fused_w8a16(*args(64, 2048, 512, 256, 300, ws)) == binding.MOE_EINVAL
    # out aliasing x
    assert lib.moe_fused_w8a16(*args(64, 2048, 512, 256, 8, ws, 0, f)) == binding.MOE_EINVAL
    assert b"alias" in lib.moe_last_error()
    # shared descriptor with a NULL member
    bad = binding.ExpertW8(0x1000, 0, 0x1000, 0x1000)
    a = list(args(64, 2048, 512, 256, 8, ws + 10**9))
    a[12] = ctypes.pointer(bad)
    a[13] = ctypes.c_void_p(0x2000)
    lib.moe_fused_w8a16.argtypes[12] = ctypes.POINTER(binding.ExpertW8)
    assert lib.moe_fused_w8a16(*a) == binding.MOE_EINVAL
    assert b"shared" in lib.moe_last_error()
    # the prefill variant needs H and 2I in multiples of 256: refused before any launch
    ws384 = lib.moe_fused_workspace_bytes(64, 384, 128, 256, 8, 0, 2)
    assert lib.moe_fused_w8a16(*args(64, 384, 128, 256, 8, ws384, 2)) == binding.MOE_EUNSUPPORTED
    assert b"prefill variant needs" in lib.moe_last_error()
    # T == 0 is a no-op
    assert lib.moe_fused_w8a16(*args(0, 2048, 512, 256, 8, 0)) == binding.MOE_OK


def test_fused_alignment_checks():
    """16-byte vector accesses on x, the weights, out and the workspace and
    4-byte ones on the scales, ids and affinities: misaligned pointers are
    refused before any launch."""
    lib = binding.load_library()
    f = 0x1000
    ws = lib.moe_fused_workspace_bytes(64, 2048, 512, 256, 8, 0, 0)

    def call(**over):
        p = dict(x=f, w13=f, w13s=f, w2=f, w2s=f, ids=f, aff=f, out=0x3000, ws=0x5000)
        p.update(over)
        v = lambda a: ctypes.c_void_p(a)  # noqa: E731
        return lib.moe_fused_w8a16(v(p["x"]), v(p["w13"]), v(p["w13s"]), v(p["w2"]), v(p["w2s"]),
                                   v(p["ids"]), v(p["aff"]), 64, 2048, 512, 256, 8, None,
                                   v(p["out"]), None, v(p["ws"]), ws, 0, 0, None)

    for name, addr in (("x", 0x1008), ("w13", 0x1004), ("w2", 0x1001), ("out", 0x3008),
                       ("ws", 0x5004), ("w13s", 0x1002), ("w2s", 0x1001), ("ids", 0x1002),
                       ("aff", 0x1003)):
        assert call(**{name: addr}) == binding.MOE_EINVAL, name
        assert b"aligned" in lib.moe_last_error(), name


def test_workspace_is_sized_per_variant():
    """Decode rows of contributions are fp32 (4 bytes a value), prefill rows
    block floating point (2 bytes a value + an exponent byte per 8); AUTO is
    sized for either."""
    lib = binding.load_library()
    T, H, I, E, k = 16384, 8192, 256, 512, 10
    rows = T * k + T + 1
    dec = lib.moe_fused_workspace_bytes(T, H, I, E, k, 1, 1)
    pf = lib.moe_fused_workspace_bytes(T, H, I, E, k, 1, 2)
    auto = lib.moe_fused_workspace_bytes(T, H, I, E, k, 1, 0)
    assert dec >= rows * 4 * H and pf >= rows * (2 * H + H // 8)
    assert pf < rows * 4 * H < dec and auto == dec
    assert lib.moe_fused_workspace_bytes(T, H, I, E, k, 1, 9) == 0


def test_workspace_grows_with_shared_expert():
    lib = binding.load_library()
    a = lib.moe_fused_workspace_bytes(512, 2048, 512, 256, 8, 0, 0)
    b = lib.moe_fused_workspace_bytes(512, 2048, 512, 256, 8, 1, 0)
    assert b > a


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        binding.route(torch.zeros((4, 8), dtype=torch.float32), 2)


def test_pack_mx_scales_argument_checks():
    lib = binding.load_library()
    f = ctypes.c_void_p(0x1000)
    g = ctypes.c_void_p(0x1000 + 8 * 256 * 64)
    assert lib.moe_pack_mx_scales(f, g, 8, 250, 64, None) == binding.MOE_EINVAL   # rows % 16
    assert lib.moe_pack_mx_scales(f, g, 8, 256, 6, None) == binding.MOE_EINVAL    # cols % 4
    assert lib.moe_pack_mx_scales(f, ctypes.c_void_p(0x1040), 8, 256, 64, None) == binding.MOE_EINVAL
    assert b"overlap" in lib.moe_last_error()
    assert lib.moe_pack_mx_scales(None, None, 0, 256, 64, None) == binding.MOE_OK


def test_mxfp4_argument_checks():
    """moe_fused_mxfp4 refuses an explicit prefill variant (bf16 or fp8
    activations) on E8M0 scale arrays that are not 4-byte aligned, and
    unknown arguments, before any launch."""
    lib = binding.load_library()
    f, o = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x3000)
    ws = lib.moe_fused_workspace_bytes(64, 2048, 512, 256, 8, 0, 0)
    args = lambda variant, act=0, s13=f, ws_ptr=f: (  # noqa: E731
        f, f, s13, f, f, f, f, 64, 2048, 512, 256, 8, None, o, None, ws_ptr, ws, 0, variant, act, None)
    for v in (2, 3):
        assert lib.moe_fused_mxfp4(*args(v, 0, ctypes.c_void_p(0x1001))) == binding.MOE_EINVAL
        assert b"aligned MXFP4 scale" in lib.moe_last_error()
    assert lib.moe_fused_mxfp4(*args(1, 2)) == binding.MOE_EINVAL
    assert b"activation" in lib.moe_last_error()
    assert lib.moe_fused_mxfp4(*args(1, 0, f, ctypes.c_void_p(0x1004))) == binding.MOE_EINVAL
    assert b"aligned" in lib.moe_last_error()


def test_pack_argument_checks():
    lib = binding.load_library()
    f = ctypes.c_void_p(0x1000)
    g = ctypes.c_void_p(0x1000 + 8 * 256 * 512)
    assert lib.moe_pack_w8(f, g, 8, 250, 512, None) == binding.MOE_EINVAL   # rows % 16
    assert lib.moe_pack_w8(f, g, 8, 256, 100, None) == binding.MOE_EINVAL   # cols % 64
    assert lib.moe_pack_w8(f, ctypes.c_void_p(0x1000 + 64), 8, 256, 512, None) == binding.MOE_EINVAL
    assert b"overlap" in lib.moe_last_error()
    assert lib.moe_pack_w8(None, None, 0, 256, 512, None) == binding.MOE_OK
