"""Thin Python binding of libmoe_w8a16.so (argument marshalling only).

Every step of the path runs in the HIP library; this module checks tensor
shapes/dtypes/devices, allocates outputs and workspaces with torch (device
memory plumbing) and passes raw pointers plus torch's current HIP stream.
There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so the library binds to the process's HIP runtime

from .build import LIB_PATH

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EHIP = 0, -1, -2, -3
MOE_STATUS_BAD_EXPERT_ID = 1
MOE_STATUS_NONFINITE_LOGIT = 2
MOE_MAX_EXPERTS = 1024
MOE_MAX_TOPK = 16
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
VARIANTS = {"auto": 0, "decode": 1, "prefill": 2, "prefill_a8": 3, "prefill_a4": 4, "prefill_fp4": 5}
ACTIVATIONS = {"swiglu": 0, "relu2": 1}
LAYOUTS = {"rowmajor": 0, "tiled": 1}

EXPORTED = (
    "moe_last_error", "moe_route", "moe_route_sigmoid", "moe_route_proj_workspace_bytes",
    "moe_route_proj",
    "moe_sort_workspace_bytes", "moe_sort",
    "moe_fused_workspace_bytes", "moe_fused_w8a16", "moe_fused_w8a16_ex",
    "moe_fused_w8a16_noalloc", "moe_fused_mxfp4", "moe_quant_e4m3_rows", "moe_quant_mxfp4_rows",
    "moe_decode_e4m3fn",
    "moe_pack_w8", "moe_pack_mx_scales",
    "moe_profile_enable", "moe_profile_collect", "moe_profile_count", "moe_profile_stat",
)


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


class ExpertW8(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w13_scale", ctypes.c_void_p),
                ("w2", ctypes.c_void_p), ("w2_scale", ctypes.c_void_p)]


_lib = None


def library_path() -> str:
    return LIB_PATH


def load_library():
    """Load (once) and return the ctypes handle; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library {LIB_PATH} is not built; run `python -m block_scaled_fp8_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_route.restype = i32
    lib.moe_route.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp]
    lib.moe_route_sigmoid.restype = i32
    lib.moe_route_sigmoid.argtypes = [vp, i32, i32, i32, i32, ctypes.c_float, vp, vp, vp, vp]
    lib.moe_route_proj_workspace_bytes.restype = sz
    lib.moe_route_proj_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_route_proj.restype = i32
    lib.moe_route_proj.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_sort_workspace_bytes.restype = sz
    lib.moe_sort_workspace_bytes.argtypes = [i32, i32, i32]
    lib.moe_sort.restype = i32
    lib.moe_sort.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_fused_workspace_bytes.restype = sz
    lib.moe_fused_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.moe_fused_w8a16.restype = i32
    lib.moe_fused_w8a16.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                    ctypes.POINTER(ExpertW8), vp, vp, vp, sz, i32, i32, vp]
    lib.moe_fused_w8a16_ex.restype = i32
    lib.moe_fused_w8a16_ex.argtypes = list(lib.moe_fused_w8a16.argtypes[:-1]) + [i32, vp]
    lib.moe_fused_mxfp4.restype = i32
    lib.moe_fused_mxfp4.argtypes = list(lib.moe_fused_w8a16_ex.argtypes)
    lib.moe_fused_w8a16_noalloc.restype = i32
    lib.moe_fused_w8a16_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(ExpertW8), vp, vp, i32, i32, i32, vp]
    lib.moe_pack_mx_scales.restype = i32
    lib.moe_pack_mx_scales.argtypes = [vp, vp, i64, i32, i32, vp]
    lib.moe_pack_w8.restype = i32
    lib.moe_pack_w8.argtypes = [vp, vp, i64, i32, i32, vp]
    lib.moe_quant_e4m3_rows.restype = i32
    lib.moe_quant_e4m3_rows.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.moe_quant_mxfp4_rows.restype = i32
    lib.moe_quant_mxfp4_rows.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.moe_decode_e4m3fn.restype = i32
    lib.moe_decode_e4m3fn.argtypes = [vp, vp, i64, vp]
    lib.moe_profile_enable.restype = i32
    lib.moe_profile_enable.argtypes = [i32]
    lib.moe_profile_collect.restype = i32
    lib.moe_profile_collect.argtypes = []
    lib.moe_profile_count.restype = i32
    lib.moe_profile_count.argtypes = []
    lib.moe_profile_stat.restype = i32
    lib.moe_profile_stat.argtypes = [i32, ctypes.c_char_p, i32, ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_double)]
    _lib = lib
    return lib


def _check(rc: int):
    if rc != MOE_OK:
        msg = load_library().moe_last_error().decode(errors="replace")
        raise MoeError(rc, msg or "moe call failed")


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _need(t: torch.Tensor, name: str, dtype, dev=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def route(logits: torch.Tensor, k: int, status: torch.Tensor | None = None):
    """Softmax top-k routing: logits [T, E] fp32 -> (ids [T, k] int32, aff [T, k] fp32)."""
    lib = load_library()
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    aff = torch.empty((T, k), dtype=torch.float32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, dev)
    _check(lib.moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(aff), _ptr(status), _stream(dev)))
    return ids, aff


def route_sigmoid(logits: torch.Tensor, k: int, normalize: bool = False, scale: float = 1.0,
                  status: torch.Tensor | None = None):
    """Sigmoid top-k routing: logits [T, E] fp32 -> (ids [T, k] int32,
    aff [T, k] fp32 = scale * sigma(l), optionally normalised over the k)."""
    lib = load_library()
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    aff = torch.empty((T, k), dtype=torch.float32, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, dev)
    _check(lib.moe_route_sigmoid(_ptr(logits), T, E, k, int(bool(normalize)), float(scale),
                                 _ptr(ids), _ptr(aff), _ptr(status), _stream(dev)))
    return ids, aff


def route_proj_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(load_library().moe_route_proj_workspace_bytes(T, H, E))


def route_proj(x: torch.Tensor, wg: torch.Tensor, k: int, logits: bool = False,
               status: torch.Tensor | None = None, ws=None, out=None):
    """Router projection then routing: x [T, H] bf16, wg [E, H] bf16 ->
    (ids [T, k] int32, aff [T, k] fp32), plus the fp32 logits [T, E] when
    ``logits`` is true.  ``out`` = (ids, aff) writes into given tensors."""
    lib = load_library()
    _need(x, "x", torch.bfloat16)
    dev = x.device
    _need(wg, "wg", torch.bfloat16, dev)
    T, H = x.shape
    E = wg.shape[0]
    if wg.shape[1] != H:
        raise ValueError(f"wg has shape {tuple(wg.shape)}, expected [E, {H}]")
    if out is not None:
        ids, aff = out
        _need(ids, "ids", torch.int32, dev, (T, k))
        _need(aff, "aff", torch.float32, dev, (T, k))
    else:
        ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        aff = torch.empty((T, k), dtype=torch.float32, device=dev)
    lg = torch.empty((T, E), dtype=torch.float32, device=dev) if logits else None
    if ws is None:
        need = int(lib.moe_route_proj_workspace_bytes(T, H, E))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, dev)
    _check(lib.moe_route_proj(_ptr(x), _ptr(wg), T, H, E, k, _ptr(lg), _ptr(ids), _ptr(aff),
                              _ptr(status), _ptr(ws), ws.numel(), _stream(dev)))
    return (ids, aff, lg) if logits else (ids, aff)


def sort_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(load_library().moe_sort_workspace_bytes(T, k, E))


def sort(ids: torch.Tensor, E: int, status: torch.Tensor | None = None, ws=None):
    """Sort routes by expert: returns (counts, offsets, sorted_route, inv_route)."""
    lib = load_library()
    _need(ids, "ids", torch.int32)
    T, k = ids.shape
    dev = ids.device
    R = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_route = torch.empty(R, dtype=torch.int32, device=dev)
    inv_route = torch.empty(R, dtype=torch.int32, device=dev)
    need = int(lib.moe_sort_workspace_bytes(T, k, E))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if status is not None:
        _need(status, "status", torch.int32, dev)
    _check(lib.moe_sort(_ptr(ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(sorted_route),
                        _ptr(inv_route), _ptr(status), _ptr(ws), ws.numel(), _stream(dev)))
    return counts, offsets, sorted_route, inv_route


def fused_workspace_bytes(T, H, I, E, k, has_shared=False, variant="auto") -> int:
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    return int(load_library().moe_fused_workspace_bytes(T, H, I, E, k, int(bool(has_shared)), v))


def _layout(layout):
    return LAYOUTS[layout] if isinstance(layout, str) else int(layout)


def pack_w8(w: torch.Tensor) -> torch.Tensor:
    """Row-major FP8 weights [..., rows, cols] uint8 -> the tile-coalesced layout
    (same shape and bytes, reordered on the GPU)."""
    lib = load_library()
    _need(w, "w", torch.uint8)
    rows, cols = w.shape[-2], w.shape[-1]
    n = w.numel() // max(1, rows * cols)
    out = torch.empty_like(w)
    _check(lib.moe_pack_w8(_ptr(w), _ptr(out), n, rows, cols, _stream(w.device)))
    return out


def pack_mx_scales(s: torch.Tensor) -> torch.Tensor:
    """MXFP4 E8M0 scales [..., rows, K/32] uint8 -> the tiled layout's order
    (same shape and bytes, reordered on the GPU)."""
    lib = load_library()
    _need(s, "s", torch.uint8)
    rows, cols = s.shape[-2], s.shape[-1]
    n = s.numel() // max(1, rows * cols)
    out = torch.empty_like(s)
    _check(lib.moe_pack_mx_scales(_ptr(s), _ptr(out), n, rows, cols, _stream(s.device)))
    return out


def pack_weights(w: dict, weight_format="e4m3_128") -> dict:
    """A copy of one weight set (w13, w13_scale, w2, w2_scale and an optional
    "shared" dict of the same) in the tiled layout: codes by pack_w8 and,
    for MXFP4, scales by pack_mx_scales."""
    mx = weight_format == "mxfp4"

    def one(d):
        r = dict(d, w13=pack_w8(d["w13"]), w2=pack_w8(d["w2"]))
        if mx:
            r["w13_scale"] = pack_mx_scales(d["w13_scale"])
            r["w2_scale"] = pack_mx_scales(d["w2_scale"])
        return r

    out = one(w)
    if w.get("shared") is not None:
        out["shared"] = one(w["shared"])
    return out


def fused_w8a16(x, w13, w13_scale, w2, w2_scale, ids, aff, shared=None, out=None, ws=None,
                status=None, variant="auto", layout="rowmajor", activation="swiglu",
                weight_format="e4m3_128"):
    """Routed expert FFN with block-scaled weights -> out [T, H] fp32.

    x bf16 [T, H]; ids int32 [T, k]; aff fp32 [T, k]; shared: None or a dict
    with the four tensors of one expert.  weight_format "e4m3_128": w13 uint8
    [E, 2I, H] (activation "relu2": [E, I, H], the up projection alone),
    w13_scale fp32 [E, rows/128, H/128], w2 uint8 [E, H, I], w2_scale fp32
    [E, H/128, I/128].  weight_format "mxfp4" (moe_fused_mxfp4): w13 uint8
    [E, rows, H/2] (two E2M1 codes a byte), w13_scale uint8 E8M0 [E, rows,
    H/32], w2 [E, H, I/2], w2_scale [E, H, I/32]."""
    lib = load_library()
    _need(x, "x", torch.bfloat16)
    dev = x.device
    T, H = x.shape
    _need(w13, "w13", torch.uint8, dev)
    act = ACTIVATIONS[activation] if isinstance(activation, str) else int(activation)
    mx = weight_format == "mxfp4"
    if not mx and weight_format != "e4m3_128":
        raise ValueError(f"unknown weight format {weight_format!r}")
    E, I2, H2 = w13.shape
    I = I2 // 2 if act == 0 else I2
    if (H2 * 2 if mx else H2) != H or (act == 0 and I2 % 2):
        raise ValueError(f"w13 shape {tuple(w13.shape)} does not match x {tuple(x.shape)}")
    if mx:
        _need(w13_scale, "w13_scale", torch.uint8, dev, (E, I2, H // 32))
        _need(w2, "w2", torch.uint8, dev, (E, H, I // 2))
        _need(w2_scale, "w2_scale", torch.uint8, dev, (E, H, I // 32))
    else:
        _need(w13_scale, "w13_scale", torch.float32, dev, (E, -(-I2 // 128), -(-H // 128)))
        _need(w2, "w2", torch.uint8, dev, (E, H, I))
        _need(w2_scale, "w2_scale", torch.float32, dev, (E, -(-H // 128), -(-I // 128)))
    _need(ids, "ids", torch.int32, dev)
    k = ids.shape[1] if ids.dim() == 2 else -1
    if ids.dim() != 2 or ids.shape[0] != T:
        raise ValueError(f"ids must be [T, k] (got {tuple(ids.shape)})")
    _need(aff, "aff", torch.float32, dev, (T, k))
    sh_ptr = None
    if shared is not None:
        sdt = torch.uint8 if mx else torch.float32
        _need(shared["w13"], "shared.w13", torch.uint8, dev, w13.shape[1:])
        _need(shared["w13_scale"], "shared.w13_scale", sdt, dev, w13_scale.shape[1:])
        _need(shared["w2"], "shared.w2", torch.uint8, dev, w2.shape[1:])
        _need(shared["w2_scale"], "shared.w2_scale", sdt, dev, w2_scale.shape[1:])
        sh = ExpertW8(shared["w13"].data_ptr(), shared["w13_scale"].data_ptr(),
                      shared["w2"].data_ptr(), shared["w2_scale"].data_ptr())
        sh_ptr = ctypes.pointer(sh)
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, dev, (T, H))
    if status is not None:
        _need(status, "status", torch.int32, dev)
    head = (_ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), _ptr(ids), _ptr(aff),
            T, H, I, E, k, sh_ptr, _ptr(out), _ptr(status))
    if isinstance(ws, str) and ws == "noalloc":
        # the library's own device scratch array: no workspace argument
        if mx:
            raise ValueError("the no-allocation entry point takes E4M3FN weights")
        _check(lib.moe_fused_w8a16_noalloc(*head, _layout(layout), v, act, _stream(dev)))
        return out
    need = int(lib.moe_fused_workspace_bytes(T, H, I, E, k, int(shared is not None), v))
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    fn = lib.moe_fused_mxfp4 if mx else lib.moe_fused_w8a16_ex
    _check(fn(*head, _ptr(ws), ws.numel(), _layout(layout), v, act, _stream(dev)))
    return out


def fused_w8a16_noalloc(x, w13, w13_scale, w2, w2_scale, ids, aff, out, shared=None,
                        status=None, variant="auto", layout="rowmajor", activation="swiglu"):
    """fused_w8a16 through moe_fused_w8a16_noalloc: the same call with the
    library's device scratch array as its workspace (``out`` is required, so
    that nothing is allocated)."""
    return fused_w8a16(x, w13, w13_scale, w2, w2_scale, ids, aff, shared=shared, out=out,
                       ws="noalloc", status=status, variant=variant, layout=layout,
                       activation=activation)


def quant_e4m3_rows(x: torch.Tensor):
    """Per-token E4M3 quantisation: x [T, H] bf16 -> (codes [T, H] uint8, scales [T] fp32)."""
    lib = load_library()
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    codes = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    scales = torch.empty(T, dtype=torch.float32, device=x.device)
    _check(lib.moe_quant_e4m3_rows(_ptr(x), T, H, _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


def quant_mxfp4_rows(x: torch.Tensor):
    """MXFP4 quantisation of activation rows: x [T, H] bf16 -> (codes [T, H/2]
    uint8, two E2M1 a byte; scales [T, H/32] uint8 E8M0)."""
    lib = load_library()
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    codes = torch.empty((T, H // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((T, H // 32), dtype=torch.uint8, device=x.device)
    _check(lib.moe_quant_mxfp4_rows(_ptr(x), T, H, _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


def decode_e4m3fn(codes: torch.Tensor) -> torch.Tensor:
    """uint8 E4M3FN codes -> bf16 tensor, decoded on the GPU."""
    lib = load_library()
    _need(codes, "codes", torch.uint8)
    out = torch.empty(codes.shape, dtype=torch.bfloat16, device=codes.device)
    _check(lib.moe_decode_e4m3fn(_ptr(codes), _ptr(out), codes.numel(), _stream(codes.device)))
    return out


def forward(x, logits, k, w13, w13_scale, w2, w2_scale, shared=None, variant="auto",
            layout="rowmajor", activation="swiglu"):
    """Whole hot path: route, then the fused sort + expert FFN."""
    ids, aff = route(logits, k)
    out = fused_w8a16(x, w13, w13_scale, w2, w2_scale, ids, aff, shared=shared, variant=variant,
                      layout=layout, activation=activation)
    return ids, aff, out


# ---------------------------------------------------------------- profiling
def profile_enable(on: bool = True):
    _check(load_library().moe_profile_enable(int(bool(on))))


def profile_collect():
    """Wait for recorded kernels; return {kernel: (launches, mean_ms)}."""
    lib = load_library()
    _check(lib.moe_profile_collect())
    out = {}
    name = ctypes.create_string_buffer(128)
    n, ms = ctypes.c_int64(), ctypes.c_double()
    for i in range(lib.moe_profile_count()):
        _check(lib.moe_profile_stat(i, name, 128, ctypes.byref(n), ctypes.byref(ms)))
        out[name.value.decode()] = (int(n.value), ms.value / max(1, n.value))
    return out


class MoeStep:
    """Pre-bound route + fused calls for a fixed set of tensors (no per-call
    checks or allocations): call() enqueues one whole pass on the current
    stream of the tensors' device."""

    def __init__(self, x, logits, k, w13, w13_scale, w2, w2_scale, shared=None,
                 variant="auto", layout="rowmajor", activation="swiglu",
                 weight_format="e4m3_128"):
        lib = load_library()
        dev = x.device
        T, H = x.shape
        E = w13.shape[0]
        act = ACTIVATIONS[activation] if isinstance(activation, str) else int(activation)
        I = w13.shape[1] // 2 if act == 0 else w13.shape[1]
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.aff = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, H), dtype=torch.float32, device=dev)
        # one checked call validates every argument and sizes the workspace
        mx = weight_format == "mxfp4"
        self.ws = torch.empty(max(1, fused_workspace_bytes(T, H, I, E, k, shared is not None,
                                                           variant)),
                              dtype=torch.uint8, device=dev)
        ids, aff = route(logits, k)
        fused_w8a16(x, w13, w13_scale, w2, w2_scale, ids, aff, shared=shared, out=self.out,
                    ws=self.ws, variant=variant, layout=layout, activation=act,
                    weight_format=weight_format)
        self._fused_fn = lib.moe_fused_mxfp4 if mx else lib.moe_fused_w8a16_ex
        self._keep = (x, logits, w13, w13_scale, w2, w2_scale, shared)
        self._sh = None
        if shared is not None:
            self._sh = ctypes.pointer(ExpertW8(shared["w13"].data_ptr(),
                                               shared["w13_scale"].data_ptr(),
                                               shared["w2"].data_ptr(),
                                               shared["w2_scale"].data_ptr()))
        v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
        self._route_args = (_ptr(logits), T, logits.shape[1], k, _ptr(self.ids),
                            _ptr(self.aff), None)
        self._fused_args = (_ptr(x), _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
                            _ptr(self.ids), _ptr(self.aff), T, H, I, E, k, self._sh,
                            _ptr(self.out), None, _ptr(self.ws), self.ws.numel(),
                            _layout(layout), v, act)
        self._lib = lib
        self._dev = dev

    def __call__(self):
        st = _stream(self._dev)
        rc = self._lib.moe_route(*self._route_args, st)
        if rc == MOE_OK:
            rc = self._fused_fn(*self._fused_args, st)
        _check(rc)
        return self.out

    def fused(self):
        """Enqueue only the fused call (sort + expert FFN + expert sum) on the
        ids and affinities of the last routing pass."""
        _check(self._fused_fn(*self._fused_args, _stream(self._dev)))
        return self.out
