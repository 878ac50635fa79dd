"""Python binding of ``libmoe.so`` (include/moe.h): the routed, block-quantized MoE expert layer on
AMD Instinct MI355X (gfx950).

This module only marshals arguments: torch tensors supply device memory and the current HIP
stream, ctypes passes plain pointers to the C ABI, and every step of the layer runs in the HIP
kernels of ``csrc/``. There is no fallback: if the library is missing or fails to load, importing
the binding works but every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MoeError", "LayerDesc", "DeviceLayer", "Workspace", "lib", "library_path",
    "moe_route", "moe_permute", "moe_experts_decode", "moe_experts_prefill", "moe_combine", "moe_layer",
    "moe_layer_static", "moe_layer_static_max_bytes",
    "moe_kv_encode", "moe_kv_gather",
    "moe_workspace_size", "moe_status_string", "moe_abi_version",
    "MOE_Q8_B32", "MOE_Q4_B32", "MOE_Q2_B32",
    "MOE_CALL_ROUTE", "MOE_CALL_PERMUTE", "MOE_CALL_EXPERTS_DECODE", "MOE_CALL_EXPERTS_PREFILL",
    "MOE_CALL_COMBINE", "MOE_CALL_LAYER",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_Q8_B32, MOE_Q4_B32, MOE_Q2_B32 = 0, 1, 2
(MOE_CALL_ROUTE, MOE_CALL_PERMUTE, MOE_CALL_EXPERTS_DECODE, MOE_CALL_EXPERTS_PREFILL, MOE_CALL_COMBINE,
 MOE_CALL_LAYER) = range(6)
_BITS = {MOE_Q8_B32: 8, MOE_Q4_B32: 4, MOE_Q2_B32: 2}


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__("%s: %s (status %d)" % (what, moe_status_string(status), status))
        self.status = status


class _QMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("decode_max_tokens", ctypes.c_int32)]


class _Weights(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("gate", _QMat), ("up", _QMat), ("down", _QMat),
                ("sh_gate", _QMat), ("sh_up", _QMat), ("sh_down", _QMat),
                ("prefill_codes", ctypes.c_void_p)]


_lib = None
_lib_error = None


def lib():
    """The loaded C library (raises if it is not built or does not load)."""
    global _lib, _lib_error
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError("libmoe.so is not built (run quantized_expert_ffn_moe_amd/build.py); "
                               "there is no fallback path")
        L = ctypes.CDLL(library_path)
        vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32
        D, W = ctypes.POINTER(_Desc), ctypes.POINTER(_Weights)
        sz = ctypes.c_size_t
        L.moe_route.restype = st
        L.moe_route.argtypes = [D, W, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_permute.restype = st
        L.moe_permute.argtypes = [D, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_experts_decode.restype = st
        L.moe_experts_decode.argtypes = [D, W, vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_kv_encode.restype = st
        L.moe_kv_encode.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_kv_gather.restype = st
        L.moe_kv_gather.argtypes = [vp, vp, i32, i32, vp, i32, vp, vp]
        L.moe_experts_prefill.restype = st
        L.moe_experts_prefill.argtypes = [D, W, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_experts_prefill_f16.restype = st
        L.moe_experts_prefill_f16.argtypes = [D, W, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_combine.restype = st
        L.moe_combine.argtypes = [D, i32, vp, vp, vp, vp, vp, vp]
        L.moe_layer.restype = st
        L.moe_layer.argtypes = [D, W, vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_layer_static.restype = st
        L.moe_layer_static.argtypes = [D, W, vp, i32, vp, vp, vp, vp, vp]
        L.moe_layer_static_max_bytes.restype = sz
        L.moe_layer_static_max_bytes.argtypes = []
        L.moe_workspace_size.restype = st
        L.moe_workspace_size.argtypes = [D, i32, i32, ctypes.POINTER(sz)]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_status_string.argtypes = [st]
        L.moe_abi_version.restype = i32
        L.moe_abi_version.argtypes = []
        L.moe_prefill_codes_bytes.restype = sz
        L.moe_prefill_codes_bytes.argtypes = [D]
        L.moe_pack_prefill_codes.restype = st
        L.moe_pack_prefill_codes.argtypes = [D, W, vp, vp]
        _lib = L
    return _lib


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_abi_version() -> int:
    return int(lib().moe_abi_version())


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError("expected a device tensor, got %s" % t.device)
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _keep(stream, *tensors):
    """Tensors the binding allocated on torch's current stream but handed to work queued on another
    stream: tell the caching allocator so their memory is not reused before that work is done."""
    if stream is None or not isinstance(stream, torch.cuda.Stream) or stream == torch.cuda.current_stream():
        return
    for t in tensors:
        if isinstance(t, torch.Tensor) and t.device.type == "cuda":
            t.record_stream(stream)


class LayerDesc:
    def __init__(self, hidden: int, inter: int, num_experts: int, top_k: int, shared_inter: int, fmt: int,
                 decode_max_tokens: int = 0):
        self.hidden, self.inter, self.num_experts = hidden, inter, num_experts
        self.top_k, self.shared_inter, self.fmt = top_k, shared_inter, fmt
        self.decode_max_tokens = decode_max_tokens
        self.c = _Desc(hidden, inter, num_experts, top_k, shared_inter, fmt, decode_max_tokens)

    @classmethod
    def from_spec(cls, spec, decode_max_tokens: int = 0) -> "LayerDesc":
        return cls(spec.H, spec.I, spec.E, spec.k, spec.Is, spec.fmt, decode_max_tokens)


class DeviceLayer:
    """Device-resident weights of one layer in the canonical layout, plus the C descriptor."""

    def __init__(self, desc: LayerDesc, w_router, router_bias, gate, up, down, sh_gate=None, sh_up=None, sh_down=None):
        self.desc = desc
        self.w_router, self.router_bias = w_router, router_bias
        self.mats = dict(gate=gate, up=up, down=down, sh_gate=sh_gate, sh_up=sh_up, sh_down=sh_down)

        def qm(pair):
            return _QMat(None, None) if pair is None else _QMat(_ptr(pair[0]), _ptr(pair[1]))

        self.c = _Weights(_ptr(w_router), _ptr(router_bias), qm(gate), qm(up), qm(down), qm(sh_gate), qm(sh_up),
                          qm(sh_down), None)
        self.prefill_codes = None

    def pack_prefill_codes(self, stream=None) -> "DeviceLayer":
        """Make the packed copy of the expert codes (moe_pack_prefill_codes) and hand it to every
        later call through the weights (the grouped GEMMs then read it); a one-time cost."""
        n = int(lib().moe_prefill_codes_bytes(ctypes.byref(self.desc.c)))
        if n == 0:
            raise MoeError(MOE_ERR_INVALID_ARG, "moe_prefill_codes_bytes")
        buf = torch.empty(n, dtype=torch.uint8, device=self.mats["gate"][0].device)
        self.c.prefill_codes = None
        _check(lib().moe_pack_prefill_codes(ctypes.byref(self.desc.c), ctypes.byref(self.c), _ptr(buf),
                                            _stream(stream)), "moe_pack_prefill_codes")
        self.prefill_codes = buf
        self.c.prefill_codes = _ptr(buf)
        return self

    def drop_prefill_codes(self) -> "DeviceLayer":
        """Back to the row-major codes only."""
        self.c.prefill_codes = None
        self.prefill_codes = None
        return self

    @classmethod
    def from_host(cls, desc: LayerDesc, d: dict, device="cuda") -> "DeviceLayer":
        """Upload a dict of numpy arrays (w_router, router_bias, gate/up/down/sh_* as (codes, scales))."""
        def up(a, dt):
            if a is None:
                return None
            return torch.from_numpy(a).to(device=device, dtype=dt).contiguous()

        def pair(p):
            if p is None:
                return None
            return (torch.from_numpy(p[0]).to(device), torch.from_numpy(p[1].view("int16")).to(device))

        return cls(desc, up(d["w_router"], torch.float32), up(d.get("router_bias"), torch.float32), pair(d["gate"]),
                   pair(d["up"]), pair(d["down"]), pair(d.get("sh_gate")), pair(d.get("sh_up")), pair(d.get("sh_down")))


class Workspace:
    """A growable device byte buffer handed to the library (the library itself allocates nothing).
    When it grows, the old buffer is released to torch's caching allocator; calls queued on a
    stream other than torch's current one keep the buffer they used alive through record_stream."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self.buf


def moe_workspace_size(desc: LayerDesc, T: int, call: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(desc.c), T, call, ctypes.byref(n)), "moe_workspace_size")
    return int(n.value)


def _ws(layer_desc, T, call, ws):
    need = moe_workspace_size(layer_desc, T, call)
    if ws is None:
        ws = Workspace()
    buf = ws.get(need) if isinstance(ws, Workspace) else ws
    return buf, (0 if buf is None else buf.numel())


def _x_bits(x):
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16)
    if x.dtype in (torch.int16, torch.uint16):
        return x
    raise TypeError("x must be bf16 (or its 16-bit pattern)")


def moe_route(layer: DeviceLayer, x, logits=None, ids=None, p=None, ws=None, stream=None):
    d = layer.desc
    T = x.shape[0]
    dev = x.device
    ids = torch.empty((T, d.top_k), dtype=torch.int32, device=dev) if ids is None else ids
    p = torch.empty((T, d.top_k), dtype=torch.float32, device=dev) if p is None else p
    buf, nb = _ws(d, T, MOE_CALL_ROUTE, ws)
    _check(lib().moe_route(ctypes.byref(d.c), ctypes.byref(layer.c), _ptr(_x_bits(x)), T, _ptr(logits), _ptr(ids),
                           _ptr(p), _ptr(buf), nb, _stream(stream)), "moe_route")
    _keep(stream, buf, ids, p)
    return logits, ids, p


def moe_permute(layer: DeviceLayer, ids, offsets=None, perm=None, inv=None, ws=None, stream=None):
    d = layer.desc
    T = ids.shape[0]
    dev = ids.device
    offsets = torch.empty(d.num_experts + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    perm = torch.empty(T * d.top_k, dtype=torch.int32, device=dev) if perm is None else perm
    inv = torch.empty(T * d.top_k, dtype=torch.int32, device=dev) if inv is None else inv
    buf, nb = _ws(d, T, MOE_CALL_PERMUTE, ws)
    _check(lib().moe_permute(ctypes.byref(d.c), _ptr(ids), T, _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(buf), nb,
                             _stream(stream)), "moe_permute")
    _keep(stream, buf, offsets, perm, inv)
    return offsets, perm, inv


def moe_experts_decode(layer: DeviceLayer, x, ids, y_pairs=None, y_shared=None, ws=None, stream=None):
    d = layer.desc
    T = x.shape[0]
    dev = x.device
    y_pairs = torch.empty((T * d.top_k, d.hidden), dtype=torch.float32, device=dev) if y_pairs is None else y_pairs
    if y_shared is None and d.shared_inter > 0:
        y_shared = torch.empty((T, d.hidden), dtype=torch.float32, device=dev)
    buf, nb = _ws(d, T, MOE_CALL_EXPERTS_DECODE, ws)
    _check(lib().moe_experts_decode(ctypes.byref(d.c), ctypes.byref(layer.c), _ptr(_x_bits(x)), T, _ptr(ids),
                                    _ptr(y_pairs), _ptr(y_shared), _ptr(buf), nb, _stream(stream)),
           "moe_experts_decode")
    _keep(stream, buf, y_pairs, y_shared)
    return y_pairs, y_shared


def moe_experts_prefill(layer: DeviceLayer, x, offsets, perm, y_sorted=None, y_shared=None, ws=None, stream=None,
                        half=False):
    """Grouped-GEMM experts; fp32 rows, or fp16 rows (moe_experts_prefill_f16) when half is true."""
    d = layer.desc
    T = x.shape[0]
    dev = x.device
    dt = torch.float16 if half else torch.float32
    y_sorted = torch.empty((T * d.top_k, d.hidden), dtype=dt, device=dev) if y_sorted is None else y_sorted
    if y_shared is None and d.shared_inter > 0:
        y_shared = torch.empty((T, d.hidden), dtype=dt, device=dev)
    for y in (y_sorted, y_shared):
        if y is not None and y.dtype != dt:
            raise TypeError("moe_experts_prefill: output rows must be %s" % dt)
    buf, nb = _ws(d, T, MOE_CALL_EXPERTS_PREFILL, ws)
    fn = lib().moe_experts_prefill_f16 if half else lib().moe_experts_prefill
    _check(fn(ctypes.byref(d.c), ctypes.byref(layer.c), _ptr(_x_bits(x)), T, _ptr(offsets), _ptr(perm),
              _ptr(y_sorted), _ptr(y_shared), _ptr(buf), nb, _stream(stream)),
           "moe_experts_prefill_f16" if half else "moe_experts_prefill")
    _keep(stream, buf, y_sorted, y_shared)
    return y_sorted, y_shared


def moe_combine(layer_or_desc, p, y_rows, row_of_pair=None, y_shared=None, out=None, stream=None):
    d = layer_or_desc.desc if isinstance(layer_or_desc, DeviceLayer) else layer_or_desc
    T = p.shape[0]
    out = torch.empty((T, d.hidden), dtype=torch.float32, device=p.device) if out is None else out
    _check(lib().moe_combine(ctypes.byref(d.c), T, _ptr(p), _ptr(y_rows), _ptr(row_of_pair), _ptr(y_shared),
                             _ptr(out), _stream(stream)), "moe_combine")
    _keep(stream, out)
    return out


def moe_layer(layer: DeviceLayer, x, out=None, logits=None, ids=None, p=None, ws=None, stream=None):
    d = layer.desc
    T = x.shape[0]
    out = torch.empty((T, d.hidden), dtype=torch.float32, device=x.device) if out is None else out
    buf, nb = _ws(d, T, MOE_CALL_LAYER, ws)
    _check(lib().moe_layer(ctypes.byref(d.c), ctypes.byref(layer.c), _ptr(_x_bits(x)), T, _ptr(out), _ptr(logits),
                           _ptr(ids), _ptr(p), _ptr(buf), nb, _stream(stream)), "moe_layer")
    _keep(stream, buf, out)
    return out


def moe_layer_static(layer: DeviceLayer, x, out=None, logits=None, ids=None, p=None, stream=None):
    """moe_layer with the library's own fixed device workspace (no workspace argument): for callers
    that cannot allocate. Calls that may overlap on one GPU must be ordered by the caller."""
    d = layer.desc
    T = x.shape[0]
    out = torch.empty((T, d.hidden), dtype=torch.float32, device=x.device) if out is None else out
    _check(lib().moe_layer_static(ctypes.byref(d.c), ctypes.byref(layer.c), _ptr(_x_bits(x)), T, _ptr(out),
                                  _ptr(logits), _ptr(ids), _ptr(p), _stream(stream)), "moe_layer_static")
    _keep(stream, out)
    return out


def moe_layer_static_max_bytes() -> int:
    return int(lib().moe_layer_static_max_bytes())


def moe_kv_encode(src, codes=None, scales=None, stream=None):
    """bf16 rows [rows][D] (torch bf16 or int16 bits) -> (int8 codes [rows][D], fp16 scale bits as
    int16 [rows][D/32])."""
    bits = _x_bits(src)
    rows, D = bits.shape
    dev = bits.device
    codes = torch.empty((rows, D), dtype=torch.int8, device=dev) if codes is None else codes
    scales = torch.empty((rows, D // 32), dtype=torch.int16, device=dev) if scales is None else scales
    _check(lib().moe_kv_encode(_ptr(bits), rows, D, _ptr(codes), _ptr(scales), _stream(stream)), "moe_kv_encode")
    _keep(stream, codes, scales)
    return codes, scales


def moe_kv_gather(codes, scales, idx, out=None, stream=None):
    """Dequantised rows idx of the int8 cache as fp32 [n_idx][D] (rows outside the cache are 0)."""
    n_rows, D = codes.shape
    n_idx = idx.numel()
    out = torch.empty((n_idx, D), dtype=torch.float32, device=codes.device) if out is None else out
    _check(lib().moe_kv_gather(_ptr(codes), _ptr(scales), n_rows, D, _ptr(idx), n_idx, _ptr(out), _stream(stream)),
           "moe_kv_gather")
    _keep(stream, out)
    return out
