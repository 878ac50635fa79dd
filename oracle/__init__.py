"""Oracle of the routed, block-quantized MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. It wraps ``moe_oracle.c`` (plain single-threaded fp64 C, see its header for the
definitions and the passages they follow) with numpy marshalling and nothing else: every step of
the arithmetic happens in the C file. It shares no code with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ORC_Q8, ORC_Q4, ORC_Q2 = 0, 1, 2
_BITS = {ORC_Q8: 8, ORC_Q4: 4, ORC_Q2: 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: -O2, no fused multiply-add contraction, one thread."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _QMat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("Is", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("w_router", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("gate", _QMat), ("up", _QMat), ("down", _QMat),
                ("sh_gate", _QMat), ("sh_up", _QMat), ("sh_down", _QMat)]


_lib = None


def load(path: str):
    """Open a compiled oracle and declare its signatures."""
    L = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    L.orc_bf16.restype = ctypes.c_double
    L.orc_bf16.argtypes = [ctypes.c_uint16]
    L.orc_f16.restype = ctypes.c_double
    L.orc_f16.argtypes = [ctypes.c_uint16]
    L.orc_code_value.restype = ctypes.c_double
    L.orc_code_value.argtypes = [ctypes.c_int, vp, i32]
    L.orc_dequant.argtypes = [ctypes.c_int, vp, vp, i32, i32, vp]
    L.orc_router.argtypes = [ctypes.POINTER(_Layer), vp, i32, vp]
    L.orc_topk_softmax.restype = ctypes.c_int
    L.orc_topk_softmax.argtypes = [vp, i32, i32, i32, vp, vp]
    L.orc_permute.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    L.orc_expert.argtypes = [ctypes.c_int, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.orc_routed_expert.argtypes = [ctypes.POINTER(_Layer), i32, vp, vp]
    L.orc_shared_expert.argtypes = [ctypes.POINTER(_Layer), vp, vp]
    L.orc_token.restype = ctypes.c_int
    L.orc_token.argtypes = [ctypes.POINTER(_Layer), vp, vp, vp, vp, vp, vp, vp, vp]
    L.orc_layer_forward.restype = ctypes.c_int
    L.orc_layer_forward.argtypes = [ctypes.POINTER(_Layer), vp, i32, vp, vp, vp, vp, vp, vp, vp]
    L.orc_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    L.orc_dense_masked.restype = ctypes.c_int
    L.orc_dense_masked.argtypes = [ctypes.POINTER(_Layer), vp, i32, vp]
    L.orc_f32_to_f16.restype = ctypes.c_uint16
    L.orc_f32_to_f16.argtypes = [ctypes.c_float]
    L.orc_kv_encode.argtypes = [vp, i32, i32, vp, vp]
    L.orc_kv_gather.argtypes = [vp, vp, i32, i32, vp, i32, vp]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = load(_LIB)
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy arrays"
    return a.ctypes.data


class Layer:
    """Holds numpy weights (canonical layout) and the C descriptor that points into them."""

    def __init__(self, H, I, E, k, fmt, w_router, bias, gate, up, down, Is=0, sh_gate=None, sh_up=None,
                 sh_down=None):
        self._keep = []

        def arr(a, dt):
            if a is None:
                return None
            a = np.ascontiguousarray(a, dt)
            self._keep.append(a)
            return a

        def qm(pair):
            if pair is None:
                return _QMat(None, None)
            c, s = arr(pair[0], np.uint8), arr(pair[1], np.uint16)
            return _QMat(_p(c), _p(s))

        self.H, self.I, self.E, self.k, self.Is, self.fmt = H, I, E, k, Is, fmt
        self.c = _Layer(H, I, E, k, Is, fmt, _p(arr(w_router, np.float32)), _p(arr(bias, np.float32)),
                        qm(gate), qm(up), qm(down), qm(sh_gate), qm(sh_up), qm(sh_down))

    @classmethod
    def from_synth(cls, spec, d):
        return cls(spec.H, spec.I, spec.E, spec.k, spec.fmt, d["w_router"], d["router_bias"], d["gate"], d["up"],
                   d["down"], spec.Is, d["sh_gate"], d["sh_up"], d["sh_down"])

    # ---- steps
    def router(self, x_bf16: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x_bf16, np.uint16)
        T = x.shape[0]
        out = np.empty((T, self.E), np.float64)
        lib().orc_router(ctypes.byref(self.c), _p(x), T, _p(out))
        return out

    def expert(self, e: int, x: np.ndarray) -> np.ndarray:
        xd = np.ascontiguousarray(x, np.float64)
        y = np.empty(self.H, np.float64)
        lib().orc_routed_expert(ctypes.byref(self.c), int(e), _p(xd), _p(y))
        return y

    def shared(self, x: np.ndarray) -> np.ndarray:
        xd = np.ascontiguousarray(x, np.float64)
        y = np.empty(self.H, np.float64)
        lib().orc_shared_expert(ctypes.byref(self.c), _p(xd), _p(y))
        return y

    def token(self, x_row: np.ndarray, logits_in: np.ndarray | None = None) -> dict:
        x = np.ascontiguousarray(x_row, np.uint16)
        li = None if logits_in is None else np.ascontiguousarray(logits_in, np.float64)
        out = dict(logits=np.empty(self.E), ids=np.empty(self.k, np.int32), p=np.empty(self.k),
                   y_pairs=np.empty((self.k, self.H)), y_shared=np.empty(self.H), Y=np.empty(self.H))
        rc = lib().orc_token(ctypes.byref(self.c), _p(x), _p(li), _p(out["logits"]), _p(out["ids"]), _p(out["p"]),
                             _p(out["y_pairs"]), _p(out["y_shared"]), _p(out["Y"]))
        if rc != 0:
            raise ValueError("oracle: NaN logits")
        return out

    def forward(self, x_bf16: np.ndarray, logits_in: np.ndarray | None = None) -> dict:
        x = np.ascontiguousarray(x_bf16, np.uint16)
        T = x.shape[0]
        li = None if logits_in is None else np.ascontiguousarray(logits_in, np.float64)
        out = dict(logits=np.empty((T, self.E)), ids=np.empty((T, self.k), np.int32), p=np.empty((T, self.k)),
                   y_pairs=np.empty((T, self.k, self.H)), y_shared=np.empty((T, self.H)), Y=np.empty((T, self.H)))
        rc = lib().orc_layer_forward(ctypes.byref(self.c), _p(x), T, _p(li), _p(out["logits"]), _p(out["ids"]),
                                     _p(out["p"]), _p(out["y_pairs"]), _p(out["y_shared"]), _p(out["Y"]))
        if rc != 0:
            raise ValueError("oracle: NaN logits")
        return out

    def dense_masked(self, x_bf16: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x_bf16, np.uint16)
        Y = np.empty((x.shape[0], self.H))
        lib().orc_dense_masked(ctypes.byref(self.c), _p(x), x.shape[0], _p(Y))
        return Y


def bf16_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, np.uint16).ravel()
    return np.array([lib().orc_bf16(int(v)) for v in b]).reshape(np.shape(bits))


def f16_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, np.uint16).ravel()
    return np.array([lib().orc_f16(int(v)) for v in b]).reshape(np.shape(bits))


def dequant(fmt: int, codes: np.ndarray, scales: np.ndarray, N: int, K: int) -> np.ndarray:
    c = np.ascontiguousarray(codes, np.uint8)
    s = np.ascontiguousarray(scales, np.uint16)
    out = np.empty((N, K), np.float64)
    lib().orc_dequant(fmt, _p(c), _p(s), N, K, _p(out))
    return out


def topk_softmax(logits: np.ndarray, k: int):
    l = np.ascontiguousarray(logits, np.float64)
    T, E = l.shape
    ids = np.empty((T, k), np.int32)
    p = np.empty((T, k), np.float64)
    if lib().orc_topk_softmax(_p(l), T, E, k, _p(ids), _p(p)) != 0:
        raise ValueError("oracle: NaN logits")
    return ids, p


def permute(ids: np.ndarray, E: int):
    i = np.ascontiguousarray(ids, np.int32)
    T, k = i.shape
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(T * k, np.int32)
    inv = np.empty(T * k, np.int32)
    lib().orc_permute(_p(i), T, k, E, _p(offsets), _p(perm), _p(inv))
    return offsets, perm, inv


def combine(p: np.ndarray, y_rows: np.ndarray, row_of_pair=None, y_shared=None) -> np.ndarray:
    """Weighted combine of given expert outputs (fp64): p [T][k], y_rows [rows][H]."""
    pp = np.ascontiguousarray(p, np.float64)
    T, k = pp.shape
    yr = np.ascontiguousarray(y_rows, np.float64)
    H = yr.shape[-1]
    rp = None if row_of_pair is None else np.ascontiguousarray(row_of_pair, np.int32)
    ys = None if y_shared is None else np.ascontiguousarray(y_shared, np.float64)
    out = np.empty((T, H))
    lib().orc_combine(T, k, H, _p(pp), _p(yr), _p(rp), _p(ys), _p(out))
    return out


def expert_ffn(fmt, H, I, gate, up, down, x):
    """One SwiGLU expert from explicit (codes, scales) pairs on one fp64 row; returns (h, y)."""
    g = [np.ascontiguousarray(a) for a in gate]
    u = [np.ascontiguousarray(a) for a in up]
    d = [np.ascontiguousarray(a) for a in down]
    xd = np.ascontiguousarray(x, np.float64)
    h = np.empty(I)
    y = np.empty(H)
    lib().orc_expert(fmt, H, I, _p(g[0]), _p(g[1]), _p(u[0]), _p(u[1]), _p(d[0]), _p(d[1]), _p(xd), _p(h), _p(y))
    return h, y


def f32_to_f16(q: float) -> int:
    """fp32 value -> fp16 bits, round to nearest even (the KV codec's scale rounding)."""
    return int(lib().orc_f32_to_f16(float(q)))


def kv_encode(src_bf16: np.ndarray):
    """bf16 bits [rows][D] -> (int8 codes [rows][D], fp16 scale bits [rows][D/32])."""
    x = np.ascontiguousarray(src_bf16, np.uint16)
    rows, D = x.shape
    assert D % 32 == 0
    codes = np.empty((rows, D), np.int8)
    scales = np.empty((rows, D // 32), np.uint16)
    lib().orc_kv_encode(_p(x), rows, D, _p(codes), _p(scales))
    return codes, scales


def kv_gather(codes: np.ndarray, scales: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Dequantised rows idx of the int8 cache (fp64; rows outside the cache give zeros)."""
    c = np.ascontiguousarray(codes, np.int8)
    s = np.ascontiguousarray(scales, np.uint16)
    i = np.ascontiguousarray(idx, np.int32).ravel()
    out = np.empty((len(i), c.shape[1]), np.float64)
    lib().orc_kv_gather(_p(c), _p(s), c.shape[0], c.shape[1], _p(i), len(i), _p(out))
    return out
