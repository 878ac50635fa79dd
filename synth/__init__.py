"""Seeded synthetic inputs for the routed, block-quantized MoE expert layer.

This module serves both the oracle (tests) and the HIP path (tests, benchmark). It contains none
of the layer's arithmetic: only keyed random draws, the Zipf routing bias, bf16/fp16 rounding and
the data-preparation encoder into block-32 codes (see ``synth.c`` for the exact recipe).

Workloads follow the shapes the pages describe: 256 experts with top-8 for a 35B-A3B model whose
routed experts are 89% of its bytes (648news "cyber-on-strata" article, opening summary and the
section on tiered VRAM/RAM inference), about ten active experts out of 24,576 over 48 layers
(bagrov.by article, section on MoE and hierarchical caching; 648news "nano-cuda-moe" article,
section on CPU/GPU asynchronous compute), 8K-token prompt chunks (648news "nano-cuda-moe"
article, section on speed comparison) and a verify pass of one token plus three MTP drafts (same
article, same section as the 48-layer pass).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, replace

import numpy as np

Q8, Q4, Q2 = 0, 1, 2
FMT_BITS = {Q8: 8, Q4: 4, Q2: 2}
FMT_NAMES = {Q8: "Q8_B32", Q4: "Q4_B32", Q2: "Q2_B32"}

# tensor labels of the keyed streams
T_X, T_WR, T_ZIPF, T_GATE, T_UP, T_DOWN, T_SH_GATE, T_SH_UP, T_SH_DOWN = range(1, 10)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")


def build(force: bool = True) -> str:
    """Compile ``libsynth.so`` with gcc (OpenMP only changes speed, never the bytes)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=gnu11", _SRC,
                               "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        u64, i32, i64, dbl = ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u64, u64, u64, u64]
        L.synth_normal_f32.argtypes = [u64, dbl, i64, vp]
        L.synth_normal_bf16.argtypes = [u64, dbl, i64, vp]
        L.synth_permutation.argtypes = [u64, i32, vp]
        L.synth_zipf_bias.argtypes = [u64, i32, dbl, vp, vp]
        L.synth_quantize_rows.restype = ctypes.c_int
        L.synth_quantize_rows.argtypes = [ctypes.c_int, vp, i64, i32, vp, vp]
        L.synth_expert_stack.restype = ctypes.c_int
        L.synth_expert_stack.argtypes = [ctypes.c_int, u64, i32, i32, i32, dbl, vp, vp, ctypes.c_int]
        L.synth_expert_weights_f32.argtypes = [u64, i32, i32, i32, dbl, vp]
        L.synth_f32_to_bf16.restype = ctypes.c_uint16
        L.synth_f32_to_bf16.argtypes = [ctypes.c_float]
        L.synth_f32_to_f16.restype = ctypes.c_uint16
        L.synth_f32_to_f16.argtypes = [ctypes.c_float]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ---------------------------------------------------------------- primitive draws

def key(seed: int, a: int, b: int = 0, c: int = 0, d: int = 0) -> int:
    return int(lib().synth_key(seed, a, b, c, d))


def normal_f32(k: int, n: int, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(k, sigma, n, _ptr(out))
    return out


def normal_bf16(k: int, n: int, sigma: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().synth_normal_bf16(k, sigma, n, _ptr(out))
    return out


def permutation(k: int, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_permutation(k, n, _ptr(out))
    return out


def zipf_bias(k: int, n: int, alpha: float = 1.1):
    out = np.empty(n, np.float32)
    rank = np.empty(n, np.int32)
    lib().synth_zipf_bias(k, n, alpha, _ptr(out), _ptr(rank))
    return out, rank


def quantize_rows(fmt: int, w: np.ndarray):
    """Encode fp32 rows [R, K] into (codes uint8 [R, K*bits/8], scales uint16 [R, K/32])."""
    w = np.ascontiguousarray(w, np.float32)
    R, K = w.shape
    codes = np.zeros((R, K * FMT_BITS[fmt] // 8), np.uint8)
    scales = np.zeros((R, K // 32), np.uint16)
    rc = lib().synth_quantize_rows(fmt, _ptr(w), R, K, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("bad quantize arguments")
    return codes, scales


def expert_stack(fmt: int, k: int, E: int, N: int, K: int, sigma: float = 0.02, nthreads=None):
    """E experts of [N, K] N(0, sigma^2) weights, encoded. Returns (codes [E,N,Kb], scales [E,N,K/32])."""
    codes = np.empty((E, N, K * FMT_BITS[fmt] // 8), np.uint8)
    scales = np.empty((E, N, K // 32), np.uint16)
    rc = lib().synth_expert_stack(fmt, k, E, N, K, sigma, _ptr(codes), _ptr(scales),
                                  nthreads or default_threads())
    if rc != 0:
        raise ValueError("bad expert stack arguments")
    return codes, scales


def expert_weights_f32(k: int, e: int, N: int, K: int, sigma: float = 0.02) -> np.ndarray:
    out = np.empty((N, K), np.float32)
    lib().synth_expert_weights_f32(k, e, N, K, sigma, _ptr(out))
    return out


# ---------------------------------------------------------------- workloads

@dataclass(frozen=True)
class LayerSpec:
    name: str
    T: int          # tokens in one call
    H: int          # hidden size (K of gate/up, N of down)
    E: int          # routed experts
    k: int          # experts per token
    I: int          # SwiGLU intermediate of a routed expert
    Is: int         # shared-expert intermediate (0 = no shared expert)
    fmt: int        # Q8 / Q4 / Q2
    zipf: bool      # Zipf-biased router logits
    layers: int = 1
    cfg_id: int = 0
    sigma_w: float = 0.02
    sigma_router: float = 0.02
    zipf_alpha: float = 1.1

    def with_(self, **kw) -> "LayerSpec":
        return replace(self, **kw)

    @property
    def bits(self) -> int:
        return FMT_BITS[self.fmt]

    def expert_bytes(self, inter: int | None = None) -> int:
        inter = self.I if inter is None else inter
        return 3 * self.H * inter * self.bits // 8 + (3 * self.H * inter // 32) * 2


CONFIGS = {
    # 4 tokens through a tiny layer: parity in seconds
    "tiny": LayerSpec("tiny", T=4, H=256, E=16, k=2, I=128, Is=0, fmt=Q8, zipf=False, cfg_id=1),
    # one decode token, 256 experts top-8 + shared, 4-bit experts
    "decode1": LayerSpec("decode1", T=1, H=2048, E=256, k=8, I=512, Is=512, fmt=Q4, zipf=True, cfg_id=2),
    # verify pass: 1 token + 3 drafts, 8-bit experts
    "verify4": LayerSpec("verify4", T=4, H=2048, E=256, k=8, I=512, Is=512, fmt=Q8, zipf=True, cfg_id=3),
    # 48 independent layers of 512 experts top-10, 2-bit experts, one token
    "stack48": LayerSpec("stack48", T=1, H=2048, E=512, k=10, I=768, Is=0, fmt=Q2, zipf=True, layers=48,
                         cfg_id=4),
    # an 8K-token prefill chunk, 4-bit experts + shared
    "prefill8k": LayerSpec("prefill8k", T=8192, H=2048, E=256, k=8, I=512, Is=512, fmt=Q4, zipf=True,
                           cfg_id=5),
}


def make_x(spec: LayerSpec, layer: int = 0, seed: int = 0, T: int | None = None, sigma: float = 1.0) -> np.ndarray:
    """bf16 activations [T][H], N(0, sigma^2) (sigma = 1 for every named workload)."""
    T = spec.T if T is None else T
    return normal_bf16(key(seed, spec.cfg_id, layer, T_X), T * spec.H, sigma).reshape(T, spec.H)


def make_router(spec: LayerSpec, layer: int = 0, seed: int = 0):
    w_r = normal_f32(key(seed, spec.cfg_id, layer, T_WR), spec.E * spec.H, spec.sigma_router)
    w_r = w_r.reshape(spec.E, spec.H)
    bias = None
    if spec.zipf:
        bias, _ = zipf_bias(key(seed, spec.cfg_id, layer, T_ZIPF), spec.E, spec.zipf_alpha)
    return w_r, bias


def make_weights(spec: LayerSpec, layer: int = 0, seed: int = 0, nthreads=None) -> dict:
    """All weights of one layer as numpy arrays in the canonical layout."""
    w_r, bias = make_router(spec, layer, seed)
    out = {"w_router": w_r, "router_bias": bias}
    H, I, E = spec.H, spec.I, spec.E
    for name, t, n, kk, ee in (("gate", T_GATE, I, H, E), ("up", T_UP, I, H, E), ("down", T_DOWN, H, I, E)):
        out[name] = expert_stack(spec.fmt, key(seed, spec.cfg_id, layer, t), ee, n, kk, spec.sigma_w, nthreads)
    if spec.Is > 0:
        Is = spec.Is
        for name, t, n, kk in (("sh_gate", T_SH_GATE, Is, H), ("sh_up", T_SH_UP, Is, H), ("sh_down", T_SH_DOWN, H, Is)):
            out[name] = expert_stack(spec.fmt, key(seed, spec.cfg_id, layer, t), 1, n, kk, spec.sigma_w, nthreads)
    else:
        for name in ("sh_gate", "sh_up", "sh_down"):
            out[name] = None
    return out


def make_layer(spec: LayerSpec, layer: int = 0, seed: int = 0, nthreads=None, T: int | None = None) -> dict:
    d = make_weights(spec, layer, seed, nthreads)
    d["x"] = make_x(spec, layer, seed, T)
    return d
