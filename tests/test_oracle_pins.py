"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

- hand-computed worked examples (tests/golden/*.json, each with its citation);
- exhaustive checks of the fp16/bf16 readers against numpy's own conversions;
- quantize -> dequantize round-trip bounds (encoder in ``synth``, decoder in the oracle);
- routing and permutation invariants;
- library reductions: numpy stable argsort (top-k and permutation), numpy matmul (router and a
  dense SwiGLU expert from an independent numpy decode of the packed formats), a softmax mixture
  for k = E;
- brute force: every expert evaluated densely and masked by the routing;
- metamorphic relations: relabelling experts, doubling one expert's down scales.

Every check is a ``pin_*`` function so that ``test_oracle_mutants.py`` can run the same checks
against deliberately broken copies of the oracle and show that each plausible mistake is caught.
"""
import glob
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
FMTS = {"Q8": synth.Q8, "Q4": synth.Q4, "Q2": synth.Q2}


# ---------------------------------------------------------------- helpers (test side)

def np_levels(fmt, codes, K):
    """Independent numpy decode of the packed levels (layout stated in synth.c / include/moe.h)."""
    codes = np.asarray(codes, np.uint8)
    lead = codes.shape[:-1]
    if fmt == synth.Q8:
        return codes.view(np.int8).astype(np.float64)
    if fmt == synth.Q4:
        v = np.stack([codes & 15, codes >> 4], -1).reshape(lead + (K,)).astype(np.int64)
        return np.where(v >= 8, v - 16, v).astype(np.float64)
    v = np.stack([(codes >> (2 * m)) & 3 for m in range(4)], -1).reshape(lead + (K,))
    return v.astype(np.float64) - 1.5


def np_dequant(fmt, codes, scales, K):
    s = np.asarray(scales, np.uint16).view(np.float16).astype(np.float64)
    return np_levels(fmt, codes, K) * np.repeat(s, 32, axis=-1)


def bf16_np(bits):
    with np.errstate(invalid="ignore"):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_silu(z):
    return z / (1.0 + np.exp(-z))


def tiny_spec(fmt, H=64, I=64, E=8, k=2, Is=32, T=5, zipf=True):
    return synth.LayerSpec("t", T=T, H=H, E=E, k=k, I=I, Is=Is, fmt=fmt, zipf=zipf, cfg_id=99 + fmt)


def tiny_layer(fmt, seed=1, **kw):
    spec = tiny_spec(fmt, **kw)
    d = synth.make_layer(spec, seed=seed)
    return spec, d, oracle.Layer.from_synth(spec, d)


def pack_spec(fmt, spec, N, K):
    """Codes/scales for one golden matrix spec (fill byte or diagonal level)."""
    bits = synth.FMT_BITS[fmt]
    codes = np.zeros((N, K * bits // 8), np.uint8)
    if "fill" in spec:
        codes[:] = int(spec["fill"], 16)
    else:
        v = int(spec["diag"])
        for n in range(N):
            if fmt == synth.Q8:
                codes[n, n] = v & 0xFF
            elif fmt == synth.Q4:
                codes[n, n // 2] |= (v & 0xF) << (4 * (n % 2))
            else:
                raise ValueError("diag patterns are only used for Q8/Q4 fixtures")
    scales = np.full((N, K // 32), int(spec["scale"], 16), np.uint16)
    return codes, scales


def golden_layer(g):
    fmt, H, I, E, k, Is = FMTS[g["fmt"]], g["H"], g["I"], g["E"], g["k"], g["Is"]
    x = np.zeros((1, H), np.float32)
    for i, v in g["x"].items():
        x[0, int(i)] = v
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)  # exact: the values are small integers
    wr = np.zeros((E, H), np.float32)
    for ij, v in g["w_router"].items():
        e, h = map(int, ij.split(","))
        wr[e, h] = v
    mats = {}
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        cs = [pack_spec(fmt, g["experts"][e][name], N, K) for e in range(E)]
        mats[name] = (np.stack([c for c, _ in cs]), np.stack([s for _, s in cs]))
    sh = {"sh_gate": None, "sh_up": None, "sh_down": None}
    if Is:
        for name, (N, K) in (("gate", (Is, H)), ("up", (Is, H)), ("down", (H, Is))):
            c, s = pack_spec(fmt, g["shared"][name], N, K)
            sh["sh_" + name] = (c[None], s[None])
    L = oracle.Layer(H, I, E, k, fmt, wr, None, mats["gate"], mats["up"], mats["down"], Is, **sh)
    L.host = dict(w_router=wr, router_bias=None, gate=mats["gate"], up=mats["up"], down=mats["down"], **sh)
    return L, xb


GOLDEN_FILES = sorted(f for f in glob.glob(os.path.join(GOLDEN, "*.json")) if not os.path.basename(f).startswith("kv_"))


# ---------------------------------------------------------------- pins

def pin_golden(path):
    g = json.load(open(path))
    L, xb = golden_layer(g)
    out = L.forward(xb)
    np.testing.assert_allclose(out["logits"][0], g["expect_logits"], rtol=0, atol=1e-15)
    assert out["ids"][0].tolist() == g["expect_ids"]
    np.testing.assert_allclose(out["p"][0], g["expect_p"], rtol=1e-15, atol=0)
    want = np.zeros(g["H"])
    if "expect_Y_all" in g:
        want[:] = g["expect_Y_all"]
    else:
        for i, v in g["expect_Y"].items():
            want[int(i)] = v
    np.testing.assert_allclose(out["Y"][0], want, rtol=1e-14, atol=1e-15)


def pin_f16_reader():
    bits = np.arange(65536, dtype=np.uint16)
    mine = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def pin_bf16_reader():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    mine = oracle.bf16_to_f64(bits)
    ref = bf16_np(bits)
    nan = np.isnan(ref)
    assert np.array_equal(mine[~nan], ref[~nan]) and np.isnan(mine[nan]).all()


def pin_levels_exhaustive():
    """Every byte value of every format through the oracle's level reader vs the numpy decode."""
    L = oracle.lib()
    for fmt, per in ((synth.Q8, 1), (synth.Q4, 2), (synth.Q2, 4)):
        row = np.arange(256, dtype=np.uint8)
        want = np_levels(fmt, row[None, :], 256 * per)[0]
        got = np.array([L.orc_code_value(fmt, row.ctypes.data, i) for i in range(256 * per)])
        assert np.array_equal(got, want), synth.FMT_NAMES[fmt]


def pin_roundtrip(fmt):
    """|w - dequant(quant(w))| <= s/2 inside the representable range, else the clamp gap."""
    qmax = {synth.Q8: 127.0, synth.Q4: 7.0, synth.Q2: 1.5}[fmt]
    rng = np.random.default_rng(5 + fmt)
    w = synth.normal_f32(synth.key(7, fmt), 64 * 256, 0.02).reshape(64, 256)
    w[0] = 0.0                                              # all-zero blocks: scale 0
    w[1, :32] = 0.0125                                      # constant block: lands on +qmax
    w[2] = rng.standard_normal(256).astype(np.float32) * np.float32(1e3)   # wide range
    w[3, :32] = np.float32(1e-6) * np.arange(32, dtype=np.float32)          # tiny block
    codes, scales = synth.quantize_rows(fmt, w)
    deq = oracle.dequant(fmt, codes, scales, 64, 256)
    s = np.repeat(oracle.f16_to_f64(scales), 32, axis=1)
    wd = w.astype(np.float64)
    inside = np.abs(wd) <= qmax * s
    err = np.abs(wd - deq)
    assert np.all(err[inside] <= s[inside] / 2 * (1 + 1e-12))
    assert np.all(err[~inside] <= np.abs(wd[~inside]) - qmax * s[~inside] + 1e-300)
    # relative to the block maximum, while the scale is an fp16 normal (rounded by at most 2^-11)
    amax = np.repeat(np.abs(wd).reshape(64, 8, 32).max(-1), 32, axis=1)
    normal = s >= 2.0 ** -14
    assert normal[3].sum() < 256 and normal.sum() > 60 * 256     # the tiny row has subnormal scales
    assert np.all(err[normal] <= amax[normal] / (2 * qmax) * (1 + 2.0 ** -10))
    assert np.all(deq[0] == 0.0)                                  # scale 0 decodes to exact zeros


def pin_routing_invariants():
    rng = np.random.default_rng(11)
    for E, k in ((16, 2), (256, 8), (512, 10), (33, 33)):
        l = rng.standard_normal((64, E)) * 1.4
        ids, p = oracle.topk_softmax(l, k)
        assert np.all(np.abs(p.sum(1) - 1) <= 1e-12)
        assert np.all(np.diff(p, axis=1) <= 0)
        assert np.all((ids >= 0) & (ids < E))
        assert all(len(set(r)) == k for r in ids.tolist())


def pin_topk_stable_sort():
    """Top-k == the first k of a stable sort by descending logit (lower index first on ties)."""
    rng = np.random.default_rng(12)
    l = np.round(rng.standard_normal((200, 40)), 1)          # many exact ties
    l[0, :] = 0.0
    l[1, :] = 0.0
    l[1, ::2] = -0.0                                        # -0 and +0 are one value
    l[2, :] = np.linspace(3, -3, 40)
    for k in (1, 3, 8, 40):
        ids, p = oracle.topk_softmax(l, k)
        want = np.argsort(-l, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, want)
        lk = np.take_along_axis(l, want, 1)
        z = np.exp(lk - lk[:, :1])
        np.testing.assert_allclose(p, z / z.sum(1, keepdims=True), rtol=1e-14)
    assert oracle.topk_softmax(l, 5)[0][1].tolist() == [0, 1, 2, 3, 4]


def pin_permutation():
    rng = np.random.default_rng(13)
    for T, E, k in ((1, 16, 2), (300, 64, 8), (50, 8, 8)):
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        off, perm, inv = oracle.permute(ids, E)
        flat = ids.ravel()
        assert off[0] == 0 and off[E] == T * k
        assert np.array_equal(np.diff(off), np.bincount(flat, minlength=E))
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))
        assert np.array_equal(np.sort(perm), np.arange(T * k))
        assert np.array_equal(inv[perm], np.arange(T * k))
        assert np.all(np.diff(flat[perm]) >= 0)


def pin_router_matmul():
    spec, d, L = tiny_layer(synth.Q8, H=256, E=16)
    x = d["x"]
    want = bf16_np(x) @ d["w_router"].astype(np.float64).T + d["router_bias"].astype(np.float64)
    np.testing.assert_allclose(L.router(x), want, rtol=1e-13, atol=1e-14)


def pin_expert_numpy(fmt):
    spec, d, L = tiny_layer(fmt, H=128, I=96, E=4, Is=64)
    xr = bf16_np(d["x"][0])
    for e in range(spec.E):
        G = np_dequant(fmt, d["gate"][0][e], d["gate"][1][e], spec.H)
        U = np_dequant(fmt, d["up"][0][e], d["up"][1][e], spec.H)
        D = np_dequant(fmt, d["down"][0][e], d["down"][1][e], spec.I)
        want = D @ (np_silu(G @ xr) * (U @ xr))
        np.testing.assert_allclose(L.expert(e, xr), want, rtol=1e-12, atol=1e-13)
    G = np_dequant(fmt, d["sh_gate"][0][0], d["sh_gate"][1][0], spec.H)
    U = np_dequant(fmt, d["sh_up"][0][0], d["sh_up"][1][0], spec.H)
    D = np_dequant(fmt, d["sh_down"][0][0], d["sh_down"][1][0], spec.Is)
    np.testing.assert_allclose(L.shared(xr), D @ (np_silu(G @ xr) * (U @ xr)), rtol=1e-12, atol=1e-13)


def pin_dense_masked(fmt):
    spec, d, L = tiny_layer(fmt, H=96, I=64, E=12, k=3, Is=32, T=6)
    Y = L.forward(d["x"])["Y"]
    Yd = L.dense_masked(d["x"])
    assert np.max(np.abs(Y - Yd)) <= 1e-12 * max(1.0, np.max(np.abs(Yd)))


def pin_full_mixture():
    """k = E: the layer is a softmax mixture of all experts (order of slots irrelevant)."""
    spec, d, L = tiny_layer(synth.Q4, H=64, I=32, E=6, k=6, Is=0, T=3)
    out = L.forward(d["x"])
    for t in range(spec.T):
        l = L.router(d["x"][t:t + 1])[0]
        w = np.exp(l - l.max())
        w /= w.sum()
        ys = np.stack([L.expert(e, bf16_np(d["x"][t])) for e in range(spec.E)])
        np.testing.assert_allclose(out["Y"][t], w @ ys, rtol=1e-12, atol=1e-13)


def pin_k1_single_ffn():
    spec, d, L = tiny_layer(synth.Q2, H=64, I=64, E=5, k=1, Is=32, T=4)
    out = L.forward(d["x"])
    for t in range(spec.T):
        xr = bf16_np(d["x"][t])
        want = L.expert(out["ids"][t][0], xr) + L.shared(xr)
        assert out["p"][t][0] == 1.0
        np.testing.assert_allclose(out["Y"][t], want, rtol=1e-14, atol=1e-15)


def pin_relabel():
    """Relabelling the experts (router rows and expert matrices alike) maps ids and keeps Y."""
    spec, d, L = tiny_layer(synth.Q8, H=64, I=32, E=8, k=3, Is=32, T=4)
    pi = np.random.default_rng(3).permutation(spec.E)       # new label j holds old expert pi[j]
    d2 = dict(d)
    d2["w_router"] = d["w_router"][pi]
    d2["router_bias"] = d["router_bias"][pi]
    for n in ("gate", "up", "down"):
        d2[n] = (d[n][0][pi], d[n][1][pi])
    L2 = oracle.Layer.from_synth(spec, d2)
    a, b = L.forward(d["x"]), L2.forward(d["x"])
    assert np.array_equal(pi[b["ids"]], a["ids"])
    np.testing.assert_allclose(b["Y"], a["Y"], rtol=1e-14, atol=1e-15)


def pin_scale_down():
    """Doubling every down scale of one chosen expert doubles exactly its contribution to Y."""
    spec, d, L = tiny_layer(synth.Q4, H=64, I=32, E=6, k=2, Is=32, T=1)
    a = L.forward(d["x"])
    e = int(a["ids"][0][1])
    d2 = dict(d)
    ds = d["down"][1].copy()
    ds[e] = (ds[e].view(np.float16) * np.float16(2)).view(np.uint16)
    d2["down"] = (d["down"][0], ds)
    b = oracle.Layer.from_synth(spec, d2).forward(d["x"])
    np.testing.assert_allclose(b["Y"][0] - a["Y"][0], a["p"][0][1] * a["y_pairs"][0][1], rtol=1e-12, atol=1e-14)


def pin_logits_override():
    """Routing with externally supplied logits uses exactly those logits."""
    spec, d, L = tiny_layer(synth.Q8, H=64, I=32, E=8, k=2, Is=0, T=2)
    l = np.zeros((2, 8))
    l[0, 5] = l[0, 6] = 1.0
    l[1, 3] = -0.0
    out = L.forward(d["x"], logits_in=l)
    assert out["ids"].tolist() == [[5, 6], [0, 1]]
    np.testing.assert_allclose(out["p"], 0.5, rtol=1e-15)


def pin_combine_alone():
    """The stand-alone combine reproduces the layer's Y from its own parts, in pair order and through a
    row map (rows stored in a shuffled order)."""
    spec, d, L = tiny_layer(synth.Q4, H=64, I=32, E=6, k=3, Is=32, T=4)
    out = L.forward(d["x"])
    yp = out["y_pairs"].reshape(-1, spec.H)
    np.testing.assert_allclose(oracle.combine(out["p"], yp, None, out["y_shared"]), out["Y"], rtol=1e-14, atol=1e-15)
    order = np.random.default_rng(4).permutation(yp.shape[0]).astype(np.int32)   # row r holds pair order[r]
    rows = np.empty_like(order)
    rows[order] = np.arange(len(order), dtype=np.int32)
    got = oracle.combine(out["p"], yp[order], rows, out["y_shared"])
    np.testing.assert_allclose(got, out["Y"], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(oracle.combine(out["p"], yp, None, None), out["Y"] - out["y_shared"], rtol=1e-12,
                               atol=1e-14)


# ------------------------------------------------------------------------- KV int8 block codec

def pin_kv_f16_rounding():
    """The codec's fp32 -> fp16 rounding against numpy's IEEE conversion (round to nearest even):
    random bit patterns over the whole fp32 range, the subnormal range, ties and the overflow edge."""
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    edge = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                     2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -11), 1 + 2 ** -11, 1 + 3 * 2 ** -11, 1 / 127,
                     7.0e-9, 1.0e-7], np.float32)
    small = (rng.standard_normal(5000) * 1e-5).astype(np.float32)
    for v in np.concatenate([vals, edge, small]):
        want = int(np.float32(v).astype(np.float16).view(np.uint16))
        assert oracle.f32_to_f16(float(v)) == want, (float(v), hex(want))


def pin_kv_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "kv_b32_example.json")))
    src = np.array(g["src_bf16"], np.uint16)
    codes, scales = oracle.kv_encode(src)
    assert scales.tolist() == g["expect_scales"]
    assert codes[0, :4].tolist() == g["expect_codes_block0_head"]
    assert np.all(codes[0, 4:] == 0)
    out = oracle.kv_gather(codes, scales, np.array([0]))
    assert out[0, :4].tolist() == g["expect_dequant_block0_head"]
    assert np.all(out[0, 4:] == 0.0)


def _bf16_rows(rng, rows, D, sigma=1.0):
    v = (rng.standard_normal((rows, D)) * sigma).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)   # truncation is fine: any bf16 is a valid input


def pin_kv_round_trip():
    """|v - code * s| <= s / 2 (rounding to the nearest level; no clamping happens because
    s >= m / 127 up to fp16 rounding), codes within [-127, 127], the block maximum maps to +-127
    (or +-126/128 within one fp16 rounding of s)."""
    rng = np.random.default_rng(6)
    for sigma in (1e-3, 1.0, 300.0):
        src = _bf16_rows(rng, 40, 256, sigma)
        codes, scales = oracle.kv_encode(src)
        deq = oracle.kv_gather(codes, scales, np.arange(40))
        v = oracle.bf16_to_f64(src)
        s = np.repeat(oracle.f16_to_f64(scales), 32, axis=1)
        assert np.all(np.abs(codes.astype(int)) <= 127)
        assert np.all(np.abs(v - deq) <= 0.5 * s * (1 + 2.0 ** -20) + 1e-300)
        blockmax = np.abs(codes.astype(int)).reshape(40, -1, 32).max(axis=2)
        assert np.all(blockmax >= 126)


def pin_kv_symmetry():
    """encode(-v) = (-codes, same scale); encode(2^j v) = (same codes, scale * 2^j) away from the
    fp16 subnormal and overflow ranges."""
    rng = np.random.default_rng(7)
    src = _bf16_rows(rng, 16, 128)
    c, s = oracle.kv_encode(src)
    cn, sn = oracle.kv_encode(src ^ np.uint16(0x8000))
    assert np.array_equal(sn, s) and np.array_equal(cn, -c)
    for j in (-3, 4):
        scaled = src.copy()
        e = ((scaled >> 7) & 0xFF).astype(int)
        nz = e != 0
        scaled[nz] = ((scaled[nz].astype(int) & ~(0xFF << 7)) | ((e[nz] + j) << 7)).astype(np.uint16)
        c2, s2 = oracle.kv_encode(scaled)
        assert np.array_equal(c2, c)
        assert np.allclose(oracle.f16_to_f64(s2), oracle.f16_to_f64(s) * 2.0 ** j, rtol=0, atol=0)


def pin_kv_gather():
    rng = np.random.default_rng(8)
    src = _bf16_rows(rng, 50, 96)
    codes, scales = oracle.kv_encode(src)
    full = np.array([[codes[r, d] * oracle.f16_to_f64(np.array([scales[r, d // 32]], np.uint16))[0]
                      for d in range(96)] for r in range(50)])
    idx = np.array([3, 3, 49, 0, -1, 50, 1 << 30, 17])
    out = oracle.kv_gather(codes, scales, idx)
    for j, r in enumerate(idx):
        if 0 <= r < 50:
            assert np.array_equal(out[j], full[r])
        else:
            assert np.all(out[j] == 0.0)


def pin_kv_ties_to_even():
    """s = 2^-7 exactly (m = 127 * 2^-7), so v / s = 2.5, 3.5, 1.5, -2.5 are exact ties: the code
    rounding is to nearest, ties to even (2, 4, 2, -2), not away from zero."""
    vals = np.zeros((1, 32), np.float32)
    vals[0, :5] = [127 * 2.0 ** -7, 2.5 * 2.0 ** -7, 3.5 * 2.0 ** -7, 1.5 * 2.0 ** -7, -2.5 * 2.0 ** -7]
    src = (vals.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_to_f64(src)[0, :5], vals[0, :5].astype(np.float64))
    codes, scales = oracle.kv_encode(src)
    assert oracle.f16_to_f64(scales)[0, 0] == 2.0 ** -7
    assert codes[0, :5].tolist() == [127, 2, 4, 2, -2]


def pin_kv_scale_saturates():
    """A block maximum beyond 127 * 65504 would need an fp16 scale past the range: the scale
    saturates at 65504 (0x7BFF) and the codes clamp at +-127, so no code times the scale is NaN."""
    vals = np.zeros((1, 32), np.float32)
    vals[0, :3] = [1.0e7, -2.0e7, 65504.0 * 3]
    src = (vals.view(np.uint32) >> 16).astype(np.uint16)
    codes, scales = oracle.kv_encode(src)
    assert int(scales[0, 0]) == 0x7BFF
    v = oracle.bf16_to_f64(src)[0, :3]
    assert codes[0, :3].tolist() == [127, -127, 3]
    assert np.all(np.isfinite(oracle.kv_gather(codes, scales, np.array([0]))))
    assert abs(v[2] - 3 * 65504.0) < 0.5 * 65504.0   # the truncated bf16 input still rounds to code 3


def pin_kv_nan_inputs():
    """Reading of the codec for NaN inputs (the pages say nothing of them): a NaN takes no part in
    its block's maximum and gets code 0; a block of NaNs only gets scale 0. Hand-computed block:
    [NaN, 127, -63.5, -NaN, 0 ...] -> max 127, scale fp16(127 / 127) = 1.0 (0x3C00), codes
    [0, 127, -64 (a tie, to even), 0, 0 ...]."""
    vals = np.zeros((2, 32), np.float32)
    vals[0, 1:3] = [127.0, -63.5]
    src = (vals.view(np.uint32) >> 16).astype(np.uint16)
    src[0, 0] = 0x7FC0            # quiet NaN
    src[0, 3] = 0xFFC1            # negative NaN with a payload
    src[1, :] = 0x7F81            # a whole block of NaNs
    codes, scales = oracle.kv_encode(src)
    assert int(scales[0, 0]) == 0x3C00 and int(scales[1, 0]) == 0
    assert codes[0, :4].tolist() == [0, 127, -64, 0]
    assert np.all(codes[0, 4:] == 0) and np.all(codes[1] == 0)


KV_PINS = [("kv_nan_inputs", pin_kv_nan_inputs), ("kv_scale_saturates", pin_kv_scale_saturates), ("kv_f16_rounding", pin_kv_f16_rounding), ("kv_worked_example", pin_kv_worked_example),
           ("kv_round_trip", pin_kv_round_trip), ("kv_symmetry", pin_kv_symmetry), ("kv_gather", pin_kv_gather),
           ("kv_ties_to_even", pin_kv_ties_to_even)]

ALL_PINS = (
    [("golden:" + os.path.basename(f), (lambda f=f: pin_golden(f))) for f in GOLDEN_FILES]
    + [("f16_reader", pin_f16_reader), ("bf16_reader", pin_bf16_reader), ("levels", pin_levels_exhaustive)]
    + [("roundtrip:" + synth.FMT_NAMES[f], (lambda f=f: pin_roundtrip(f))) for f in (synth.Q8, synth.Q4, synth.Q2)]
    + [("routing_invariants", pin_routing_invariants), ("topk_stable_sort", pin_topk_stable_sort),
       ("permutation", pin_permutation), ("router_matmul", pin_router_matmul)]
    + [("expert_numpy:" + synth.FMT_NAMES[f], (lambda f=f: pin_expert_numpy(f))) for f in (synth.Q8, synth.Q4, synth.Q2)]
    + [("dense_masked:" + synth.FMT_NAMES[f], (lambda f=f: pin_dense_masked(f))) for f in (synth.Q8, synth.Q4, synth.Q2)]
    + [("full_mixture", pin_full_mixture), ("k1_single_ffn", pin_k1_single_ffn), ("relabel", pin_relabel),
       ("scale_down", pin_scale_down), ("logits_override", pin_logits_override), ("combine_alone", pin_combine_alone)]
    + KV_PINS
)


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_pin(name, fn):
    fn()


def test_golden_files_present():
    assert len(GOLDEN_FILES) >= 4
    for f in GOLDEN_FILES:
        g = json.load(open(f))
        assert g["citation"] and g["expect_Y_closed_form"]


def test_golden_closed_forms():
    """The stored values are the closed forms they state (guards a typo in the fixtures)."""
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    byname = {os.path.basename(f): json.load(open(f)) for f in GOLDEN_FILES}
    assert byname["w1_q8_top1.json"]["expect_Y"]["0"] == pytest.approx(4 * sig(2), rel=1e-15)
    assert byname["w1_q8_top1.json"]["expect_Y"]["1"] == pytest.approx(sig(1), rel=1e-15)
    assert byname["w1b_q8_tie.json"]["expect_Y"]["1"] == pytest.approx(0.5 * sig(1), rel=1e-15)
    assert byname["w2_q2_top1.json"]["expect_Y_all"] == pytest.approx(-27 * sig(3), rel=1e-15)
    assert byname["w3_q4_k2_shared.json"]["expect_Y"]["0"] == pytest.approx(0.5 * sig(1) + 3.5 * sig(7), rel=1e-15)


