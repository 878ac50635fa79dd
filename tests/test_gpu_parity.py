"""GPU parity: every C-ABI entry point against the fp64 oracle on the same seeded inputs.

Matching rules: top-k ids and the permutation bit-exact given identical router logits (the GPU's
fp32 logits, widened to fp64, are handed to the oracle's top-k); every float tensor within relative
L2 <= 2e-3 and max-abs <= 1e-2 * rms(oracle output). Large workloads compare sampled outputs the
oracle computes one token at a time.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_float_match, float_errors, host_layer

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("quantized_expert_ffn_moe_amd")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


def dev_layer(spec, d, dmt=0):
    return moe.DeviceLayer.from_host(moe.LayerDesc.from_spec(spec, decode_max_tokens=dmt), d)


def dev_x(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def orc_layer(spec, d):
    return oracle.Layer.from_synth(spec, d)


def run_layer(spec, d, x=None, dmt=0):
    """moe_layer on the GPU; returns numpy logits, ids, p, Y. dmt: decode_max_tokens of the descriptor
    (0 = the library's default; 1 sends every batch of two or more tokens to the grouped GEMMs)."""
    x = d["x"] if x is None else x
    T = x.shape[0]
    L = dev_layer(spec, d, dmt)
    xd = dev_x(x)
    logits = torch.empty((T, spec.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda")
    p = torch.empty((T, spec.k), dtype=torch.float32, device="cuda")
    Y = moe.moe_layer(L, xd, logits=logits, ids=ids, p=p)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), ids.cpu().numpy(), p.cpu().numpy(), Y.cpu().numpy()


def check_routing(O, x_rows, g_logits, g_ids, g_p, token_rows=None):
    """Oracle logits (float rule), ids bit-exact and p (float rule) from the GPU's logits."""
    rows = np.arange(g_logits.shape[0]) if token_rows is None else np.asarray(token_rows)
    o_logits = O.router(x_rows[rows])
    assert_float_match(g_logits[rows], o_logits, "logits")
    ids, p = oracle.topk_softmax(g_logits.astype(np.float64), g_ids.shape[1])
    assert np.array_equal(g_ids, ids), "top-k ids differ from the oracle's top-k of the same logits"
    assert_float_match(g_p, p, "p")
    # near-ties: tokens whose chosen set differs under the oracle's own logits (reported, allowed)
    own_ids, _ = oracle.topk_softmax(o_logits, g_ids.shape[1])
    flips = sum(set(a.tolist()) != set(b.tolist()) for a, b in zip(own_ids, ids[rows]))
    return flips


def oracle_tokens(O, x, g_logits, rows):
    """Oracle Y (and parts) for the given token rows, routed with the GPU's logits."""
    outs = [O.token(x[t], logits_in=g_logits[t].astype(np.float64)) for t in rows]
    return {k: np.stack([o[k] for o in outs]) for k in outs[0]}


# ------------------------------------------------------------------------- small / decode configs

@pytest.mark.parametrize("name", ["tiny", "decode1", "verify4"])
def test_layer_decode_configs(name):
    _need_gpu()
    spec, d = host_layer(name)
    say("layer", name, "T=%d E=%d k=%d fmt=%s" % (spec.T, spec.E, spec.k, synth.FMT_NAMES[spec.fmt]))
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    flips = check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(spec.T))
    rel, mx = assert_float_match(Y, ref["Y"], "Y")
    say(name, "Y rel %.2e maxabs/rms %.2e near-tie flips %d" % (rel, mx, flips))


@pytest.mark.parametrize("name", ["tiny", "decode1", "verify4"])
def test_experts_decode_pairs(name):
    """moe_route + moe_experts_decode + moe_combine as separate calls, each checked."""
    _need_gpu()
    spec, d = host_layer(name)
    say("experts_decode", name)
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    logits = torch.empty((spec.T, spec.E), dtype=torch.float32, device="cuda")
    _, ids, p = moe.moe_route(L, xd, logits=logits)
    y_pairs, y_shared = moe.moe_experts_decode(L, xd, ids)
    Y = moe.moe_combine(L, p, y_pairs, None, y_shared)
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy()
    check_routing(O, d["x"], g_logits, ids.cpu().numpy(), p.cpu().numpy())
    ref = oracle_tokens(O, d["x"], g_logits, range(spec.T))
    assert_float_match(y_pairs.cpu().numpy().reshape(spec.T, spec.k, spec.H), ref["y_pairs"], "y_pairs")
    if spec.Is:
        assert_float_match(y_shared.cpu().numpy(), ref["y_shared"], "y_shared")
    assert_float_match(Y.cpu().numpy(), ref["Y"], "Y")
    comb = oracle.combine(p.cpu().numpy(), y_pairs.cpu().numpy(), None, None if not spec.Is else y_shared.cpu().numpy())
    assert_float_match(Y.cpu().numpy(), comb, "combine alone")


@pytest.mark.parametrize("fmt", [synth.Q8, synth.Q4, synth.Q2])
@pytest.mark.parametrize("T", [1, 2])
def test_decode_ragged_row_groups(fmt, T):
    """The one- and two-token gate/up kernel (four rows per wave, 16 lanes per row, four 32-blocks
    per lane and step) at a hidden size of 65 blocks (the second step of every row holds one
    block), an intermediate size of 3 blocks (the down kernel steps a lane's items with a
    remainder and sums per-pair partials one at a time) and a shared expert of 2 blocks:
    moe_layer and moe_experts_decode against the oracle."""
    _need_gpu()
    spec = synth.LayerSpec("rg", T=T, H=2080, E=40, k=3, I=96, Is=64, fmt=fmt, zipf=True, cfg_id=240 + 4 * fmt + T)
    d = synth.make_layer(spec)
    say("ragged row groups", synth.FMT_NAMES[fmt], "T=%d" % T)
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    logits = torch.empty((T, spec.E), dtype=torch.float32, device="cuda")
    ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda")
    p = torch.empty((T, spec.k), dtype=torch.float32, device="cuda")
    Y = moe.moe_layer(L, xd, logits=logits, ids=ids, p=p)
    y_pairs, y_shared = moe.moe_experts_decode(L, xd, ids)
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy()
    check_routing(O, d["x"], g_logits, ids.cpu().numpy(), p.cpu().numpy())
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    assert_float_match(Y.cpu().numpy(), ref["Y"], "Y")
    assert_float_match(y_pairs.cpu().numpy().reshape(T, spec.k, spec.H), ref["y_pairs"], "y_pairs")
    assert_float_match(y_shared.cpu().numpy(), ref["y_shared"], "y_shared")


@pytest.mark.parametrize("T", [5, 6, 7])
def test_layer_default_switch(T):
    """moe_layer with the library's default regime switch on both sides of it (decode kernels up to
    6 tokens, grouped GEMMs from 7): the same oracle rule either way."""
    _need_gpu()
    spec = synth.LayerSpec("sw", T=T, H=512, E=64, k=8, I=128, Is=64, fmt=synth.Q4, zipf=True, cfg_id=260 + T)
    d = synth.make_layer(spec)
    say("default switch T=%d" % T)
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    assert_float_match(Y, ref["Y"], "Y")


@pytest.mark.parametrize("layer", [0, 47])
def test_stack48_layer(layer):
    """One layer of the 48-layer, 512-expert, top-10, 2-bit stack at full size."""
    _need_gpu()
    spec, d = host_layer("stack48", layer)
    say("stack48 layer", layer)
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(spec.T))
    assert_float_match(Y, ref["Y"], "Y")


def test_decode_eight_tokens_full_plan():
    """Eight tokens with top-8 on the decode1 shape: all 64 pairs of the routing plan, through
    moe_layer (decode kernels) and moe_experts_decode."""
    _need_gpu()
    spec = synth.CONFIGS["decode1"].with_(name="dec8", T=8, cfg_id=99)
    d = synth.make_layer(spec)
    say("decode T=8 k=8 (64 pairs)")
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d, dmt=8)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(spec.T))
    assert_float_match(Y, ref["Y"], "Y")
    L = dev_layer(spec, d)
    y_pairs, y_sh = moe.moe_experts_decode(L, dev_x(d["x"]), torch.from_numpy(g_ids).cuda())
    torch.cuda.synchronize()
    assert_float_match(y_pairs.cpu().numpy().reshape(8, spec.k, spec.H), ref["y_pairs"], "y_pairs")
    assert_float_match(y_sh.cpu().numpy(), ref["y_shared"], "y_shared")


def test_layer_decode_lds_fallback():
    """T = 4, k = 8, I = 1536: the 36 pairs' activations (221 KB) exceed the decode kernels' LDS, so
    moe_layer takes the grouped-GEMM path; it still meets the rule against the oracle, and
    moe_experts_decode refuses the shape before enqueueing anything."""
    _need_gpu()
    spec = synth.LayerSpec("ldsfb", T=4, H=1024, E=64, k=8, I=1536, Is=0, fmt=synth.Q4, zipf=True, cfg_id=97)
    d = synth.make_layer(spec)
    say("decode LDS fallback T=4 k=8 I=1536")
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(spec.T))
    assert_float_match(Y, ref["Y"], "Y")
    L = dev_layer(spec, d)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_experts_decode(L, dev_x(d["x"]), torch.from_numpy(g_ids).cuda())
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED


def test_experts_decode_stack48_four_tokens():
    """moe_experts_decode on a full-size stack48 layer (512 experts, top-10, 2-bit) with 4 tokens:
    the per-pair partial sums are reduced in chunks of slots to fit the LDS."""
    _need_gpu()
    spec, d = host_layer("stack48", 0)
    x = synth.make_x(spec, layer=0, seed=5, T=4)
    say("stack48 moe_experts_decode T=4")
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    xd = dev_x(x)
    logits = torch.empty((4, spec.E), dtype=torch.float32, device="cuda")
    _, ids, p = moe.moe_route(L, xd, logits=logits)
    y_pairs, _ = moe.moe_experts_decode(L, xd, ids)
    Y = moe.moe_layer(L, xd)
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy()
    check_routing(O, x, g_logits, ids.cpu().numpy(), p.cpu().numpy())
    ref = oracle_tokens(O, x, g_logits, range(4))
    assert_float_match(y_pairs.cpu().numpy().reshape(4, spec.k, spec.H), ref["y_pairs"], "y_pairs")
    assert_float_match(Y.cpu().numpy(), ref["Y"], "Y")


def test_experts_decode_chunked_odd_blocks():
    """moe_experts_decode where the per-pair partial sums do not fit the LDS at once and the block
    counts are odd (I = 352: 11 blocks per slot, Is = 96: 3 blocks): 64 pairs of 4 tokens reduced
    in chunks of slots, the partials read one at a time."""
    _need_gpu()
    T = 4
    spec = synth.LayerSpec("chunk", T=T, H=256, E=64, k=16, I=352, Is=96, fmt=synth.Q8, zipf=True, cfg_id=270)
    d = synth.make_layer(spec)
    say("chunked odd blocks T=4 k=16 I=352 Is=96")
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    logits = torch.empty((T, spec.E), dtype=torch.float32, device="cuda")
    _, ids, p = moe.moe_route(L, xd, logits=logits)
    y_pairs, y_shared = moe.moe_experts_decode(L, xd, ids)
    torch.cuda.synchronize()
    g_logits = logits.cpu().numpy()
    check_routing(O, d["x"], g_logits, ids.cpu().numpy(), p.cpu().numpy())
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    assert_float_match(y_pairs.cpu().numpy().reshape(T, spec.k, spec.H), ref["y_pairs"], "y_pairs")
    assert_float_match(y_shared.cpu().numpy(), ref["y_shared"], "y_shared")


def test_golden_examples_on_gpu():
    """The hand-computed worked examples through moe_layer (T = 1, decode path)."""
    _need_gpu()
    import test_oracle_pins as pins
    for path in pins.GOLDEN_FILES:
        g = json.load(open(path))
        OL, xb = pins.golden_layer(g)
        fmt, H, I, E, k, Is = pins.FMTS[g["fmt"]], g["H"], g["I"], g["E"], g["k"], g["Is"]
        spec = synth.LayerSpec("golden", T=1, H=H, E=E, k=k, I=I, Is=Is, fmt=fmt, zipf=False)
        d = OL.host
        _, ids, p, Y = run_layer(spec, d, xb)
        assert ids[0].tolist() == g["expect_ids"], path
        want = np.zeros(H)
        if "expect_Y_all" in g:
            want[:] = g["expect_Y_all"]
        else:
            for i, v in g["expect_Y"].items():
                want[int(i)] = v
        np.testing.assert_allclose(Y[0], want, rtol=1e-5, atol=1e-6, err_msg=path)


# ------------------------------------------------------------------------- router accuracy

@pytest.mark.parametrize("T,E", [(3, 256), (8, 256), (16, 256), (17, 256), (300, 200), (1000, 512), (1500, 256)])
def test_router_fp32_error_bound(T, E):
    """Router logits (GEMV for T <= 16, bf16x3 MFMA GEMM above) stay within the worst-case fp32
    summation bound of the oracle's fp64 logits: |err| <= 3H * 2^-24 * sum_h |x_h w_h| + 2^-24 |b|
    (3H additions: three bf16 terms per weight on the matrix-core path)."""
    _need_gpu()
    spec = synth.LayerSpec("rt", T=T, H=2048, E=E, k=8, I=32, Is=0, fmt=synth.Q8, zipf=True, cfg_id=60)
    d = synth.make_layer(spec)
    say("router bound T=%d E=%d" % (T, E))
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.moe_route(L, dev_x(d["x"]), logits=logits)
    torch.cuda.synchronize()
    g = logits.cpu().numpy().astype(np.float64)
    o = O.router(d["x"])
    xf = oracle.bf16_to_f64(d["x"])
    w = d["w_router"].astype(np.float64)
    b = d["router_bias"].astype(np.float64) if d["router_bias"] is not None else np.zeros(E)
    bound = 3 * spec.H * 2.0 ** -24 * (np.abs(xf) @ np.abs(w).T) + 2.0 ** -24 * np.abs(b)[None, :]
    err = np.abs(g - o)
    assert np.all(err <= bound), "max err/bound %.3f" % float(np.max(err / bound))


@pytest.mark.parametrize("T,H,mbits", [(3, 96, 17), (7, 96, 17), (300, 96, 17), (40, 256, 16), (600, 96, 17),
                                       (1100, 96, 17)])
def test_router_exact_on_representable_sums(T, H, mbits):
    """Inputs whose every partial sum is exact in fp32: x in {-1, 0, 1}, w = m * 2^-mbits with m in
    [2^(mbits-1), 2^mbits), H * 2^mbits <= 2^24 (17 bits at H = 96: all three bf16 terms of the
    split are needed; H = 256 with 16 bits runs the K-split GEMM with its partial-sum reduction;
    T = 600 spans ten token tiles, T = 1100 nine of the 128-token tiles large batches use).
    Any fp32 evaluation order gives the exact value, so the logits must equal the oracle's bit for
    bit."""
    _need_gpu()
    E = 200
    spec = synth.LayerSpec("rx", T=T, H=H, E=E, k=4, I=32, Is=0, fmt=synth.Q8, zipf=False, cfg_id=61)
    d = synth.make_layer(spec)
    rng = np.random.default_rng(7)
    xv = rng.integers(-1, 2, size=(T, H)).astype(np.float32)
    d["x"] = (xv.view(np.uint32) >> 16).astype(np.uint16)
    m = rng.integers(1 << (mbits - 1), 1 << mbits, size=(E, H)) * rng.choice([-1, 1], size=(E, H))
    d["w_router"] = (m * 2.0 ** -mbits).astype(np.float32)
    d["router_bias"] = (rng.integers(-64, 64, size=E) * 2.0 ** -6).astype(np.float32)
    say("router exact T=%d H=%d" % (T, H))
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    moe.moe_route(L, dev_x(d["x"]), logits=logits)
    torch.cuda.synchronize()
    assert np.array_equal(logits.cpu().numpy().astype(np.float64), O.router(d["x"]))


# ------------------------------------------------------------------------- prefill

def small_prefill_spec(fmt, T, E=16, k=4, Is=64, H=256, I=128, zipf=True):
    return synth.LayerSpec("pf", T=T, H=H, E=E, k=k, I=I, Is=Is, fmt=fmt, zipf=zipf, cfg_id=40 + fmt)


@pytest.mark.parametrize("fmt", [synth.Q8, synth.Q4, synth.Q2])
@pytest.mark.parametrize("T", [5, 130, 300])
def test_layer_prefill_small(fmt, T):
    """Prefill path at sizes the oracle finishes in seconds: several row tiles and ragged tails (the
    grouped GEMMs forced at every T through decode_max_tokens = 1)."""
    _need_gpu()
    spec = small_prefill_spec(fmt, T)
    d = synth.make_layer(spec)
    say("prefill small", synth.FMT_NAMES[fmt], "T=%d" % T)
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d, dmt=1)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    assert_float_match(Y, ref["Y"], "Y")


@pytest.mark.parametrize("fmt,T,E,k", [(synth.Q8, 2, 16, 4), (synth.Q4, 7, 100, 8), (synth.Q2, 16, 256, 8),
                                       (synth.Q4, 16, 500, 10), (synth.Q8, 13, 1000, 16), (synth.Q4, 17, 256, 8)])
def test_layer_small_batch_front_end(fmt, T, E, k):
    """Batches of 2 to 16 tokens on the grouped-GEMM path take their logits from the router GEMV and
    run the top-k, permutation, tile list and x conversion as one kernel (one block routes while the
    others convert x), over every keys-per-lane width of the top-k (E = 16 ... 1000); T = 17 takes
    the router GEMM and the separate kernels. ids bit-exact, logits, p and Y against the oracle."""
    _need_gpu()
    spec = small_prefill_spec(fmt, T, E=E, k=k, Is=64 if T % 2 else 0, H=512, I=96)
    d = synth.make_layer(spec)
    say("small-batch front end", synth.FMT_NAMES[fmt], "T=%d E=%d k=%d" % (T, E, k))
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d, dmt=1)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    assert_float_match(Y, ref["Y"], "Y")


@pytest.mark.parametrize("fmt", [synth.Q8, synth.Q4, synth.Q2])
def test_layer_prefill_ragged_shapes(fmt):
    """H, I, Is that leave partial weight-row tiles (H = 800 = 3 * 256 + 32, I = 160, Is = 96)."""
    _need_gpu()
    T = 200
    spec = small_prefill_spec(fmt, T, E=16, k=4, Is=96, H=800, I=160)
    d = synth.make_layer(spec)
    say("prefill ragged", synth.FMT_NAMES[fmt], "T=%d H=800 I=160 Is=96" % T)
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    assert_float_match(Y, ref["Y"], "Y")


@pytest.mark.parametrize("T,k,Is", [(1, 2, 4096), (5, 1, 0)])
def test_layer_max_shapes(T, k, Is):
    """The largest hidden and intermediate sizes the library accepts (H = 16384, I = Is = 4096, int8
    codes): the decode kernels (T = 1, with the shared expert) and the grouped GEMMs (T = 5), whose
    32-bit lane offsets and 64 MB weight matrices sit at their limits."""
    _need_gpu()
    spec = synth.LayerSpec("max", T=T, H=16384, E=2, k=k, I=4096, Is=Is, fmt=synth.Q8, zipf=False,
                           cfg_id=95)
    d = synth.make_layer(spec)
    say("max shapes", "T=%d k=%d Is=%d" % (T, k, Is))
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d, dmt=1)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    assert_float_match(Y, ref["Y"], "Y")


@pytest.mark.parametrize("T", [1, 4, 65])
def test_experts_prefill_entry(T):
    """moe_permute + moe_experts_prefill as separate calls: permutation bit-exact, y_sorted rows."""
    _need_gpu()
    spec = small_prefill_spec(synth.Q4, T, E=16, k=3, Is=128, I=64)
    d = synth.make_layer(spec)
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    logits = torch.empty((T, spec.E), dtype=torch.float32, device="cuda")
    _, ids, p = moe.moe_route(L, xd, logits=logits)
    offsets, perm, inv = moe.moe_permute(L, ids)
    y_sorted, y_shared = moe.moe_experts_prefill(L, xd, offsets, perm)
    Y = moe.moe_combine(L, p, y_sorted, inv, y_shared)
    torch.cuda.synchronize()
    g_ids = ids.cpu().numpy()
    o_off, o_perm, o_inv = oracle.permute(g_ids, spec.E)
    assert np.array_equal(offsets.cpu().numpy(), o_off)
    assert np.array_equal(perm.cpu().numpy(), o_perm)
    assert np.array_equal(inv.cpu().numpy(), o_inv)
    g_logits = logits.cpu().numpy()
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    ys = y_sorted.cpu().numpy()
    want_sorted = ref["y_pairs"].reshape(T * spec.k, spec.H)[o_perm]
    assert_float_match(ys, want_sorted, "y_sorted")
    assert_float_match(y_shared.cpu().numpy(), ref["y_shared"], "y_shared")
    assert_float_match(Y.cpu().numpy(), ref["Y"], "Y")


def test_experts_prefill_hot_experts():
    """Every token routed to experts 0 and 1 (ids given): each of the two groups holds 700 rows,
    five full 128-row tiles and a 60-row remainder, more than the four tiles per expert that the
    tile list's first pass writes, so its second pass places the rest. Every y_sorted row against
    the oracle's expert outputs for that routing."""
    _need_gpu()
    T = 700
    spec = small_prefill_spec(synth.Q4, T, E=8, k=2, Is=64, I=64)
    d = synth.make_layer(spec)
    say("prefill hot experts T=%d" % T)
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    g_ids = np.tile(np.array([[0, 1]], dtype=np.int32), (T, 1))
    offsets, perm, inv = moe.moe_permute(L, torch.from_numpy(g_ids).cuda())
    y_sorted, y_shared = moe.moe_experts_prefill(L, xd, offsets, perm)
    torch.cuda.synchronize()
    o_off, o_perm, o_inv = oracle.permute(g_ids, spec.E)
    assert np.array_equal(offsets.cpu().numpy(), o_off)
    assert np.array_equal(perm.cpu().numpy(), o_perm)
    # logits that make the oracle choose experts 0 then 1 for every token
    lg = np.full((T, spec.E), -10.0)
    lg[:, 0], lg[:, 1] = 10.0, 9.0
    ref = oracle_tokens(O, d["x"], lg, range(T))
    assert np.array_equal(ref["ids"], g_ids)
    want_sorted = ref["y_pairs"].reshape(T * spec.k, spec.H)[o_perm]
    assert_float_match(y_sorted.cpu().numpy(), want_sorted, "y_sorted")
    assert_float_match(y_shared.cpu().numpy(), ref["y_shared"], "y_shared")


@pytest.mark.parametrize("fmt,T,H,I,Is,E,k", [(synth.Q8, 200, 800, 160, 96, 16, 4),
                                              (synth.Q4, 300, 256, 128, 64, 16, 4),
                                              (synth.Q2, 130, 800, 160, 0, 16, 4),
                                              (synth.Q4, 700, 512, 96, 64, 8, 2),
                                              (synth.Q8, 260, 512, 256, 256, 16, 4),
                                              (synth.Q2, 200, 256, 256, 0, 8, 2)])
def test_packed_prefill_codes_bitwise(fmt, T, H, I, Is, E, k):
    """The grouped GEMMs reading the packed copy of the codes (moe_pack_prefill_codes) give the same
    bits as reading the row-major codes (same operands, same MFMA order): y_sorted / y_shared of
    moe_experts_prefill and the output of moe_layer. H = 800 and I = 160 leave a half-empty last K
    step in every matrix; where K is a multiple of 256 (H = 256 or 512, I or Is = 256) the GEMMs
    also read the packed scales. The row-major path is checked against the oracle elsewhere; Y of the
    packed path is also checked against it here."""
    _need_gpu()
    spec = synth.LayerSpec("pk", T=T, H=H, E=E, k=k, I=I, Is=Is, fmt=fmt, zipf=True, cfg_id=130 + fmt)
    d = synth.make_layer(spec)
    say("packed codes", synth.FMT_NAMES[fmt], "T=%d H=%d I=%d Is=%d" % (T, H, I, Is))
    L = dev_layer(spec, d, dmt=1)
    xd = dev_x(d["x"])
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    _, ids, p = moe.moe_route(L, xd, logits=logits)
    offsets, perm, inv = moe.moe_permute(L, ids)
    ys0, ysh0 = moe.moe_experts_prefill(L, xd, offsets, perm)
    Y0 = moe.moe_layer(L, xd)
    L.pack_prefill_codes()
    ys1, ysh1 = moe.moe_experts_prefill(L, xd, offsets, perm)
    Y1 = moe.moe_layer(L, xd)
    torch.cuda.synchronize()
    assert torch.equal(ys0, ys1)
    if Is:
        assert torch.equal(ysh0, ysh1)
    assert torch.equal(Y0, Y1)
    O = orc_layer(spec, d)
    rows = list(range(0, T, max(1, T // 16)))
    ref = oracle_tokens(O, d["x"], logits.cpu().numpy(), rows)
    assert_float_match(Y1.cpu().numpy()[rows], ref["Y"], "Y (packed)")


def test_packed_prefill_codes_prefill8k_bitwise():
    """The 8192-token chunk the benchmark times: moe_layer with the packed codes gives the same
    bits as with the row-major codes."""
    _need_gpu()
    spec, d = host_layer("prefill8k")
    say("packed codes: prefill8k")
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    Y0 = moe.moe_layer(L, xd)
    L.pack_prefill_codes()
    Y1 = moe.moe_layer(L, xd)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1)


@pytest.mark.parametrize("fmt,T,H,I,Is", [(synth.Q4, 300, 256, 128, 64), (synth.Q8, 200, 800, 160, 96),
                                           (synth.Q2, 130, 800, 160, 0)])
def test_experts_prefill_f16_entry(fmt, T, H, I, Is):
    """moe_experts_prefill_f16: every fp16 row is the fp32 entry's row rounded to nearest even (same
    accumulators), and the rows meet the float rule against the oracle."""
    _need_gpu()
    spec = small_prefill_spec(fmt, T, E=16, k=4, Is=Is, H=H, I=I)
    d = synth.make_layer(spec)
    say("experts_prefill_f16", synth.FMT_NAMES[fmt], "T=%d H=%d I=%d Is=%d" % (T, H, I, Is))
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    logits = torch.empty((T, spec.E), dtype=torch.float32, device="cuda")
    _, ids, p = moe.moe_route(L, xd, logits=logits)
    offsets, perm, inv = moe.moe_permute(L, ids)
    y32, ysh32 = moe.moe_experts_prefill(L, xd, offsets, perm)
    y16, ysh16 = moe.moe_experts_prefill(L, xd, offsets, perm, half=True)
    torch.cuda.synchronize()
    assert y16.dtype == torch.float16
    assert torch.equal(y16.view(torch.int16), y32.to(torch.float16).view(torch.int16))
    if Is > 0:
        assert torch.equal(ysh16.view(torch.int16), ysh32.to(torch.float16).view(torch.int16))
    o_off, o_perm, o_inv = oracle.permute(ids.cpu().numpy(), spec.E)
    ref = oracle_tokens(O, d["x"], logits.cpu().numpy(), range(T))
    want_sorted = ref["y_pairs"].reshape(T * spec.k, spec.H)[o_perm]
    assert_float_match(y16.float().cpu().numpy(), want_sorted, "y_sorted f16")
    if Is > 0:
        assert_float_match(ysh16.float().cpu().numpy(), ref["y_shared"], "y_shared f16")


def test_decode_and_prefill_agree():
    """The same 4 tokens through the decode entry and the prefill entry both meet the rule."""
    _need_gpu()
    spec = small_prefill_spec(synth.Q8, 4, E=16, k=2, Is=64)
    d = synth.make_layer(spec)
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    logits = torch.empty((4, spec.E), dtype=torch.float32, device="cuda")
    _, ids, p = moe.moe_route(L, xd, logits=logits)
    yp, ysh = moe.moe_experts_decode(L, xd, ids)
    Yd = moe.moe_combine(L, p, yp, None, ysh)
    offsets, perm, inv = moe.moe_permute(L, ids)
    ys, ysh2 = moe.moe_experts_prefill(L, xd, offsets, perm)
    Yp = moe.moe_combine(L, p, ys, inv, ysh2)
    torch.cuda.synchronize()
    ref = oracle_tokens(O, d["x"], logits.cpu().numpy(), range(4))
    assert_float_match(Yd.cpu().numpy(), ref["Y"], "decode Y")
    assert_float_match(Yp.cpu().numpy(), ref["Y"], "prefill Y")


def _pool_map(fn, items):
    """The oracle is single-threaded C called through ctypes (which releases the GIL) and keeps no
    state between calls, so independent calls run side by side on the host's cores."""
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        return list(ex.map(fn, items))


def host_tiles(counts, T, has_shared, tm=128):
    """The grouped GEMM's row tiles, by the kernel's rule: per group, full tiles of 128 rows and one
    remainder tile; the shared group (all T tokens) last. Returns (group, first row, rows)."""
    tiles = []
    for e, n in enumerate(counts):
        for r0 in range(0, int(n), tm):
            tiles.append((e, r0, min(tm, int(n) - r0)))
    if has_shared:
        for r0 in range(0, T, tm):
            tiles.append((len(counts), r0, min(tm, T - r0)))
    return tiles


def test_prefill8k_full_size():
    """The 8192-token chunk at full size, in the launch configuration the benchmark times: every
    token's ids and p, the full permutation, one y_sorted row in every row tile of the grouped GEMMs
    (all column tiles of that row) and one shared-expert row per shared tile against the oracle's
    expert outputs, and Y on sampled tokens."""
    _need_gpu()
    spec, d = host_layer("prefill8k")
    say("prefill8k: GPU layer")
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    T, k, H = spec.T, spec.k, spec.H
    rows = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(0).integers(0, T, 125)]))
    say("prefill8k: routing check")
    flips = check_routing(O, d["x"], g_logits, g_ids, g_p, token_rows=rows)
    L = dev_layer(spec, d)
    xd = dev_x(d["x"])
    off, perm, inv = moe.moe_permute(L, torch.from_numpy(g_ids).cuda())
    ys, ysh = moe.moe_experts_prefill(L, xd, off, perm)
    torch.cuda.synchronize()
    o_off, o_perm, o_inv = oracle.permute(g_ids, spec.E)
    assert np.array_equal(off.cpu().numpy(), o_off) and np.array_equal(perm.cpu().numpy(), o_perm)
    assert np.array_equal(inv.cpu().numpy(), o_inv)
    # one checked row in every tile of the tile list
    counts = np.diff(o_off)
    tiles = host_tiles(counts, T, spec.Is > 0)
    rng = np.random.default_rng(2)
    picks = [(g, r0 + int(rng.integers(0, n))) for g, r0, n in tiles]
    routed = [(g, o_off[g] + r) for g, r in picks if g < spec.E]
    shared = [r for g, r in picks if g == spec.E]
    xf = oracle.bf16_to_f64(d["x"])
    say("prefill8k: oracle on %d routed tile rows, %d shared tile rows" % (len(routed), len(shared)))
    want_r = np.stack(_pool_map(lambda it: O.expert(int(it[0]), xf[o_perm[it[1]] // k]), routed))
    want_s = np.stack(_pool_map(lambda t: O.shared(xf[t]), shared))
    ysn, yshn = ys.cpu().numpy(), ysh.cpu().numpy()
    rel_r, mx_r = assert_float_match(ysn[[i for _, i in routed]], want_r, "y_sorted (a row of every tile)")
    assert_float_match(yshn[shared], want_s, "y_shared (a row of every shared tile)")
    # Y on sampled tokens (incl. tokens of the hottest and of a 1-token expert)
    hot = int(np.argmax(counts))
    single = np.nonzero(counts == 1)[0]
    pick = [0, T - 1, int(np.nonzero((g_ids == hot).any(1))[0][0])]
    if len(single):
        pick.append(int(np.nonzero((g_ids == single[0]).any(1))[0][0]))
    pick += np.random.default_rng(1).integers(0, T, 12).tolist()
    pick = sorted(set(pick))
    say("prefill8k: oracle on %d tokens" % len(pick))
    outs = _pool_map(lambda t: O.token(d["x"][t], logits_in=g_logits[t].astype(np.float64)), pick)
    rel, mx = assert_float_match(Y[pick], np.stack([o["Y"] for o in outs]), "Y (sampled)")
    say("prefill8k %d tiles: y_sorted rel %.2e; Y rel %.2e maxabs/rms %.2e; flips %d of %d sampled"
        % (len(tiles), rel_r, rel, mx, flips, len(rows)))


# ------------------------------------------------------------------------- permutation edge cases

@pytest.mark.parametrize("T,E,k", [(1, 16, 2), (63, 256, 8), (64, 256, 8), (65, 1024, 16), (1000, 512, 10),
                                   (4097, 256, 8)])
def test_permute_edges(T, E, k):
    _need_gpu()
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[: T // 2] = ids[0]  # a very hot expert set for half the tokens
    spec = synth.LayerSpec("perm", T=T, H=64, E=E, k=k, I=64, Is=0, fmt=synth.Q8, zipf=False)
    desc = moe.LayerDesc.from_spec(spec)

    class _L:  # moe_permute only needs the descriptor
        pass
    lay = _L()
    lay.desc = desc
    off, perm, inv = moe.moe_permute(lay, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    o_off, o_perm, o_inv = oracle.permute(ids, E)
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(perm.cpu().numpy(), o_perm)
    assert np.array_equal(inv.cpu().numpy(), o_inv)


# ------------------------------------------------------------------------- special cases

@pytest.mark.parametrize("T,E,k", [(300, 64, 4), (3000, 1024, 8)])
def test_permute_drops_out_of_range_ids(T, E, k):
    """Ids outside [0, E) are dropped: no slot, inv = -1, offsets count the kept pairs, and the
    kept pairs keep the stable expert order (the one-block permutation at T = 300, the three-kernel
    one at T = 3000 with 1024 experts)."""
    _need_gpu()
    spec = synth.LayerSpec("permbad", T=T, H=64, E=E, k=k, I=64, Is=0, fmt=synth.Q8, zipf=False)
    rng = np.random.default_rng(11)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    bad = rng.random(ids.shape) < 0.05
    ids[bad] = rng.choice([-1, E, E + 7, -(1 << 30)], size=int(bad.sum()))
    class _L:  # moe_permute only needs the descriptor
        pass
    lay = _L()
    lay.desc = moe.LayerDesc.from_spec(spec)
    offsets, perm, inv = moe.moe_permute(lay, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    flat = ids.reshape(-1)
    keep = np.nonzero((flat >= 0) & (flat < E))[0]
    order = keep[np.argsort(flat[keep], kind="stable")]
    want_off = np.concatenate([[0], np.cumsum(np.bincount(flat[keep], minlength=E))])
    assert np.array_equal(offsets.cpu().numpy(), want_off)
    assert np.array_equal(perm.cpu().numpy()[:len(order)], order)
    want_inv = np.full(T * k, -1)
    want_inv[order] = np.arange(len(order))
    assert np.array_equal(inv.cpu().numpy(), want_inv)


def test_ties_and_signed_zero():
    """Equal logits pick the lower expert index; -0 and +0 are one value."""
    _need_gpu()
    spec = synth.LayerSpec("ties", T=3, H=64, E=16, k=4, I=64, Is=0, fmt=synth.Q4, zipf=False, cfg_id=77)
    d = synth.make_layer(spec)
    d["w_router"] = np.zeros_like(d["w_router"])
    bias = np.zeros(16, np.float32)
    bias[[3, 9]] = 1.0
    bias[[0, 5, 7]] = -0.0
    d["router_bias"] = bias
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    assert g_ids.tolist() == [[3, 9, 0, 1]] * 3
    O = orc_layer(spec, d)
    ref = oracle_tokens(O, d["x"], g_logits, range(3))
    assert np.array_equal(ref["ids"], g_ids)
    assert_float_match(Y, ref["Y"], "Y")


def test_k_equals_E_and_no_shared():
    _need_gpu()
    spec = synth.LayerSpec("kE", T=2, H=128, E=8, k=8, I=96, Is=0, fmt=synth.Q8, zipf=True, cfg_id=78)
    d = synth.make_layer(spec)
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(2))
    assert_float_match(Y, ref["Y"], "Y")


@pytest.mark.parametrize("T", [4, 100, 400])
def test_layer_max_experts(T):
    """The largest expert count and top-k (E = 1024, k = 16, with a shared expert): 64 routed pairs in
    the decode plan (T = 4); in the prefill path the top-k over 16 logits per lane, the one-block
    permutation (T = 100) and the three-kernel one (T = 400), the tile list with a group per thread."""
    _need_gpu()
    spec = synth.LayerSpec("maxE", T=T, H=256, E=1024, k=16, I=64, Is=64, fmt=synth.Q4, zipf=True, cfg_id=96)
    d = synth.make_layer(spec)
    say("max experts", "T=%d" % T)
    O = orc_layer(spec, d)
    g_logits, g_ids, g_p, Y = run_layer(spec, d)
    check_routing(O, d["x"], g_logits, g_ids, g_p)
    ref = oracle_tokens(O, d["x"], g_logits, range(T))
    assert_float_match(Y, ref["Y"], "Y")


def test_determinism():
    """Two calls give identical bits (atomic-free combine, stable permutation)."""
    _need_gpu()
    for name in ("decode1",):
        spec, d = host_layer(name)
        a = run_layer(spec, d)
        b = run_layer(spec, d)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)
    spec = small_prefill_spec(synth.Q4, 300)
    d = synth.make_layer(spec)
    a, b = run_layer(spec, d), run_layer(spec, d)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("T,H,E,k,I,Is", [(4, 1024, 64, 8, 1536, 0), (64, 2048, 256, 8, 512, 512),
                                          (5, 256, 16, 4, 128, 64)])
def test_prefill_repeat_bitwise(T, H, E, k, I, Is):
    """Repeated grouped-GEMM calls on identical inputs give identical bits (fp32 entry and fused
    layer). Guards the end of each tile's K loop: no transfer into LDS may still be in flight when
    the epilogue reuses the stages (small T, few tiles, short K loops expose any such race)."""
    _need_gpu()
    spec = synth.LayerSpec("rep", T=T, H=H, E=E, k=k, I=I, Is=Is, fmt=synth.Q4, zipf=True, cfg_id=98)
    d = synth.make_layer(spec)
    say("prefill repeat T=%d H=%d I=%d" % (T, H, I))
    L = dev_layer(spec, d, dmt=1)   # the fused layer on the grouped GEMMs too
    xd = dev_x(d["x"])
    _, ids, p = moe.moe_route(L, xd)
    off, perm, inv = moe.moe_permute(L, ids)
    first_y = first_Y = None
    for rep in range(6):
        ws = torch.full((moe.moe_workspace_size(L.desc, T, moe.MOE_CALL_EXPERTS_PREFILL),), rep * 37 % 256,
                        dtype=torch.uint8, device="cuda")
        y, _ = moe.moe_experts_prefill(L, xd, off, perm, ws=ws)
        Y = moe.moe_layer(L, xd)
        torch.cuda.synchronize()
        if first_y is None:
            first_y, first_Y = y.clone(), Y.clone()
        else:
            assert torch.equal(y, first_y), rep
            assert torch.equal(Y, first_Y), rep


def test_decode_layer_in_hip_graph():
    """moe_layer captured in a HIP graph: every replay (with eager work and syncs in between) meets
    the oracle (ids bit-exact from the replay's own logits, Y within the float rule) and equals the
    eager result bit for bit (the graph holds no memset nodes)."""
    _need_gpu()
    spec, d = host_layer("decode1")
    O = orc_layer(spec, d)
    L = dev_layer(spec, d)
    x = dev_x(d["x"])
    ws = moe.Workspace()
    out = torch.empty((spec.T, spec.H), dtype=torch.float32, device="cuda")
    ids = torch.empty((spec.T, spec.k), dtype=torch.int32, device="cuda")
    logits = torch.empty((spec.T, spec.E), dtype=torch.float32, device="cuda")
    moe.moe_layer(L, x, out=out, logits=logits, ids=ids, ws=ws)
    torch.cuda.synchronize()
    want_out, want_ids = out.clone(), ids.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_layer(L, x, out=out, logits=logits, ids=ids, ws=ws)
    ref = None
    for rep in range(3):
        out.fill_(float("nan"))
        ids.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        lg = logits.cpu().numpy()
        if ref is None:
            ref = oracle_tokens(O, d["x"], lg, range(spec.T))
        assert np.array_equal(ids.cpu().numpy(), oracle.topk_softmax(lg.astype(np.float64), spec.k)[0]), rep
        assert_float_match(out.cpu().numpy(), ref["Y"], "graph replay %d: Y" % rep)
        assert torch.equal(ids, want_ids), rep
        assert torch.equal(out, want_out), rep
        moe.moe_layer(L, x, out=torch.empty_like(out), ws=moe.Workspace())   # eager work between replays
        torch.cuda.synchronize()


def test_stack48_graph_replay():
    """The 48-layer decode stack as the benchmark runs it: 48 moe_layer calls (one per layer, each
    with its own input token and output) captured once as a HIP graph and replayed twice. Layers 0,
    23 and 47 carry their own generated weights and are checked against the oracle after every
    replay; the other 45 positions hold device copies of layer 0's weights (distinct addresses, same
    bytes) with their own inputs, so that the graph has the full length and memory footprint."""
    _need_gpu()
    spec = synth.CONFIGS["stack48"]
    checked = {}
    for l in (0, 23, 47):
        _, dl = host_layer("stack48", l)
        checked[l] = dl
    base = dev_layer(spec, checked[0])
    layers, xs = [], []
    for l in range(spec.layers):
        if l in checked:
            layers.append(base if l == 0 else dev_layer(spec, checked[l]))
            xs.append(dev_x(checked[l]["x"]))
        else:
            m = base.mats
            layers.append(moe.DeviceLayer(base.desc, base.w_router.clone(),
                                          None if base.router_bias is None else base.router_bias.clone(),
                                          *[(m[n][0].clone(), m[n][1].clone()) for n in ("gate", "up", "down")]))
            xs.append(dev_x(synth.make_x(spec, layer=l)))
    say("stack48 graph: %d layers resident" % len(layers))
    ws = moe.Workspace()
    outs = [torch.empty((1, spec.H), dtype=torch.float32, device="cuda") for _ in layers]
    lgs = [torch.empty((1, spec.E), dtype=torch.float32, device="cuda") for _ in layers]
    for L, x, o, lg in zip(layers, xs, outs, lgs):   # warm-up (workspace sized outside the capture)
        moe.moe_layer(L, x, out=o, logits=lg, ws=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for L, x, o, lg in zip(layers, xs, outs, lgs):
            moe.moe_layer(L, x, out=o, logits=lg, ws=ws)
    for rep in range(2):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for l, dl in checked.items():
            O = orc_layer(spec, dl)
            lg = lgs[l].cpu().numpy()
            ref = oracle_tokens(O, dl["x"], lg, range(1))
            assert_float_match(outs[l].cpu().numpy(), ref["Y"], "replay %d, layer %d: Y" % (rep, l))
        say("stack48 graph replay %d: layers 0, 23, 47 match the oracle" % rep)


# ------------------------------------------------------------------------- KV int8 codec

def _kv_rows(rng, rows, D):
    """bf16 rows mixing the cases the codec must get right: normal blocks, all-zero blocks, blocks
    whose scale is subnormal or rounds to 0, blocks near the fp16 scale overflow, signed zeros."""
    v = rng.standard_normal((rows, D)).astype(np.float32)
    nb = D // 32
    kind = rng.integers(0, 8, size=(rows, nb))
    for r in range(rows):
        for b in range(nb):
            blk = v[r, 32 * b:32 * b + 32]
            if kind[r, b] == 0:
                blk[:] = 0.0
            elif kind[r, b] == 1:
                blk *= 1e-6                  # scale subnormal in fp16
            elif kind[r, b] == 2:
                blk *= 1e-9                  # scale rounds to 0
            elif kind[r, b] == 3:
                blk *= 5e6                   # scale near / above the fp16 range
            elif kind[r, b] == 4:
                blk[::3] = -0.0
    bits = (v.view(np.uint32) >> 16).astype(np.uint16)
    # NaNs (code 0, left out of the block maximum) and infinities (scale saturates, code +-127)
    nan_at = rng.random(bits.shape) < 0.01
    bits[nan_at] = rng.choice(np.array([0x7FC0, 0xFFC0, 0x7F81, 0xFFFF], np.uint16), size=int(nan_at.sum()))
    inf_at = rng.random(bits.shape) < 0.002
    bits[inf_at] = rng.choice(np.array([0x7F80, 0xFF80], np.uint16), size=int(inf_at.sum()))
    if rows > 1:
        bits[1, :32] = 0x7FC0   # a whole block of NaNs
    return bits


def test_kv_encode_bit_exact():
    _need_gpu()
    rng = np.random.default_rng(21)
    src = _kv_rows(rng, 300, 512)
    say("kv encode 300 x 512")
    codes, scales = moe.moe_kv_encode(dev_x(src))
    torch.cuda.synchronize()
    o_codes, o_scales = oracle.kv_encode(src)
    assert np.array_equal(scales.cpu().numpy().view(np.uint16), o_scales)
    assert np.array_equal(codes.cpu().numpy(), o_codes)


def test_kv_gather_exact():
    _need_gpu()
    rng = np.random.default_rng(22)
    n_rows, D = 4096, 256
    src = _kv_rows(rng, n_rows, D)
    o_codes, o_scales = oracle.kv_encode(src)
    codes = torch.from_numpy(o_codes).cuda()
    scales = torch.from_numpy(o_scales.view(np.int16)).cuda()
    idx = rng.integers(0, n_rows, size=2048 * 3).astype(np.int32)
    idx[:5] = [0, n_rows - 1, -1, n_rows, 1 << 30]    # edges and out-of-range rows
    idx[5:9] = 17                                      # repeats
    say("kv gather %d rows of %d" % (len(idx), n_rows))
    out = moe.moe_kv_gather(codes, scales, torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    want = oracle.kv_gather(o_codes, o_scales, idx)
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))   # NaN and inf inputs still give finite rows
    assert np.array_equal(got, want)


def test_kv_full_size_sampled():
    """Cache of 131072 positions x 512 (the size the benchmark gathers from): GPU encode of every
    row, checked bit for bit on 256 sampled rows; gather of 16 x 2048 positions checked exactly."""
    _need_gpu()
    rng = np.random.default_rng(23)
    n_rows, D = 131072, 512
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((n_rows, D), generator=g, device="cuda").to(torch.bfloat16)
    say("kv full size encode %d x %d" % (n_rows, D))
    codes, scales = moe.moe_kv_encode(x)
    idx = torch.from_numpy(rng.integers(0, n_rows, size=16 * 2048).astype(np.int32)).cuda()
    out = moe.moe_kv_gather(codes, scales, idx)
    torch.cuda.synchronize()
    rows = np.sort(rng.choice(n_rows, 256, replace=False))
    xs = x[torch.from_numpy(rows).cuda()].view(torch.int16).cpu().numpy().view(np.uint16)
    o_codes, o_scales = oracle.kv_encode(xs)
    assert np.array_equal(codes[torch.from_numpy(rows).cuda()].cpu().numpy(), o_codes)
    assert np.array_equal(scales[torch.from_numpy(rows).cuda()].cpu().numpy().view(np.uint16), o_scales)
    pick = rng.choice(len(idx), 512, replace=False)
    ii = idx.cpu().numpy()[pick]
    want = oracle.kv_gather(codes.cpu().numpy(), scales.cpu().numpy().view(np.uint16), ii)
    assert np.array_equal(out.cpu().numpy()[pick].astype(np.float64), want)


def test_error_statuses_on_gpu():
    _need_gpu()
    spec, d = host_layer("tiny")
    L = dev_layer(spec, d)
    x9 = dev_x(np.zeros((9, spec.H), np.uint16))
    ids = torch.zeros((9, spec.k), dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_experts_decode(L, x9, ids)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    tiny_ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as e:
        moe.moe_layer(L, dev_x(d["x"]), ws=tiny_ws)
    assert e.value.status == moe.MOE_ERR_WORKSPACE
