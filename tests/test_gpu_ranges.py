"""GPU parity over the activation range and the decode kernel matrix.

The 16-bit operands of the HIP path (x and the SwiGLU activation h as fp16 on the dot-product and
matrix-core paths, and the fused layer's fp16 expert rows) are taken at a power-of-two scale of
each token, so the layer must meet the float rule (relative L2 <= 2e-3, max-abs <= 1e-2 *
rms(oracle)) whatever the size of the activations: tokens of rms 1e-6 ... 1e4, tokens holding
values beyond the fp16 range (|x| >= 65504), and all-zero tokens (output exactly 0). The oracle is
fp64 throughout, so it needs no such care.

The decode kernels are instantiated per format and token count (T = 1 .. 8); every one of the 24
runs here through moe_layer (top-k inside the gate/up kernel) and moe_experts_decode (ids given),
with and without a shared expert, and with E in (64, 128] (two router keys per lane in the top-k).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_float_match

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("quantized_expert_ffn_moe_amd")

SCALES = [1.0, 1e-6, 1e-4, 1e-2, 1e2, 1e4]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[gpu-ranges]", *a, flush=True)
    sys.stdout.flush()


def bf16_bits(v):
    """fp32 values -> bf16 bits, round to nearest even."""
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def activation_cases(spec, T, seed):
    """(label, x bits [T][H]) for every activation size under test."""
    out = []
    for s in SCALES:
        out.append(("rms %g" % s, synth.make_x(spec, seed=seed, T=T, sigma=s)))
    # tokens holding values beyond the fp16 range, next to ordinary ones
    xv = synth.make_x(spec, seed=seed, T=T).view(np.uint16).astype(np.uint32) << 16
    xf = xv.view(np.float32).copy()
    rng = np.random.default_rng(seed)
    for t in range(T):
        cols = rng.choice(spec.H, 3, replace=False)
        if t % 2 == 0:
            xf[t, cols] = [99840.0, -70000.0, 3.0e5]
        else:
            xf[t] *= 1e4
            xf[t, cols[0]] = -2.5e5
    out.append(("|x| >= 65504", bf16_bits(xf)))
    # an all-zero token (output exactly 0) next to ordinary ones
    z = synth.make_x(spec, seed=seed, T=T).copy()
    z[0] = 0
    out.append(("zero token", z))
    return out


def orc_tokens(O, x, g_logits):
    outs = [O.token(x[t], logits_in=g_logits[t].astype(np.float64)) for t in range(x.shape[0])]
    return {k: np.stack([o[k] for o in outs]) for k in outs[0]}


def check_y(got, want, what):
    if not np.any(want):
        assert np.array_equal(got, np.zeros_like(got)), what + ": expected exact zeros"
        return
    assert np.all(np.isfinite(got)), what + ": non-finite values"
    assert_float_match(got, want, what)


@pytest.mark.parametrize("fmt", [synth.Q8, synth.Q4, synth.Q2])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 6, 7, 8])
def test_decode_matrix_and_ranges(fmt, T):
    _need_gpu()
    E = 100 if T % 2 else 16           # E in (64, 128]: two keys per lane in the top-k
    Is = 64 if T % 2 == 0 else 0
    spec = synth.LayerSpec("dm", T=T, H=512, E=E, k=4, I=160, Is=Is, fmt=fmt, zipf=True, cfg_id=200 + fmt)
    d = synth.make_layer(spec)
    # moe_layer on the decode kernels at every T here (its default switch is lower)
    L = moe.DeviceLayer.from_host(moe.LayerDesc.from_spec(spec, decode_max_tokens=8), d)
    O = oracle.Layer.from_synth(spec, d)
    for label, x in activation_cases(spec, T, 3 + T):
        say(synth.FMT_NAMES[fmt], "T=%d E=%d Is=%d" % (T, E, Is), label)
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda")
        Y = moe.moe_layer(L, xd, logits=logits, ids=ids)
        y_pairs, y_sh = moe.moe_experts_decode(L, xd, ids)
        torch.cuda.synchronize()
        g_logits = logits.cpu().numpy()
        ref = orc_tokens(O, x, g_logits)
        assert np.array_equal(ids.cpu().numpy(), ref["ids"]), label
        check_y(Y.cpu().numpy(), ref["Y"], "%s Y" % label)
        check_y(y_pairs.cpu().numpy().reshape(T, spec.k, spec.H), ref["y_pairs"], "%s y_pairs" % label)
        if Is:
            check_y(y_sh.cpu().numpy(), ref["y_shared"], "%s y_shared" % label)


@pytest.mark.parametrize("fmt", [synth.Q8, synth.Q4, synth.Q2])
def test_prefill_ranges(fmt):
    """The grouped-GEMM path (130 tokens: several row tiles, ragged groups) at every activation
    size: the fused layer (fp16 rows at the token scale, unscaled in the combine), the fp32 entry
    and the fp16 entry (true scale, saturating at +-65504: bitwise the fp32 rows clamped and
    rounded)."""
    _need_gpu()
    T = 130
    spec = synth.LayerSpec("pr", T=T, H=256, E=16, k=4, I=128, Is=64, fmt=fmt, zipf=True, cfg_id=210 + fmt)
    d = synth.make_layer(spec)
    L = moe.DeviceLayer.from_host(moe.LayerDesc.from_spec(spec), d)
    O = oracle.Layer.from_synth(spec, d)
    for label, x in activation_cases(spec, T, 11):
        say("prefill", synth.FMT_NAMES[fmt], label)
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        logits = torch.empty((T, spec.E), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda")
        Y = moe.moe_layer(L, xd, logits=logits, ids=ids)
        offsets, perm, inv = moe.moe_permute(L, ids)
        y32, ysh32 = moe.moe_experts_prefill(L, xd, offsets, perm)
        y16, ysh16 = moe.moe_experts_prefill(L, xd, offsets, perm, half=True)
        torch.cuda.synchronize()
        g_logits = logits.cpu().numpy()
        ref = orc_tokens(O, x, g_logits)
        assert np.array_equal(ids.cpu().numpy(), ref["ids"]), label
        check_y(Y.cpu().numpy(), ref["Y"], "%s Y" % label)
        o_perm = oracle.permute(ids.cpu().numpy(), spec.E)[1]
        want_sorted = ref["y_pairs"].reshape(T * spec.k, spec.H)[o_perm]
        check_y(y32.cpu().numpy(), want_sorted, "%s y_sorted" % label)
        check_y(ysh32.cpu().numpy(), ref["y_shared"], "%s y_shared" % label)
        for a16, a32 in ((y16, y32), (ysh16, ysh32)):
            assert torch.equal(a16.view(torch.int16),
                               a32.clamp(-65504.0, 65504.0).to(torch.float16).view(torch.int16)), label
