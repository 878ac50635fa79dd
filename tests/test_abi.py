"""The C-ABI library on the CPU: it loads, exports every entry point include/moe.h declares, sizes
workspaces, and rejects bad arguments on the host before any GPU work (no compute calls here)."""
import ctypes
import os
import re

import pytest

import quantized_expert_ffn_moe_amd as moe
from quantized_expert_ffn_moe_amd import build as moe_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(moe.library_path):
        moe_build.build()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert {"moe_route", "moe_permute", "moe_experts_decode", "moe_experts_prefill", "moe_combine", "moe_layer",
            "moe_workspace_size", "moe_status_string", "moe_abi_version", "moe_kv_encode", "moe_kv_gather",
            "moe_experts_prefill_f16", "moe_prefill_codes_bytes", "moe_pack_prefill_codes"} <= set(names)
    L = ctypes.CDLL(moe.library_path)
    for n in names:
        assert hasattr(L, n), n
    assert moe.moe_abi_version() == 3
    assert moe.moe_status_string(moe.MOE_ERR_WORKSPACE) == "workspace too small"


def D(H=2048, I=512, E=256, k=8, Is=512, fmt=moe.MOE_Q4_B32, dmt=0):
    return moe.LayerDesc(H, I, E, k, Is, fmt, dmt)


def test_workspace_sizes():
    d = D()
    for call in range(6):
        n = moe.moe_workspace_size(d, 1, call)
        assert n >= 0
    assert moe.moe_workspace_size(d, 8192, moe.MOE_CALL_LAYER) > 8192 * 8 * 2048 * 2   # holds fp16 y_sorted
    assert moe.moe_workspace_size(d, 4, moe.MOE_CALL_COMBINE) == 0
    assert moe.moe_workspace_size(d, 8, moe.MOE_CALL_EXPERTS_DECODE) > 0      # up to 8 tokens (T k <= 64)
    for T, dd in ((9, d), (5, D(k=16, E=256))):                                # T > 8, or T k > 64
        with pytest.raises(moe.MoeError) as e:
            moe.moe_workspace_size(dd, T, moe.MOE_CALL_EXPERTS_DECODE)
        assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    # the prefill tiles take any H, I, Is that are multiples of 32
    assert moe.moe_workspace_size(D(H=96, I=32, Is=32), 8, moe.MOE_CALL_EXPERTS_PREFILL) > 0


@pytest.mark.parametrize("bad", [dict(k=0), dict(k=17, E=32), dict(k=9, E=8), dict(E=1025), dict(H=100),
                                 dict(I=0), dict(Is=48 + 1), dict(fmt=3), dict(H=32768), dict(dmt=9),
                                 dict(dmt=-1)])
def test_bad_descriptors(bad):
    with pytest.raises(moe.MoeError) as e:
        moe.moe_workspace_size(D(**bad), 1, moe.MOE_CALL_LAYER)
    assert e.value.status == moe.MOE_ERR_INVALID_ARG


def test_layer_regime_switch_sizes_the_workspace():
    """decode_max_tokens moves moe_layer's regime switch; the layer workspace follows the path taken
    (the grouped-GEMM path holds fp16 expert rows, the decode path does not)."""
    dec, gemm = D(dmt=8), D(dmt=1)
    assert moe.moe_workspace_size(dec, 8, moe.MOE_CALL_LAYER) < 8 * 8 * 2048 * 2
    assert moe.moe_workspace_size(gemm, 8, moe.MOE_CALL_LAYER) > 8 * 8 * 2048 * 2
    # the default switch on this shape: decode kernels up to 6 tokens, grouped GEMMs from 7
    assert moe.moe_workspace_size(D(), 6, moe.MOE_CALL_LAYER) < 6 * 8 * 2048 * 2
    assert moe.moe_workspace_size(D(), 7, moe.MOE_CALL_LAYER) > 7 * 8 * 2048 * 2


def _raw(fn, *args):
    return getattr(moe.lib(), fn)(*args)


def test_host_validation_rejects_before_launch():
    """Invalid calls return a status without touching the GPU (fake but aligned device addresses)."""
    d = D()
    fake = 0x10000
    w = moe._Weights(fake, None, moe._QMat(fake, fake), moe._QMat(fake, fake), moe._QMat(fake, fake),
                     moe._QMat(fake, fake), moe._QMat(fake, fake), moe._QMat(fake, fake))
    ref = ctypes.byref
    # T = 0
    assert _raw("moe_layer", ref(d.c), ref(w), fake, 0, fake, None, None, None, fake, 1 << 40, None) == \
        moe.MOE_ERR_INVALID_ARG
    # misaligned x
    assert _raw("moe_layer", ref(d.c), ref(w), fake + 2, 1, fake, None, None, None, fake, 1 << 40, None) == \
        moe.MOE_ERR_INVALID_ARG
    # workspace too small
    assert _raw("moe_layer", ref(d.c), ref(w), fake, 1, fake, None, None, None, fake, 64, None) == \
        moe.MOE_ERR_WORKSPACE
    # missing workspace
    assert _raw("moe_layer", ref(d.c), ref(w), fake, 1, fake, None, None, None, None, 0, None) == \
        moe.MOE_ERR_INVALID_ARG
    # decode entry with T > 8
    assert _raw("moe_experts_decode", ref(d.c), ref(w), fake, 9, fake, fake, fake, fake, 1 << 40, None) == \
        moe.MOE_ERR_UNSUPPORTED
    # null router weights for route
    w2 = moe._Weights(None, None, w.gate, w.up, w.down, w.sh_gate, w.sh_up, w.sh_down)
    assert _raw("moe_route", ref(d.c), ref(w2), fake, 1, fake, fake, fake, None, 0, None) == moe.MOE_ERR_INVALID_ARG
    # shared expert declared but missing
    w3 = moe._Weights(fake, None, w.gate, w.up, w.down, moe._QMat(None, None), w.sh_up, w.sh_down)
    assert _raw("moe_experts_decode", ref(d.c), ref(w3), fake, 1, fake, fake, fake, fake, 1 << 40, None) == \
        moe.MOE_ERR_INVALID_ARG
    # permute without outputs
    assert _raw("moe_permute", ref(d.c), fake, 4, None, fake, fake, fake, 1 << 40, None) == moe.MOE_ERR_INVALID_ARG
    # combine with misaligned rows
    assert _raw("moe_combine", ref(d.c), 1, fake, fake + 4, None, None, fake, None) == moe.MOE_ERR_INVALID_ARG
    # prefill with a shared expert but no y_shared
    assert _raw("moe_experts_prefill", ref(d.c), ref(w), fake, 8, fake, fake, fake, None, fake, 1 << 40, None) == \
        moe.MOE_ERR_INVALID_ARG
    assert _raw("moe_experts_prefill_f16", ref(d.c), ref(w), fake, 8, fake, fake, fake, None, fake, 1 << 40, None) == \
        moe.MOE_ERR_INVALID_ARG
    # fp16 rows must be 16-byte aligned
    assert _raw("moe_experts_prefill_f16", ref(d.c), ref(w), fake, 8, fake, fake, fake + 2, fake, fake, 1 << 40,
                None) == moe.MOE_ERR_INVALID_ARG


def test_prefill_codes_size_and_checks():
    """The packed copy's size from its definition in moe.h (every matrix ceil(N / 32) ceil(K / 64)
    pieces of 64 BB code bytes and ceil(N / 32) ceil(K / 256) pieces of 512 scale bytes; E gates and
    ups of I x H, E downs of H x I, the shared three), 0 for an
    invalid descriptor; moe_pack_prefill_codes refuses a missing or misaligned destination or a
    misaligned prefill_codes in the weights before launching anything (fake aligned device
    addresses, no GPU here)."""
    ref = ctypes.byref
    for fmt, BB in ((moe.MOE_Q8_B32, 32), (moe.MOE_Q4_B32, 16), (moe.MOE_Q2_B32, 8)):
        for E, H, I, Is in ((5, 800, 160, 96), (256, 2048, 512, 512), (3, 64, 32, 0)):
            d = D(H=H, I=I, E=E, k=2, Is=Is, fmt=fmt)

            def P(N, K):   # codes and scales of one matrix
                return -(-N // 32) * -(-K // 64) * 64 * BB + -(-N // 32) * -(-K // 256) * 512
            want = E * (2 * P(I, H) + P(H, I)) + ((2 * P(Is, H) + P(H, Is)) if Is else 0)
            assert _raw("moe_prefill_codes_bytes", ref(d.c)) == want
    assert _raw("moe_prefill_codes_bytes", ref(D(H=33).c)) == 0
    d, fake = D(), 0x10000
    q = moe._QMat(fake, fake)
    w = moe._Weights(fake, None, q, q, q, q, q, q, None)
    assert _raw("moe_pack_prefill_codes", ref(d.c), ref(w), None, None) == moe.MOE_ERR_INVALID_ARG
    assert _raw("moe_pack_prefill_codes", ref(d.c), ref(w), fake + 8, None) == moe.MOE_ERR_INVALID_ARG
    w_bad = moe._Weights(fake, None, q, q, q, q, q, q, fake + 4)
    assert _raw("moe_pack_prefill_codes", ref(d.c), ref(w_bad), fake, None) == moe.MOE_ERR_INVALID_ARG
    assert _raw("moe_layer", ref(d.c), ref(w_bad), fake, 100, fake, None, None, None, fake, 1 << 40, None) == \
        moe.MOE_ERR_INVALID_ARG


def test_decode_lds_limit_settled_before_launch():
    """The decode kernels keep every chosen pair's SwiGLU activations in LDS (160 KB per workgroup).
    A shape beyond that makes moe_experts_decode return MOE_ERR_UNSUPPORTED from the host check,
    before anything is enqueued (fake device addresses, no GPU here: a launch would fail
    differently), moe_workspace_size says the same, and moe_layer sizes its workspace for the
    grouped-GEMM path it then takes."""
    big = D(H=1024, I=1536, E=64, k=8, Is=0)            # 36 pairs x 1536 activations x 4 B = 221 KB
    with pytest.raises(moe.MoeError) as e:
        moe.moe_workspace_size(big, 4, moe.MOE_CALL_EXPERTS_DECODE)
    assert e.value.status == moe.MOE_ERR_UNSUPPORTED
    fake = 0x10000
    w = moe._Weights(fake, None, moe._QMat(fake, fake), moe._QMat(fake, fake), moe._QMat(fake, fake),
                     moe._QMat(None, None), moe._QMat(None, None), moe._QMat(None, None))
    assert _raw("moe_experts_decode", ctypes.byref(big.c), ctypes.byref(w), fake, 4, fake, fake, None, fake,
                1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    # the layer's workspace holds the grouped-GEMM path's fp16 expert rows for this shape
    assert moe.moe_workspace_size(big, 4, moe.MOE_CALL_LAYER) >= 4 * 8 * 1024 * 2
    # one token fits the decode kernels; the 512-expert top-10 2-bit shape fits at T = 4 too (the
    # per-pair partial sums are then reduced in chunks of slots)
    assert moe.moe_workspace_size(big, 1, moe.MOE_CALL_EXPERTS_DECODE) > 0
    s48 = D(H=2048, I=768, E=512, k=10, Is=0, fmt=moe.MOE_Q2_B32)
    assert moe.moe_workspace_size(s48, 4, moe.MOE_CALL_EXPERTS_DECODE) > 0


def test_layer_static_limits_on_host():
    """moe_layer_static: a 16 MiB device array; a shape whose layer workspace exceeds it is refused
    with MOE_ERR_UNSUPPORTED by the host check, before any GPU call (there is no GPU here)."""
    assert moe.moe_layer_static_max_bytes() == 16 << 20
    d = D()
    assert moe.moe_workspace_size(d, 4, moe.MOE_CALL_LAYER) <= moe.moe_layer_static_max_bytes()
    assert moe.moe_workspace_size(d, 8192, moe.MOE_CALL_LAYER) > moe.moe_layer_static_max_bytes()
    fake = 0x10000
    w = moe._Weights(fake, None, moe._QMat(fake, fake), moe._QMat(fake, fake), moe._QMat(fake, fake),
                     moe._QMat(fake, fake), moe._QMat(fake, fake), moe._QMat(fake, fake))
    assert _raw("moe_layer_static", ctypes.byref(d.c), ctypes.byref(w), fake, 8192, fake, None, None, None,
                None) == moe.MOE_ERR_UNSUPPORTED
    assert _raw("moe_layer_static", ctypes.byref(d.c), ctypes.byref(w), fake, 0, fake, None, None, None,
                None) == moe.MOE_ERR_INVALID_ARG


def test_kv_validation_rejects_before_launch():
    fake = 0x10000
    assert _raw("moe_kv_encode", fake, 4, 48, fake, fake, None) == moe.MOE_ERR_INVALID_ARG        # D % 32
    assert _raw("moe_kv_encode", fake, -1, 64, fake, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert _raw("moe_kv_encode", fake + 2, 4, 64, fake, fake, None) == moe.MOE_ERR_INVALID_ARG    # src align
    assert _raw("moe_kv_encode", None, 0, 64, None, None, None) == moe.MOE_OK                     # nothing to do
    assert _raw("moe_kv_gather", fake, fake, 10, 64, fake + 2, 8, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert _raw("moe_kv_gather", fake, fake, 10, 64, fake, 8, fake + 4, None) == moe.MOE_ERR_INVALID_ARG
    assert _raw("moe_kv_gather", fake, fake, 10, 64, fake, -3, fake, None) == moe.MOE_ERR_INVALID_ARG
    assert _raw("moe_kv_gather", None, None, 10, 64, None, 0, None, None) == moe.MOE_OK


def test_binding_refuses_host_tensors():
    import torch
    d = D(H=64, I=64, E=4, k=2, Is=0)
    with pytest.raises(ValueError):
        moe.DeviceLayer(d, torch.zeros(4, 64), None, (torch.zeros(1, dtype=torch.uint8), torch.zeros(1)),
                        (torch.zeros(1), torch.zeros(1)), (torch.zeros(1), torch.zeros(1)))
