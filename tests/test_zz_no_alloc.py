"""moe_layer_static (the allocation-free variant of moe_layer) against moe_layer, through the C ABI.

Two calls in a row on the library's shared device array, the second with a smaller input, for a
decode shape (4 tokens, then 1) and a grouped-GEMM shape (100 tokens, then 37): each output equals
moe_layer's bit for bit (same kernels, same inputs) and meets the float rule against the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_float_match

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("quantized_expert_ffn_moe_amd")


def _static_raw(L, x, out, logits, ids):
    T = x.shape[0]
    return moe.lib().moe_layer_static(ctypes.byref(L.desc.c), ctypes.byref(L.c), x.data_ptr(), T, out.data_ptr(),
                                      logits.data_ptr(), ids.data_ptr(), None,
                                      torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("shape,T1,T2", [("decode", 4, 1), ("prefill", 100, 37)])
def test_layer_static_matches_layer(shape, T1, T2):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if shape == "decode":
        spec = synth.LayerSpec("st", T=T1, H=2048, E=256, k=8, I=512, Is=512, fmt=synth.Q8, zipf=True, cfg_id=120)
    else:
        spec = synth.LayerSpec("st", T=T1, H=512, E=32, k=4, I=256, Is=128, fmt=synth.Q4, zipf=True, cfg_id=121)
    d = synth.make_layer(spec)
    L = moe.DeviceLayer.from_host(moe.LayerDesc.from_spec(spec), d)
    O = oracle.Layer.from_synth(spec, d)
    for T in (T1, T2):
        x = d["x"][:T]
        xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
        out = torch.full((T, spec.H), float("nan"), dtype=torch.float32, device="cuda")
        logits = torch.empty((T, spec.E), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, spec.k), dtype=torch.int32, device="cuda")
        st = _static_raw(L, xd, out, logits, ids)
        assert st == moe.MOE_OK, moe.moe_status_string(st)
        ref_out = moe.moe_layer(L, xd)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), (shape, T)
        lg = logits.cpu().numpy()
        assert np.array_equal(ids.cpu().numpy(), oracle.topk_softmax(lg.astype(np.float64), spec.k)[0])
        want = np.stack([O.token(x[t], logits_in=lg[t].astype(np.float64))["Y"] for t in range(T)])
        assert_float_match(out.cpu().numpy(), want, "%s T=%d" % (shape, T))
