"""The seeded generator: determinism, rounding against library conversions, the encoder's packing
against hand-built bytes, and the Zipf routing bias."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    v = synth.normal_f32(synth.key(1, 2), 100000, 3.0)
    v[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]          # exact ties round to even
    mine = np.array([synth.lib().synth_f32_to_bf16(float(a)) for a in v], np.uint16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(30000) * 10.0 ** rng.integers(-9, 6, 30000),
                        [65504.0, 65520.0, 65519.99, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 6.1e-5, -0.0]])
    v = v.astype(np.float32)
    mine = np.array([synth.lib().synth_f32_to_f16(float(a)) for a in v], np.uint16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)


def test_streams_deterministic_and_distinct():
    a = synth.normal_f32(synth.key(0, 5, 3, 1), 4096)
    b = synth.normal_f32(synth.key(0, 5, 3, 1), 4096)
    c = synth.normal_f32(synth.key(0, 5, 4, 1), 4096)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    big = synth.normal_f32(synth.key(0, 9), 2_000_000)
    assert abs(big.mean()) < 3e-3 and abs(big.std() - 1) < 3e-3


def test_expert_stack_regenerates_per_expert():
    k = synth.key(0, 42)
    codes, scales = synth.expert_stack(synth.Q4, k, 5, 16, 64, 0.02, nthreads=3)
    c1, s1 = synth.expert_stack(synth.Q4, k, 5, 16, 64, 0.02, nthreads=1)
    assert np.array_equal(codes, c1) and np.array_equal(scales, s1)
    w3 = synth.expert_weights_f32(k, 3, 16, 64, 0.02)
    c3, s3 = synth.quantize_rows(synth.Q4, w3)
    assert np.array_equal(c3, codes[3]) and np.array_equal(s3, scales[3])


def test_encoder_packing_hand_example():
    w = np.zeros((1, 32), np.float32)
    w[0, :4] = [0.7, -0.7, 0.35, 0.0]
    c, s = synth.quantize_rows(synth.Q4, w)
    assert s[0, 0] == np.float16(0.1).view(np.uint16)                     # fp16(0.7 / 7)
    # 0.7/s = 7.0017 -> 7; -7 -> nibble 9; 0.35/s = 3.5008 -> 4; element 2i in the low nibble
    assert c[0, :2].tolist() == [0x97, 0x04] and not c[0, 2:].any()
    c8, s8 = synth.quantize_rows(synth.Q8, w)
    # s = fp16(0.7 / 127) = 0.005512; 0.35 / s = 63.495 -> 63
    assert s8[0, 0] == np.float16(0.005512).view(np.uint16)
    assert c8[0, :4].view(np.int8).tolist() == [127, -127, 63, 0]
    w2 = np.zeros((1, 32), np.float32)
    w2[0, :4] = [0.3, -0.3, 0.1, 0.0]
    c2, s2 = synth.quantize_rows(synth.Q2, w2)
    # s = 0.2: levels c - 1.5 -> 0.3 -> c 3, -0.3 -> c 0, 0.1 -> 0.5+1.5 = 2, 0 -> rne(1.5) = 2
    assert c2[0, 0] == (3 | (0 << 2) | (2 << 4) | (2 << 6))
    z, zs = synth.quantize_rows(synth.Q2, np.zeros((1, 32), np.float32))
    assert zs[0, 0] == 0 and z[0, 0] == 0xAA                              # scale 0: c = 2 everywhere


def test_zipf_bias():
    b, rank = synth.zipf_bias(synth.key(0, 2, 0, 3), 256, 1.1)
    assert sorted(rank.tolist()) == list(range(1, 257))
    np.testing.assert_allclose(b, (-1.1 * np.log(rank.astype(np.float64))).astype(np.float32), rtol=0, atol=0)


def test_config_shapes():
    s = synth.CONFIGS["decode1"]
    assert s.expert_bytes() == 1_769_472
    assert synth.CONFIGS["verify4"].expert_bytes() == 3_342_336
    assert synth.CONFIGS["stack48"].expert_bytes() == 1_474_560
    assert synth.CONFIGS["tiny"].expert_bytes() == 104_448
