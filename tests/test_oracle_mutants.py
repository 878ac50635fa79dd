"""Plant plausible mistakes in copies of the oracle (on the CPU) and show the pins catch each one.

Each mutant is a textual edit of ``oracle/moe_oracle.c`` compiled to a temporary library; the pin
functions of ``test_oracle_pins.py`` are run against it and at least one must fail.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")

MUTANTS = {
    "q4_nibble_order": ("(kappa % 2 == 0) ? (byte & 0x0F) : (byte >> 4)", "(kappa % 2 == 0) ? (byte >> 4) : (byte & 0x0F)"),
    "q4_no_sign_extension": ("nib >= 8 ? nib - 16 : nib", "nib"),
    "q2_offset": ("(double)c - 1.5", "(double)c - 2.0"),
    "q2_lane_order": ("(byte >> (2 * (kappa % 4))) & 3", "(byte >> (2 * (3 - kappa % 4))) & 3"),
    "scale_block_index": ("(int64_t)n * (K / 32) + kappa / 32", "(int64_t)n * (K / 32) + kappa % (K / 32)"),
    "f16_exponent_bias": ("ex - 25", "ex - 24"),
    "bf16_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "router_bias_dropped": ("acc + (L->bias ? (double)L->bias[e] : 0.0)", "acc"),
    "tie_to_higher_index": ("if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] >= l[best]) best = e;"),
    "softmax_unnormalised": ("exp(l[ids[(int64_t)t * k + j]] - lmax) / denom;", "exp(l[ids[(int64_t)t * k + j]] - lmax);"),
    "silu_sign": ("h[n] = g / (1.0 + exp(-g)) * u;", "h[n] = g / (1.0 + exp(g)) * u;"),
    "swiglu_operands_swapped": ("h[n] = g / (1.0 + exp(-g)) * u;", "h[n] = u / (1.0 + exp(-u)) * g;"),
    "combine_ignores_p": ("acc[m] += pr[j] * y[m];", "acc[m] += y[m];"),
    "shared_dropped": ("for (int32_t m = 0; m < H; ++m) acc[m] += y[m];", ";"),
    "permutation_unstable": ("int32_t pos = offsets[e] + seen[e];", "int32_t pos = offsets[e + 1] - 1 - seen[e];"),
    "combine_alone_row_map": ("int64_t r = row_of_pair ? row_of_pair[q] : q;", "int64_t r = q;"),
    "kv_scale_divisor": ("float q = m / 127.0f;", "float q = m / 128.0f;"),
    "kv_scale_overflow": ("if (sb == 0x7C00u) sb = 0x7BFFu;", ";"),
    "kv_ties_away": ("float t = rintf(xv / sf);", "float t = roundf(xv / sf);"),
    "kv_nan_in_max": ("if (a > m) m = a;", "if (!(a <= m)) m = a;"),
    "kv_f16_truncation": ("double m = nearbyint(a / step);", "double m = floor(a / step);"),
    "kv_gather_block_index": ("orc_f16(scales[(int64_t)r * (D / 32) + d / 32])", "orc_f16(scales[(int64_t)r * (D / 32) + d % (D / 32)])"),
    "up_uses_gate": ("u += weight(fmt, u_codes, u_scales, H, n, kappa) * x[kappa];",
                     "u += weight(fmt, g_codes, g_scales, H, n, kappa) * x[kappa];"),
}


def _build(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation target vanished: " + name
    path_c = os.path.join(tmp, name + ".c")
    open(path_c, "w").write(src.replace(old, new))
    hdr = os.path.join(os.path.dirname(SRC))
    path_so = os.path.join(tmp, name + ".so")
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-shared", "-fPIC", "-I", hdr, path_c,
                           "-o", path_so, "-lm"])
    return path_so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        so = _build(name, old, new, tmp)
        saved = oracle._lib
        oracle._lib = oracle.load(so)
        failed = []
        try:
            for pin_name, fn in pins.ALL_PINS:
                try:
                    fn()
                except (AssertionError, ValueError):
                    failed.append(pin_name)
        finally:
            oracle._lib = saved
    assert failed, "no pin caught mutant " + name
