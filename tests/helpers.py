"""Shared test helpers: the float matching rule, layer construction on host and device."""
from __future__ import annotations

import functools

import numpy as np

import synth

REL_L2_MAX = 2e-3        # relative L2 error of a float output tensor
MAX_ABS_RMS = 1e-2       # max-abs error as a fraction of rms(oracle output)


def float_errors(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    diff = got - want
    nw = np.linalg.norm(want)
    rel = np.linalg.norm(diff) / nw if nw > 0 else np.linalg.norm(diff)
    rms = np.sqrt(np.mean(want ** 2)) if want.size else 0.0
    mx = np.max(np.abs(diff)) if diff.size else 0.0
    return rel, (mx / rms if rms > 0 else mx)


def assert_float_match(got, want, what=""):
    rel, mx = float_errors(got, want)
    assert rel <= REL_L2_MAX and mx <= MAX_ABS_RMS, "%s: rel L2 %.3e (max %.0e), max-abs/rms %.3e (max %.0e)" % (
        what, rel, REL_L2_MAX, mx, MAX_ABS_RMS)
    return rel, mx


@functools.lru_cache(maxsize=4)
def host_layer(name: str, layer: int = 0, seed: int = 0):
    spec = synth.CONFIGS[name]
    return spec, synth.make_layer(spec, layer=layer, seed=seed)
