"""The seeded generators reproduce the statistics printed on the Neutrino-1 8B
model page ("Inside the coded lane": 62.63 % zero, 18.68 % +1, 18.69 % -1;
70-72 % zeros for gate and down in layers 1-3) and are deterministic."""
from __future__ import annotations

import math

import numpy as np

import synth


def _within_5_sigma(count, n, p):
    sigma = math.sqrt(n * p * (1 - p))
    return abs(count - n * p) <= 5 * sigma


def test_code_distribution_global():
    n, k = 1024, 4096
    c = synth.ternary_codes(synth.tensor_seed(0, "q"), n, k)
    total = n * k
    assert _within_5_sigma(int((c == 0).sum()), total, synth.P_ZERO)
    assert _within_5_sigma(int((c == 1).sum()), total, synth.P_PLUS)
    assert _within_5_sigma(int((c == -1).sum()), total, synth.P_MINUS)
    assert set(np.unique(c).tolist()) == {-1, 0, 1}


def test_code_distribution_early_ffn():
    d = synth.code_dist(2, "gate")
    assert d.p_zero == 0.71 and d.p_plus == d.p_minus
    assert synth.code_dist(2, "up") == synth.GLOBAL_DIST
    assert synth.code_dist(0, "down") == synth.GLOBAL_DIST
    assert synth.code_dist(3, "down").p_zero == 0.71
    c = synth.ternary_codes(1, 512, 4096, d)
    assert _within_5_sigma(int((c == 0).sum()), c.size, 0.71)


def test_deterministic_and_ranges():
    a = synth.ternary_codes(3, 10, 100)
    assert np.array_equal(a, synth.ternary_codes(3, 10, 100))
    s = synth.row_scales(4, 10000)
    assert s.dtype == np.float32 and s.min() >= 0.01 and s.max() < 0.05
    x = synth.activations(5, 2, 100000)
    assert x.dtype == np.float16 and abs(float(x.astype(np.float64).std()) - 1.0) < 0.02
    w = synth.head_weights(6, 256, 4096)
    assert w.dtype == np.int8 and w.min() >= -127 and w.max() <= 127
    assert abs(float(w.astype(np.float64).std()) - 32.0) < 0.5
    p = synth.probe_activations(7, 3, 1000)
    assert set(np.abs(p.astype(np.int64)).reshape(-1).tolist()) <= set(range(1, 9))
    e = np.log2(synth.pow2_scales(8, 1000).astype(np.float64))
    assert np.array_equal(e, np.rint(e))


def test_seeds():
    assert synth.tensor_seed(0, "q") == 20260727
    assert synth.tensor_seed(1, "down") == 20260727 + 7 + 6
    assert synth.SEED_HEAD == 20260727 + 252
    assert synth.x_seed(3) == 20261730
