"""Shared test helpers: parity tolerances and golden-file readers.

The tolerance is the acceptance bound on floating-point outputs:
|y - y_ref| <= 1e-3 * s_r * sum_j |x_j| per element for the ternary GEMV
(codes have |c| <= 1), and 1e-3 * s_v * sum_j |w_vj| * |x_j| for the int8 head.
Any fp32-accumulating summation order meets it for K < ~16,000, since the
recursive summation error bound is about (K - 1) * 2**-24 of sum |terms|.
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-3


def ternary_bound(scale: np.ndarray, x: np.ndarray) -> np.ndarray:
    """Per-element bound [m, n] for ternary outputs."""
    xs = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return TOL * np.abs(xs).sum(axis=1)[:, None] * np.abs(scale.astype(np.float64))[None, :]


def head_bound(w: np.ndarray, scale: np.ndarray, x: np.ndarray) -> np.ndarray:
    xs = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return TOL * (np.abs(xs) @ np.abs(w.astype(np.float64)).T) * np.abs(scale.astype(np.float64))[None, :]


def assert_within(y, y_ref, bound, what=""):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    err = np.abs(y - y_ref)
    bad = ~(err <= bound)
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} elements outside tolerance; first {idx.tolist()}, "
            f"err {err[bad][:5].tolist()}, bound {np.broadcast_to(bound, err.shape)[bad][:5].tolist()}")


def read_format_words():
    """Rows of tests/golden/format_words.txt as (k, codes int8 [k], words uint32)."""
    rows = []
    with open(os.path.join(GOLDEN, "format_words.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k_s, codes_s, words_s = (p.strip() for p in line.split("|"))
            codes = np.array([int(v) for v in codes_s.split(",")], dtype=np.int8)
            words = np.array([int(v, 16) for v in words_s.split()], dtype=np.uint32)
            assert codes.size == int(k_s)
            rows.append((int(k_s), codes, words))
    return rows


def read_key_values(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (p.strip() for p in line.split("="))
            out[key] = int(val)
    return out
