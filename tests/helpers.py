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


def head_bound(w: np.ndarray, scale: np.ndarray, x: np.ndarray, row_block: int = 16384) -> np.ndarray:
    """Per-element bound [m, n] for int8 head outputs (rows in blocks to bound memory)."""
    xs = np.abs(np.atleast_2d(np.asarray(x, dtype=np.float64)))
    out = np.empty((xs.shape[0], w.shape[0]), dtype=np.float64)
    for r0 in range(0, w.shape[0], row_block):
        r1 = min(w.shape[0], r0 + row_block)
        out[:, r0:r1] = TOL * (xs @ np.abs(w[r0:r1].astype(np.float64)).T) * np.abs(
            scale[r0:r1].astype(np.float64))[None, :]
    return out


def ternary3_bound(codes: np.ndarray, scale: np.ndarray, x: np.ndarray, row_block: int = 16384) -> np.ndarray:
    """Per-element bound [m, n] for five-level outputs: 1e-3 * s_r * sum_j |c_rj| |x_j|."""
    return head_bound(codes, scale, x, row_block)


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


def read_format3_words():
    """Rows of tests/golden/format3_words.txt as (k, codes int8 [k], words uint32).

    Codes may be written "a*n" for n copies of a."""
    rows = []
    with open(os.path.join(GOLDEN, "format3_words.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k_s, codes_s, words_s = (p.strip() for p in line.split("|"))
            vals = []
            for item in codes_s.split(","):
                if "*" in item:
                    v, cnt = item.split("*")
                    vals += [int(v)] * int(cnt)
                else:
                    vals.append(int(item))
            codes = np.array(vals, dtype=np.int8)
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


def ffn_probe(seed: int, d_model: int, d_ff: int):
    """Integer probe of the gated feed-forward block (d_model a multiple of 64).

    x is +-1. Gate row r has size_r in [40, 120] nonzero codes, at columns
    (37 r + 7 t) mod d_model, equal to sign(x_j) (negated on rows r = 3 mod 5),
    so g_r = +-size_r exactly with scale 1. Up row r has at most 16 codes +-1
    at columns (13 r + 11 t + 5) mod d_model, so u_r is an integer in
    [-16, 16]. For g >= 40, 1 + e^-g rounds to 1 in fp32 and fp64 alike, so
    silu(g) * u = g * u; for g <= -40 the product is below 1e-15 and rounds to
    0 in fp16. Returns (x fp16, gate int8, up int8, h int64).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.choice(np.array([-1.0, 1.0]), size=d_model).astype(np.float16)
    sx = np.where(x > 0, 1, -1).astype(np.int64)
    r = np.arange(d_ff)
    size = rng.integers(40, min(d_model, 120) + 1, size=d_ff)
    usize = rng.integers(0, 17, size=d_ff)
    neg = (r % 5) == 3
    t = np.arange(120)
    cols = (37 * r[:, None] + 7 * t[None, :]) % d_model
    mask = t[None, :] < size[:, None]
    rows = np.broadcast_to(r[:, None], cols.shape)
    sign = np.where(neg, -1, 1)[:, None]
    gate = np.zeros((d_ff, d_model), dtype=np.int8)
    gate[rows[mask], cols[mask]] = (np.broadcast_to(sign, cols.shape) * sx[cols])[mask].astype(np.int8)
    tu = np.arange(16)
    ucols = (13 * r[:, None] + 11 * tu[None, :] + 5) % d_model
    umask = tu[None, :] < usize[:, None]
    usign = rng.choice(np.array([-1, 1]), size=ucols.shape)
    up = np.zeros((d_ff, d_model), dtype=np.int8)
    urows = np.broadcast_to(r[:, None], ucols.shape)
    up[urows[umask], ucols[umask]] = usign[umask].astype(np.int8)
    u = np.where(umask, usign * sx[ucols], 0).sum(axis=1)
    h = np.where(neg, 0, size * u).astype(np.int64)
    return x, gate, up, h


def swiglu_h_bound(silu_g: np.ndarray, u: np.ndarray, tg: np.ndarray, tu: np.ndarray) -> np.ndarray:
    """Bound on |h - h_ref| for h = fp16(silu(g) * u) when the kernel's g and u
    are within tg and tu of the exact values: silu has slope at most 1.1, the
    fp32 exp and reciprocal add at most 1e-6 relative, and two fp16 roundings of
    values that close differ by at most their distance plus one fp16 ulp."""
    a = 1.1 * tg * (np.abs(u) + tu) + np.abs(silu_g) * tu + 1e-6 * np.abs(silu_g * u)
    mag = np.abs(silu_g * u) + a
    ulp = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -14))) - 10), 2.0 ** -24)
    return a + ulp


def digit_probes(k: int, base: int) -> tuple[np.ndarray, int]:
    """Read-back activations: the codes of a row are balanced base-`base`
    digits (-(base-1)/2 .. (base-1)/2), so with x = base^i on the `nd` columns
    of one block (zero elsewhere) y_r is the integer whose digits are the
    block's codes. nd is the largest count whose powers stay fp16-exact
    integers (3^6 = 729, 5^4 = 625) and whose sums stay below 2^11. Returns
    (x [blocks, k] fp16, nd); block b covers columns nd*b .. nd*b + nd - 1."""
    nd = {3: 7, 5: 5}[base]
    blocks = (k + nd - 1) // nd
    x = np.zeros((blocks, k), dtype=np.float16)
    for b in range(blocks):
        for i in range(nd):
            if nd * b + i < k:
                x[b, nd * b + i] = float(base ** i)
    return x, nd


def read_digits(y: np.ndarray, base: int, nd: int, k: int) -> np.ndarray:
    """Inverse of digit_probes: y [blocks, n] (exact integers, unit scale) ->
    codes [n, k] as int8, digit i of block b being column nd*b + i."""
    half = (base - 1) // 2
    v = np.rint(y).astype(np.int64)
    assert np.array_equal(v.astype(np.float64), np.asarray(y, dtype=np.float64)), "not an integer"
    blocks, n = v.shape
    out = np.zeros((n, blocks * nd), dtype=np.int8)
    for i in range(nd):
        d = (v + half) % base - half
        out[:, i::nd] = d.T
        v = (v - d) // base
    assert not v.any(), "more digits than a block holds"
    return out[:, :k]
