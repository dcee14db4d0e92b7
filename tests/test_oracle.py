"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-derived word of the
layout (tests/golden/format_words.txt), a property of IEEE fp16 that the
layout is built around, exact rational arithmetic (fractions.Fraction),
Python's exactly rounded math.fsum, exact integer matmul, closed forms, or a
count printed on the Neutrino-1 8B model page.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from helpers import digit_probes, read_digits, read_format3_words, read_format_words, read_key_values

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------------
# Layout
# --------------------------------------------------------------------------
def test_words_per_row():
    assert oracle.words_per_row(1) == 4
    assert oracle.words_per_row(64) == 4
    assert oracle.words_per_row(65) == 8
    assert oracle.words_per_row(4096) == 256
    assert oracle.words_per_row(12288) == 768
    with pytest.raises(ValueError):
        oracle.words_per_row(0)


def test_bit_positions_cover_word_once():
    seen = [p for j in range(16) for p in oracle.bit_positions(j)]
    assert sorted(seen) == list(range(32))


@pytest.mark.parametrize("case", range(len(read_format_words())))
def test_golden_words(case):
    k, codes, words = read_format_words()[case]
    packed, row_sum, counts = oracle.pack(codes[None, :])
    assert packed.shape == (1, words.size)
    assert [f"{v:08X}" for v in packed[0]] == [f"{v:08X}" for v in words]
    assert np.array_equal(oracle.unpack(words[None, :], k)[0], codes)
    assert row_sum[0] == int(codes.astype(np.int64).sum())


def test_fp16_decode_property():
    """(word << 2t) & 0xC000C000, read as two fp16 values, equals
    (c[2t], c[2t+1]) * 2: bit 14/30 is the top fp16 exponent bit (2.0),
    bit 15/31 is the fp16 sign."""
    codes = synth.ternary_codes(11, 64, 256)
    packed, _, _ = oracle.pack(codes)
    words = packed.reshape(-1).astype(np.uint64)
    c = codes.reshape(-1, 16).astype(np.float64)
    for t in range(8):
        shifted = (words << np.uint64(2 * t)) & np.uint64(0xFFFFFFFF)
        m = (shifted & np.uint64(0xC000C000)).astype(np.uint32)
        halves = m.view(np.float16).reshape(-1, 2).astype(np.float64) / 2.0
        assert np.array_equal(halves[:, 0], c[:, 2 * t])
        assert np.array_equal(halves[:, 1], c[:, 2 * t + 1])


def test_fields_are_twos_complement():
    """Each 2-bit field (sign, nonzero) read as a two's-complement integer is the code."""
    codes = synth.ternary_codes(12, 8, 64)
    packed, _, _ = oracle.pack(codes)
    for j in range(16):
        nz, sg = oracle.bit_positions(j)
        assert sg == nz + 1
        field = (packed[:, 0::1] >> np.uint32(nz)) & np.uint32(3)
        val = np.where(field >= 2, field.astype(np.int64) - 4, field.astype(np.int64))
        assert np.array_equal(val, codes.reshape(8, 4, 16)[:, :, j])


@pytest.mark.slow
def test_exhaustive_single_word_round_trip():
    """All 3**16 code vectors of one word survive pack -> unpack, hence pack
    is injective on words; each pack output has only canonical fields."""
    n_all = 3 ** 16
    block = 3 ** 14
    digits = (np.arange(block, dtype=np.int64)[:, None] // (3 ** np.arange(14, dtype=np.int64))[None, :]) % 3
    low = (digits - 1).astype(np.int8)
    seen = 0
    for hi in itertools.product((-1, 0, 1), repeat=2):
        codes = np.empty((block, 16), dtype=np.int8)
        codes[:, :14] = low
        codes[:, 14] = hi[0]
        codes[:, 15] = hi[1]
        packed, _, _ = oracle.pack(codes)
        assert not np.any(packed[:, 1:])
        back = oracle.unpack(packed, 16)
        assert np.array_equal(back, codes)
        seen += block
    assert seen == n_all


def test_unpack_rejects_noncanonical_and_padding():
    k = 16
    for j in range(16):
        nz, sg = oracle.bit_positions(j)
        bad = np.zeros((1, 4), dtype=np.uint32)
        bad[0, 0] = np.uint32(1 << sg)
        with pytest.raises(ValueError):
            oracle.unpack(bad, k)
    pad = np.zeros((1, 4), dtype=np.uint32)
    pad[0, 1] = np.uint32(1 << 10)
    with pytest.raises(ValueError):
        oracle.unpack(pad, 16)


def test_pack_rejects_invalid_codes():
    codes = np.zeros((2, 8), dtype=np.int8)
    codes[1, 3] = 2
    with pytest.raises(ValueError):
        oracle.pack(codes)
    assert oracle.count_codes(codes).tolist() == [0, 15, 0, 1]


def test_row_sum_and_counts_from_bits():
    """row_sum = popcount(nonzero bits) - 2 * popcount(sign bits) per row, and
    the three counts add up to N*K and match a histogram of the codes."""
    codes = synth.ternary_codes(5, 37, 333)
    packed, row_sum, counts = oracle.pack(codes)
    nz_mask = sum(1 << oracle.bit_positions(j)[0] for j in range(16))
    sg_mask = sum(1 << oracle.bit_positions(j)[1] for j in range(16))
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))
    nz = pop(packed & np.uint32(nz_mask)).sum(axis=1)
    sg = pop(packed & np.uint32(sg_mask)).sum(axis=1)
    assert np.array_equal(row_sum.astype(np.int64), nz - 2 * sg)
    hist = np.bincount(codes.reshape(-1).astype(np.int64) + 1, minlength=3)
    assert counts.tolist() == hist.tolist()
    assert int(counts.sum()) == codes.size


# --------------------------------------------------------------------------
# Ternary GEMV arithmetic
# --------------------------------------------------------------------------
@pytest.mark.parametrize("k", [1, 2, 3, 5, 7, 8])
def test_brute_force_all_rows_exact(k):
    """Every ternary row of length k (3**k rows) against exact rational sums,
    rounded once by the scale multiply."""
    rows = np.array(list(itertools.product((-1, 0, 1), repeat=k)), dtype=np.int8)
    x = synth.activations(100 + k, 1, k)[0] * np.float16(3.0)
    s = synth.row_scales(200 + k, rows.shape[0])
    packed, _, _ = oracle.pack(rows)
    y = oracle.ternary_gemv(packed, s, k, x)
    xf = [Fraction(float(v)) for v in x]
    for r in range(rows.shape[0]):
        exact = sum((int(c) * xv for c, xv in zip(rows[r], xf)), Fraction(0))
        assert y[r] == float(Fraction(float(s[r])) * exact)


def test_fsum_exact_large_k():
    """Rows with K = 12288 against math.fsum (exactly rounded) of c_j * x_j."""
    k = 12288
    codes = synth.ternary_codes(7, 12, k)
    x = synth.activations(8, 1, k)[0]
    s = synth.row_scales(9, 12)
    packed, _, _ = oracle.pack(codes)
    y = oracle.ternary_gemv(packed, s, k, x)
    xd = x.astype(np.float64)
    for r in range(12):
        ref = math.fsum(float(c) * float(v) for c, v in zip(codes[r], xd))
        assert y[r] == float(s[r]) * ref


def test_closed_forms():
    k, n = 200, 200
    x = synth.activations(21, 1, k)[0]
    s = synth.row_scales(22, n)
    xd = x.astype(np.float64)
    zero = np.zeros((n, k), dtype=np.int8)
    assert np.all(oracle.ternary_gemv(oracle.pack(zero)[0], s, k, x) == 0.0)
    ones = np.ones((n, k), dtype=np.int8)
    assert np.allclose(oracle.ternary_gemv(oracle.pack(ones)[0], s, k, x),
                       s.astype(np.float64) * math.fsum(xd), rtol=1e-15, atol=0)
    eye = np.eye(n, k, dtype=np.int8)
    assert np.array_equal(oracle.ternary_gemv(oracle.pack(eye)[0], s, k, x), s.astype(np.float64) * xd)
    codes = synth.ternary_codes(23, n, k)
    y = oracle.ternary_gemv(oracle.pack(codes)[0], s, k, x)
    assert np.array_equal(oracle.ternary_gemv(oracle.pack(-codes)[0], s, k, x), -y)
    perm = np.random.Generator(np.random.PCG64(24)).permutation(k)
    assert np.array_equal(oracle.ternary_gemv(oracle.pack(codes[:, perm])[0], s, k, x[perm]), y)


def test_small_m_rows_equal_single_rows():
    k, n = 300, 50
    codes = synth.ternary_codes(31, n, k)
    s = synth.row_scales(32, n)
    xs = synth.activations(33, 8, k)
    packed = oracle.pack(codes)[0]
    ym = oracle.ternary_gemm_small(packed, s, k, xs)
    for m in range(8):
        assert np.array_equal(ym[m], oracle.ternary_gemv(packed, s, k, xs[m]))


def test_oracle_rejects_non_finite_activations():
    """Both sides require finite activations: the oracle raises on Inf or NaN
    (whether or not the column's codes are zero), and still accepts and sums
    exactly the largest finite fp16 values."""
    k, n = 64, 3
    codes = np.zeros((n, k), dtype=np.int8)
    codes[1, 5] = 1
    packed = oracle.pack(codes)[0]
    s = np.ones(n, dtype=np.float32)
    w = np.ones((n, k), dtype=np.int8)
    for bad in (np.inf, -np.inf, np.nan):
        x = np.zeros((2, k), dtype=np.float16)
        x[1, 0] = bad  # every code of column 0 is zero
        with pytest.raises(ValueError, match="finite"):
            oracle.ternary_gemm_small(packed, s, k, x)
        with pytest.raises(ValueError, match="finite"):
            oracle.ternary_gemv(packed, s, k, x[1])
        with pytest.raises(ValueError, match="finite"):
            oracle.int8_head_gemv(w, s, x)
        with pytest.raises(ValueError, match="finite"):
            oracle.int8_head_argmax(w, s, x)
    big = np.float16(65504.0)
    x = np.full(k, big, dtype=np.float16)
    x[7] = -big
    y = oracle.ternary_gemv(oracle.pack(np.ones((n, k), dtype=np.int8))[0], s, k, x)
    assert np.all(y == (k - 2) * 65504.0)


def test_digit_readback_recovers_codes():
    """The arithmetic path gives every code back: with x = 3^i on the 7
    columns of one block (zero elsewhere) and unit scales, y_r is that block's
    codes as a balanced-ternary integer, so reading the digits of y over all
    blocks must return the code matrix (a wrong code, sign, bit position or
    column anywhere changes a digit). The five-level codes read back the same
    way in balanced base 5 on blocks of 5 columns."""
    n = 23
    s = np.ones(n, dtype=np.float32)
    for k in (7, 60, 130):
        codes = synth.ternary_codes(61 + k, n, k)
        x, nd = digit_probes(k, 3)
        packed = oracle.pack(codes)[0]
        y = np.concatenate([oracle.ternary_gemm_small(packed, s, k, x[b:b + 8]) for b in range(0, len(x), 8)])
        assert np.array_equal(read_digits(y, 3, nd, k), codes)
        codes3 = synth.ternary3_codes(71 + k, n, k)
        x5, nd5 = digit_probes(k, 5)
        packed3 = oracle.pack3(codes3)[0]
        y5 = np.concatenate([oracle.ternary3_gemm_small(packed3, s, k, x5[b:b + 8]) for b in range(0, len(x5), 8)])
        assert np.array_equal(read_digits(y5, 5, nd5, k), codes3)


def test_integer_probe_exact():
    """Integer activations and power-of-two scales: y is an exact integer
    multiple of the scale, equal to the integer matmul."""
    k, n = 4096, 64
    codes = synth.ternary_codes(41, n, k)
    x = synth.probe_activations(42, 1, k)[0]
    s = synth.pow2_scales(43, n)
    y = oracle.ternary_gemv(oracle.pack(codes)[0], s, k, x)
    ref = codes.astype(np.int64) @ x.astype(np.int64)
    assert np.array_equal(y, ref.astype(np.float64) * s.astype(np.float64))


# --------------------------------------------------------------------------
# int8 head
# --------------------------------------------------------------------------
def test_head_integer_exact():
    n, k = 96, 4096
    w = synth.int8_full_range(51, n, k)
    x = synth.probe_activations(52, 3, k)
    s = synth.pow2_scales(53, n)
    y = oracle.int8_head_gemv(w, s, x)
    ref = x.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(y, ref.astype(np.float64) * s.astype(np.float64)[None, :])


def test_head_fsum():
    n, k = 10, 4096
    w = synth.head_weights(61, n, k)
    x = synth.activations(62, 1, k)[0]
    s = synth.row_scales(63, n)
    y = oracle.int8_head_gemv(w, s, x)[0]
    for r in range(n):
        ref = math.fsum(float(a) * float(b) for a, b in zip(w[r], x.astype(np.float64)))
        assert y[r] == float(s[r]) * ref


def test_head_chunking_invariant():
    n, k = 1000, 64
    w = synth.head_weights(71, n, k)
    x = synth.activations(72, 2, k)
    s = synth.row_scales(73, n)
    assert np.array_equal(oracle.int8_head_gemv(w, s, x, row_block=7), oracle.int8_head_gemv(w, s, x))


# --------------------------------------------------------------------------
# Geometry printed on the model page
# --------------------------------------------------------------------------
def test_geometry_matches_printed_parameter_count():
    g = read_key_values("neutrino_geometry.txt")
    coded = sum(n * k for n, k in synth.SHAPES.values()) * g["layers"]
    emb = 2 * g["vocab"] * g["hidden"]
    norms = g["layers"] * (2 * g["hidden"] + 2 * g["head_dim"]) + g["hidden"]
    assert g["layers"] * 4 + 1 == g["norm_tensors"]
    assert coded + emb + norms == g["parameters"]
    assert round(coded / 1e9, 2) == 6.95
    # The shipped lane is exactly 3 bits per coded weight; this layout is 2.
    assert g["shipped_coded_bytes_per_layer"] * 8 == 3 * (coded // g["layers"])
    packed_layer = sum(synth.words_bytes(n, k) for n, k in synth.SHAPES.values())
    assert packed_layer == 48234496
    assert synth.HEAD_SHAPE == (g["vocab"], g["hidden"])


# --------------------------------------------------------------------------
# Greedy argmax and embedding rows
# --------------------------------------------------------------------------
def test_argmax_ties_lowest_index():
    """Equal maxima resolve to the lowest row index."""
    k = 64
    w = np.zeros((10, k), dtype=np.int8)
    w[3, 0] = 5
    w[7, 0] = 5  # same logit as row 3
    w[9, 0] = 4
    s = np.ones(10, dtype=np.float32)
    x = np.zeros((2, k), dtype=np.float16)
    x[0, 0] = 1.0
    x[1, 0] = -1.0  # all logits <= 0: rows with 0 tie, lowest is row 0
    tok, y = oracle.int8_head_argmax(w, s, x)
    assert tok.tolist() == [3, 0]
    assert y[0, 3] == y[0, 7] == 5.0


def test_argmax_matches_scan():
    """Against a plain Python scan over exact integer logits."""
    n, k = 300, 128
    w = synth.int8_full_range(81, n, k)
    x = synth.probe_activations(82, 3, k)
    s = synth.pow2_scales(83, n)
    tok, _ = oracle.int8_head_argmax(w, s, x)
    for m in range(3):
        vals = [float(s[v]) * sum(int(a) * int(b) for a, b in zip(w[v], x[m].astype(np.int64))) for v in range(n)]
        best = 0
        for v in range(1, n):
            if vals[v] > vals[best]:
                best = v
        assert tok[m] == best


def test_embedding_rows_exact():
    """s_t * w_t rounded once to fp32, checked against Fraction arithmetic; out-of-range ids give NaN rows."""
    n, k = 50, 33
    table = synth.int8_full_range(84, n, k)
    s = synth.row_scales(85, n)
    tokens = np.array([0, 49, 7, 7, -1, 50])
    out = oracle.embedding_gather(table, s, tokens)
    for i, t in enumerate(tokens[:4]):
        for j in range(k):
            assert out[i, j] == np.float32(float(Fraction(float(s[t])) * int(table[t, j])))
    assert np.all(np.isnan(out[4:]))


# --------------------------------------------------------------------------
# Gated (SwiGLU) feed-forward block
# --------------------------------------------------------------------------
def test_silu_closed_forms():
    """sigmoid(ln 3) = 3/4 and sigmoid(0) = 1/2 fix silu at three points; silu(z) - silu(-z) = z."""
    l3 = math.log(3.0)
    z = np.array([0.0, l3, -l3])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 0.75 * l3) <= 1e-15
    assert abs(s[2] + 0.25 * l3) <= 1e-15
    zz = np.random.default_rng(5).normal(0, 6, 1000)
    np.testing.assert_allclose(oracle.silu(zz) - oracle.silu(-zz), zz, rtol=0, atol=1e-12)
    big = np.array([40.0, 700.0, -40.0, -745.0, -800.0])
    out = oracle.silu(big)
    assert out[0] == 40.0 and out[1] == 700.0  # 1 + e^-40 rounds to 1 in fp64
    assert abs(out[2]) < 1e-15 and abs(out[3]) < 1e-300 and out[4] == 0.0
    assert np.all(np.isfinite(out))


def test_silu_minimum_is_lambert_w():
    """silu has its minimum value -W(1/e) at z = -1 - W(1/e) (W: Lambert's function, from scipy)."""
    from scipy.special import lambertw

    w = float(lambertw(math.exp(-1.0)).real)
    z = np.linspace(-1.4, -1.1, 300001)
    s = oracle.silu(z)
    i = int(np.argmin(s))
    assert abs(s[i] + w) < 1e-11
    assert abs(z[i] - (-1.0 - w)) < 2e-6


def _ffn_probe(seed: int, d_model: int, d_ff: int):
    """Codes for which the block's result is known in integers.

    x is +-1. Gate row r has |S_r| codes equal to sign(x_j) (or all negated),
    so g_r = +-|S_r| with |S_r| >= 40 (scale 1). Up rows have at most 16
    nonzero codes, so u_r is an integer in [-16, 16]. silu(g) is then g to
    within g e^-g (positive rows) or below 1e-15 (negative rows), so
    h = g * u exactly (|h| <= 2048 is fp16-exact) or 0.
    """
    rng = np.random.default_rng(seed)
    x = rng.choice(np.array([-1.0, 1.0], dtype=np.float16), size=d_model)
    sx = np.where(x > 0, 1, -1).astype(np.int8)
    gate = np.zeros((d_ff, d_model), dtype=np.int8)
    up = np.zeros((d_ff, d_model), dtype=np.int8)
    h_exp = np.zeros(d_ff, dtype=np.int64)
    for r in range(d_ff):
        size = int(rng.integers(40, min(d_model, 120) + 1))
        cols = rng.choice(d_model, size=size, replace=False)
        neg = r % 5 == 3
        gate[r, cols] = -sx[cols] if neg else sx[cols]
        ucols = rng.choice(d_model, size=int(rng.integers(0, 17)), replace=False)
        up[r, ucols] = rng.choice(np.array([-1, 1], dtype=np.int8), size=ucols.size)
        u = int(np.dot(up[r].astype(np.int64), sx.astype(np.int64)))
        h_exp[r] = 0 if neg else size * u
    down = synth.ternary_codes(seed + 1, d_model, d_ff)
    return x, gate, up, down, h_exp


def test_ffn_integer_probe_exact():
    """h = g * u exactly and y = s_d * (C_down @ h) in exact integer arithmetic."""
    d_model, d_ff = 192, 136
    x, gate, up, down, h_exp = _ffn_probe(41, d_model, d_ff)
    one_f = np.ones(d_ff, dtype=np.float32)
    s_d = synth.pow2_scales(42, d_model)
    gp, _, _ = oracle.pack(gate)
    upk, _, _ = oracle.pack(up)
    dp, _, _ = oracle.pack(down)
    h, y = oracle.ffn_swiglu(gp, one_f, upk, one_f, dp, s_d, d_model, x)
    assert h.dtype == np.float16 and h.shape == (1, d_ff)
    assert np.array_equal(h[0].astype(np.float64), h_exp.astype(np.float64))
    assert np.count_nonzero(h_exp) > d_ff // 2
    y_exp = (down.astype(np.int64) @ h_exp).astype(np.float64) * s_d.astype(np.float64)
    assert np.array_equal(y[0], y_exp)


def test_ffn_gate_is_the_silu_input():
    """silu acts on the gate output, not on the up output: with g = ln 3 and u = 1, h = fp16(3/4 ln 3)."""
    d_model, d_ff = 64, 4
    x = np.zeros(d_model, dtype=np.float16)
    x[0] = 1.0
    gate = np.zeros((d_ff, d_model), dtype=np.int8)
    up = np.zeros((d_ff, d_model), dtype=np.int8)
    gate[:, 0] = 1
    up[:, 0] = 1
    gs = np.full(d_ff, math.log(3.0), dtype=np.float32)   # g = fp32(ln 3)
    us = np.array([1.0, 2.0, 0.5, -1.0], dtype=np.float32)  # u
    down = np.zeros((d_model, d_ff), dtype=np.int8)
    down[0, :] = 1
    h, y = oracle.ffn_swiglu(oracle.pack(gate)[0], gs, oracle.pack(up)[0], us, oracle.pack(down)[0],
                             np.ones(d_model, dtype=np.float32), d_model, x)
    want = np.float16(0.75 * math.log(3.0)) * us.astype(np.float64)
    assert np.array_equal(h[0].astype(np.float64), want.astype(np.float16).astype(np.float64))
    assert y[0, 0] == math.fsum(h[0].astype(np.float64)) and np.all(y[0, 1:] == 0)


def test_ffn_zero_gate_or_up_gives_zero():
    d_model, d_ff = 128, 70
    x = synth.activations(43, 1, d_model)[0]
    codes = synth.ternary_codes(44, d_ff, d_model)
    zeros = np.zeros_like(codes)
    down = synth.ternary_codes(45, d_model, d_ff)
    s = synth.row_scales(46, d_ff)
    sd = synth.row_scales(47, d_model)
    for g, u in ((zeros, codes), (codes, zeros)):
        h, y = oracle.ffn_swiglu(oracle.pack(g)[0], s, oracle.pack(u)[0], s, oracle.pack(down)[0], sd, d_model, x)
        assert np.all(h == 0) and np.all(y == 0)


def test_ffn_rows_independent():
    """M activation rows give the rows of M separate calls."""
    d_model, d_ff = 128, 80
    x = synth.activations(48, 3, d_model)
    g = oracle.pack(synth.ternary_codes(49, d_ff, d_model))[0]
    u = oracle.pack(synth.ternary_codes(50, d_ff, d_model))[0]
    d = oracle.pack(synth.ternary_codes(51, d_model, d_ff))[0]
    sg, su, sd = synth.row_scales(52, d_ff), synth.row_scales(53, d_ff), synth.row_scales(54, d_model)
    h, y = oracle.ffn_swiglu(g, sg, u, su, d, sd, d_model, x)
    for m in range(3):
        h1, y1 = oracle.ffn_swiglu(g, sg, u, su, d, sd, d_model, x[m])
        assert np.array_equal(h1[0], h[m]) and np.array_equal(y1[0], y[m])


# --------------------------------------------------------------------------
# The 3-bit variant (five-level codes: sign/nonzero plane + magnitude plane)
# --------------------------------------------------------------------------
def test_words_per_row3():
    assert oracle.words_per_row3(1) == 12
    assert oracle.words_per_row3(128) == 12
    assert oracle.words_per_row3(129) == 24
    assert oracle.words_per_row3(4096) == 384  # 1,536 bytes: 3 bits per code
    assert oracle.words_per_row3(12288) == 1152
    with pytest.raises(ValueError):
        oracle.words_per_row3(0)


def test_mag_bit_positions_cover_word_once():
    assert sorted(oracle.mag_bit_position(j) for j in range(32)) == list(range(32))


@pytest.mark.parametrize("case", range(len(read_format3_words())))
def test_golden_words3(case):
    k, codes, words = read_format3_words()[case]
    packed, row_sum, counts = oracle.pack3(codes[None, :])
    assert [f"{v:08X}" for v in packed[0]] == [f"{v:08X}" for v in words]
    assert np.array_equal(oracle.unpack3(words[None, :], k)[0], codes)
    assert row_sum[0] == int(codes.astype(np.int64).sum())
    assert counts.tolist() == [int(np.count_nonzero(codes == v)) for v in (-2, -1, 0, 1, 2)]


def test_page_bytes_per_layer_3bit():
    """The 3-bit rows reproduce the shipped lane's printed size exactly:
    72,351,744 bytes per layer and 2,605 MB for 36 layers."""
    g = read_key_values("neutrino_geometry.txt")
    layer = sum(4 * n * oracle.words_per_row3(k) for n, k in synth.SHAPES.values())
    assert layer == g["shipped_coded_bytes_per_layer"] == 72_351_744
    assert round(g["layers"] * layer / 1e6) == 2605


def test_fp16_reading_of_five_level_fields():
    """sign at bit 15, nonzero at 14, magnitude at 10, read as fp16, is 2c."""
    for c in (-2, -1, 0, 1, 2):
        bits = (int(c < 0) << 15) | (int(c != 0) << 14) | (int(abs(c) == 2) << 10)
        assert float(np.array([bits], dtype=np.uint16).view(np.float16)[0]) == 2.0 * c


def test_magnitude_shift_recipe():
    """The decode recipe the layout was chosen for: with M = m1:m0 the two
    magnitude words of a 64-code chunk, M << (10 - t) holds pair t of sign/
    nonzero word 0 at bits 10 and 26 of its low half and of word 2 in its
    high half; M shifted left by 2 - t (right by t - 2) does so for words 1
    and 3. Checked on random five-level codes against unpack3."""
    codes = synth.ternary3_codes(71, 32, 64)
    packed, _, _ = oracle.pack3(codes)
    c = oracle.unpack3(packed, 64)
    # k = 64 pads to 128 codes: sign/nonzero words 0..7, magnitude words 8..11; the
    # chunk of codes 0..63 is sign/nonzero words 0..3 with magnitude words 8, 9
    mags = packed[:, 8:10].astype(np.uint64)
    big = np.abs(c) == 2
    M = mags[:, 0] | (mags[:, 1] << np.uint64(32))
    mask = np.uint64(0xFFFFFFFFFFFFFFFF)
    for t in range(8):
        a = (M << np.uint64(10 - t)) & mask
        b = ((M << np.uint64(2 - t)) if t <= 2 else (M >> np.uint64(t - 2))) & mask
        for word, src, half in ((0, a, 0), (2, a, 1), (1, b, 0), (3, b, 1)):
            v = (src >> np.uint64(32 * half)) & np.uint64(0xFFFFFFFF)
            lo = ((v >> np.uint64(10)) & np.uint64(1)).astype(bool)
            hi = ((v >> np.uint64(26)) & np.uint64(1)).astype(bool)
            assert np.array_equal(lo, big[:, 16 * word + 2 * t]), (t, word)
            assert np.array_equal(hi, big[:, 16 * word + 2 * t + 1]), (t, word)


def test_round_trip3_single_codes_and_injective():
    """Every value at every position of a 128-code group (and past it) packs
    to its own bits and unpacks back; distinct rows pack to distinct words."""
    rows = []
    for j in list(range(128)) + [128, 200, 255]:
        for v in (-2, -1, 1, 2):
            r = np.zeros(256, dtype=np.int8)
            r[j] = v
            rows.append(r)
    codes = np.stack(rows)
    packed, _, _ = oracle.pack3(codes)
    assert np.array_equal(oracle.unpack3(packed, 256), codes)
    assert len({p.tobytes() for p in packed}) == len(rows)
    # each single code sets 1 (|c| = 1, +), 2 (sign) or 3 (|c| = 2) bits
    bits = np.array([sum(bin(int(w)).count("1") for w in p) for p in packed])
    expect = np.array([{-2: 3, -1: 2, 1: 1, 2: 2}[int(r[r != 0][0])] for r in codes])
    assert np.array_equal(bits, expect)


def test_round_trip3_exhaustive_six_positions():
    """All 5^6 value combinations at six positions spread over both halves,
    several pairs and both magnitude-word halves round-trip, injectively."""
    pos = [0, 1, 17, 30, 33, 127]
    vals = np.array(list(itertools.product((-2, -1, 0, 1, 2), repeat=len(pos))), dtype=np.int8)
    codes = np.zeros((vals.shape[0], 128), dtype=np.int8)
    codes[:, pos] = vals
    packed, row_sum, counts = oracle.pack3(codes)
    assert np.array_equal(oracle.unpack3(packed, 128), codes)
    assert len({p.tobytes() for p in packed}) == vals.shape[0]
    assert np.array_equal(row_sum, vals.astype(np.int64).sum(1))
    assert counts.sum() == codes.size


def test_pack3_of_ternary_codes_is_the_2bit_layout():
    """For codes in {-1, 0, +1} the sign/nonzero plane is the 2-bit layout and
    the magnitude plane is zero; doubling the codes sets the magnitude plane to
    the nonzero bits and doubles every output exactly."""
    n, k = 40, 4096
    c = synth.ternary_codes(72, n, k)
    p3, rs3, counts3 = oracle.pack3(c)
    p2, rs2, counts2 = oracle.pack(c)
    assert np.array_equal(p3[:, :256], p2) and not np.any(p3[:, 256:])
    assert np.array_equal(rs3, rs2) and counts3.tolist() == [0, counts2[0], counts2[1], counts2[2], 0]
    s = synth.row_scales(73, n)
    x = synth.activations(74, 1, k)[0]
    y1 = oracle.ternary3_gemv(p3, s, k, x)
    assert np.array_equal(y1, oracle.ternary_gemv(p2, s, k, x))
    pd, _, _ = oracle.pack3((2 * c).astype(np.int8))
    assert np.array_equal(pd[:, :256], p2)
    nzmask = np.array([[int(any(c[r, 32 * q: 32 * q + 32] != 0)) for q in range(128)] for r in range(n)])
    assert np.array_equal(pd[:, 256:] != 0, nzmask.astype(bool))
    assert np.array_equal(oracle.ternary3_gemv(pd, s, k, x), 2.0 * y1)


@pytest.mark.parametrize("k", [1, 2, 3, 5])
def test_brute_force3_all_rows_exact(k):
    """Every five-level row of length k against exact rational sums rounded once."""
    rows = np.array(list(itertools.product((-2, -1, 0, 1, 2), repeat=k)), dtype=np.int8)
    x = synth.activations(80 + k, 1, k)[0]
    s = np.full(rows.shape[0], 0.03125, dtype=np.float32)
    y = oracle.ternary3_gemv(oracle.pack3(rows)[0], s, k, x)
    xf = [Fraction(float(v)) for v in x]
    for r in range(rows.shape[0]):
        exact = sum((int(c) * xv for c, xv in zip(rows[r], xf)), Fraction(0)) * Fraction(float(s[r]))
        assert y[r] == float(exact)


def test_fsum3_exact_large_k():
    k, n = 12288, 6
    codes = synth.ternary3_codes(81, n, k)
    x = synth.activations(82, 1, k)[0]
    s = synth.row_scales(83, n)
    y = oracle.ternary3_gemv(oracle.pack3(codes)[0], s, k, x)
    for r in range(n):
        ref = math.fsum(float(c) * float(v) for c, v in zip(codes[r], x))
        assert y[r] == float(s[r]) * ref


def test_unpack3_rejects_noncanonical_and_padding():
    codes = np.zeros((1, 40), dtype=np.int8)
    codes[0, 3] = 2
    p, _, _ = oracle.pack3(codes)
    bad = p.copy()
    bad[0, 8] |= np.uint32(1 << oracle.mag_bit_position(5))  # magnitude bit on a zero code
    with pytest.raises(ValueError, match="magnitude"):
        oracle.unpack3(bad, 40)
    bad = p.copy()
    bad[0, 0] |= np.uint32(1 << oracle.bit_positions(6)[1])  # sign bit without nonzero
    with pytest.raises(ValueError):
        oracle.unpack3(bad, 40)
    bad = p.copy()
    bad[0, 3] |= np.uint32(1 << oracle.bit_positions(0)[0])  # code 48 sits in the padding
    with pytest.raises(ValueError, match="padding"):
        oracle.unpack3(bad, 40)
    with pytest.raises(ValueError):
        oracle.pack3(np.array([[3, 0]], dtype=np.int8))
    x = np.zeros(40, dtype=np.float16)
    x[2] = np.inf
    with pytest.raises(ValueError, match="finite"):
        oracle.ternary3_gemv(p, np.ones(1, dtype=np.float32), 40, x)


def test_row_sums_and_counts3():
    codes = synth.ternary3_codes(84, 50, 1000)
    _, row_sum, counts = oracle.pack3(codes)
    assert np.array_equal(row_sum, codes.astype(np.int64).sum(1))
    assert counts.sum() == codes.size
    hist = np.bincount((codes.astype(np.int64) + 2).ravel(), minlength=5)
    assert counts.tolist() == hist.tolist()


# --------------------------------------------------------------------------
# The feed-forward block in the 3-bit layout
# --------------------------------------------------------------------------
def test_ffn3_on_ternary_codes_is_the_2bit_block():
    """Codes in {-1, 0, +1} packed in the 3-bit layout give the 2-bit block's h and y bit for bit."""
    d_model, d_ff = 192, 136
    x = synth.activations(60, 2, d_model)
    g, u = synth.ternary_codes(61, d_ff, d_model), synth.ternary_codes(62, d_ff, d_model)
    d = synth.ternary_codes(63, d_model, d_ff)
    sg, su, sd = synth.row_scales(64, d_ff), synth.row_scales(65, d_ff), synth.row_scales(66, d_model)
    h2, y2 = oracle.ffn_swiglu(oracle.pack(g)[0], sg, oracle.pack(u)[0], su, oracle.pack(d)[0], sd, d_model, x)
    h3, y3 = oracle.ffn3_swiglu(oracle.pack3(g)[0], sg, oracle.pack3(u)[0], su, oracle.pack3(d)[0], sd, d_model, x)
    assert np.array_equal(h2, h3) and np.array_equal(y2, y3)


def test_ffn3_doubled_codes_equal_doubled_scales():
    """Codes 2c in the 3-bit layout with scale s equal codes c with scale 2s (exact in fp32), in each of the
    three linears at once: a dropped or misplaced magnitude anywhere in the block breaks the equality."""
    d_model, d_ff = 256, 200
    x = synth.activations(67, 3, d_model)
    g, u = synth.ternary_codes(68, d_ff, d_model), synth.ternary_codes(69, d_ff, d_model)
    d = synth.ternary_codes(70, d_model, d_ff)
    sg, su, sd = synth.row_scales(71, d_ff), synth.row_scales(72, d_ff), synth.row_scales(73, d_model)
    h2, y2 = oracle.ffn_swiglu(oracle.pack(g)[0], 2 * sg, oracle.pack(u)[0], su, oracle.pack(d)[0], 2 * sd,
                               d_model, x)
    h3, y3 = oracle.ffn3_swiglu(oracle.pack3(2 * g)[0], sg, oracle.pack3(u)[0], su, oracle.pack3(2 * d)[0], sd,
                                d_model, x)
    assert np.array_equal(h2, h3) and np.array_equal(y2, y3)
    # and the doubled up linear doubles h: silu(g) * 2u rounds to fp16 as twice the rounding of silu(g) * u
    # wherever both are normal fp16 numbers (below 2^-14 the rounding step no longer scales with the value)
    h4, _ = oracle.ffn3_swiglu(oracle.pack3(g)[0], sg, oracle.pack3(2 * u)[0], su, oracle.pack3(d)[0], sd, d_model, x)
    h1, _ = oracle.ffn3_swiglu(oracle.pack3(g)[0], sg, oracle.pack3(u)[0], su, oracle.pack3(d)[0], sd, d_model, x)
    normal = np.abs(h1.astype(np.float64)) >= 2.0 ** -14
    assert normal.mean() > 0.9
    assert np.array_equal(h4.astype(np.float64)[normal], 2 * h1.astype(np.float64)[normal])


def test_ffn3_integer_probe_exact():
    """Five-level probe: the 2-bit probe with the gate codes of rows r = 0 mod 3 and the up codes of rows
    r = 1 mod 4 doubled, so g = +-2|S_r| or +-|S_r| (|g| >= 40) and u is an integer; h = g * u (rounded
    once to fp16) or 0, and y = s_d * (C_down @ h) with five-level down codes, all in exact integers."""
    d_model, d_ff = 192, 136
    x, gate, up, _, h2 = _ffn_probe(74, d_model, d_ff)
    r = np.arange(d_ff)
    gmul = np.where(r % 3 == 0, 2, 1)
    umul = np.where(r % 4 == 1, 2, 1)
    gate3 = (gate.astype(np.int16) * gmul[:, None]).astype(np.int8)
    up3 = (up.astype(np.int16) * umul[:, None]).astype(np.int8)
    down3 = synth.ternary3_codes(75, d_model, d_ff)
    h_exp = (h2 * gmul * umul).astype(np.float16).astype(np.float64)
    one_f = np.ones(d_ff, dtype=np.float32)
    s_d = synth.pow2_scales(76, d_model)
    h, y = oracle.ffn3_swiglu(oracle.pack3(gate3)[0], one_f, oracle.pack3(up3)[0], one_f, oracle.pack3(down3)[0], s_d,
                              d_model, x)
    assert np.array_equal(h[0].astype(np.float64), h_exp)
    assert np.count_nonzero(np.abs(down3) == 2) > 0 and np.count_nonzero(h_exp) > d_ff // 2
    y_exp = (down3.astype(np.int64) @ h_exp.astype(np.int64)).astype(np.float64) * s_d.astype(np.float64)
    assert np.array_equal(y[0], y_exp)
