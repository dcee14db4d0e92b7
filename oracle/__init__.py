"""CPU oracle for the packed ternary GEMV path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it, to check the HIP kernels and to
time a plain CPU baseline. It shares no code, header, table or constant
generator with the HIP library, and it imports nothing from it.

What it computes (Neutrino-1 8B model page, English text on bittide):

* Every transformer linear is stored as ternary codes c in {-1, 0, +1} with a
  scale and a row sum per row, and the kernels expand the codes themselves
  while multiplying (introduction; "Where the bytes live"; "Inside the coded lane").
  The page calls the encoding proprietary and never specifies it, so the bit
  layout below is this project's own (2 bits per code, 16 codes per uint32).
  Its definition is stated here in words, once, and nowhere else in Python.
* A linear applied to one activation row x is y_r = s_r * sum_j c_rj * x_j.
* The untied output head is an int8 tensor with a per-row scale
  ("Where the bytes live"): y_v = s_v * sum_j w_vj * x_j.
* Speculative decoding ("speculative" section) checks a run of drafted
  tokens with one pass of the large model, so the same products run on M
  activation rows; acceptance compares each drafted token with the large
  model's greedy choice, taken here as the index of the row's largest head
  logit (the lowest index among equal maxima).
* The int8 input embedding has a per-row scale and is read one row per token
  ("Where the bytes live"): the embedding of token t is s_t * w_t.
* The feed-forward block is gated (SwiGLU) with three linears per layer
  (geometry table): h = silu(gate x) * (up x), rounded to fp16, then down h.
  The page names the gate but not its formula; silu(z) = z * sigmoid(z) is
  the usual reading. The same block is also computed with the three linears
  in the 3-bit layout below (ffn3_swiglu).

Bit layout of one 32-bit word (little-endian uint32) holding 16 codes:
  code j (0..15) belongs to pair t = j // 2 and half h = j % 2;
  its NONZERO bit is bit 16*h + 14 - 2*t,
  its SIGN bit    is bit 16*h + 15 - 2*t;
  i.e. each 16-bit half holds 8 two-bit fields, highest field first (even
  codes in the low half, odd codes in the high half), and a field read as a
  2-bit two's-complement integer is the code:
  +1 -> nonzero=1, sign=0;  -1 -> nonzero=1, sign=1;  0 -> both bits 0.
  The pattern sign=1, nonzero=0 (-2) is never written; unpacking rejects it.
Row layout: row r holds W = 4 * ceil(K / 64) words; word w holds the codes of
columns 16*w .. 16*w + 15; codes past column K - 1 are 0 (row padding, so a
row is a whole number of 16-byte chunks).

Activations must be finite (Inf and NaN raise ValueError): the product of a
zero code and a non-finite activation is left undefined, as the library's
header requires finite activations of its callers.

Arithmetic: activations arrive as fp16 and are widened to fp64 exactly; codes
and int8 weights are exact in fp64; the matrix-vector product is a float64
matmul and the scale multiplies the finished sum. fp16 values are integer
multiples of 2**-24, so with |x| < 2**9 and K < 2**20 every partial sum is an
integer multiple of 2**-24 below 2**53 * 2**-24 and the fp64 sum is exact in
any order; the only rounding is the final multiply by the scale.

The 3-bit variant (five-level codes). The page sizes the shipped coded lane
at exactly 3 bits per weight ("Where the bytes live") and splits its codes into
zero, plus and minus ("Inside the coded lane"); this project reads the third
bit as a magnitude: codes c in {-2, -1, 0, +1, +2}, y_r = s_r * sum_j c_rj x_j.
Its layout, in words (once, here):
  a row of K codes is padded with zero codes to K128 = 128 * ceil(K / 128) and
  holds 12 * ceil(K / 128) words: first the sign/nonzero plane, K128 / 16
  words in exactly the 2-bit layout above (a code of magnitude 2 is written
  there like one of magnitude 1), then the magnitude plane, K128 / 32 words:
  magnitude word q covers codes 32q .. 32q + 31, and code 32q + j, with
  j = 16 i + 2 t + h (i = 0, 1; t = 0..7; h = 0, 1), sits at bit 16 h + 8 i + t,
  set exactly when |c| = 2. A magnitude bit without its nonzero bit is
  rejected on unpacking, like a sign bit without it.

Parity pins: see tests/test_oracle.py (exhaustive single-word round trip,
hand-written format words, the fp16 reading of the layout, brute force
over all ternary rows for K <= 8 against exact rational sums, closed forms,
exact integer matmul for the head, the row-sum and count invariants, silu at
closed-form points and its Lambert-W minimum, an integer SwiGLU probe; for
the 3-bit feed-forward block, its equality with the 2-bit block on ternary
codes, the doubled-codes / doubled-scales identity and a five-level integer
probe).
"""
from __future__ import annotations

import math

import numpy as np

CODES_PER_WORD = 16


def words_per_row(k: int) -> int:
    """Words per packed row: 4 * ceil(k / 64), i.e. whole 16-byte chunks."""
    if k <= 0:
        raise ValueError("k must be positive")
    return 4 * math.ceil(k / 64)


def bit_positions(j: int) -> tuple[int, int]:
    """(nonzero bit, sign bit) of code j (0..15) inside its word."""
    if not 0 <= j < CODES_PER_WORD:
        raise ValueError("code index within a word is 0..15")
    t, h = divmod(j, 2)
    return 16 * h + 14 - 2 * t, 16 * h + 15 - 2 * t


def count_codes(codes: np.ndarray) -> np.ndarray:
    """[n_minus, n_zero, n_plus, n_invalid] over a whole code tensor (int64)."""
    c = np.asarray(codes)
    n_minus = int(np.count_nonzero(c == -1))
    n_zero = int(np.count_nonzero(c == 0))
    n_plus = int(np.count_nonzero(c == 1))
    return np.array([n_minus, n_zero, n_plus, c.size - n_minus - n_zero - n_plus], dtype=np.int64)


def pack(codes: np.ndarray):
    """Pack int8 codes [n, k] (values -1, 0, +1) into the 2-bit layout.

    Returns (packed uint32 [n, W], row_sum int32 [n], counts int64[3] =
    n_minus, n_zero, n_plus). Raises ValueError on any other code value.
    Row sums and counts are the per-row metadata and the per-tensor code
    occupancy (Neutrino-1 8B page: "Where the bytes live", "Inside the coded
    lane").
    """
    codes = np.asarray(codes)
    if codes.ndim != 2 or codes.dtype != np.int8:
        raise ValueError("codes must be a 2-D int8 array")
    n, k = codes.shape
    stats = count_codes(codes)
    if stats[3] != 0:
        raise ValueError(f"{stats[3]} codes outside {{-1, 0, +1}}")
    w = words_per_row(k)
    padded = np.zeros((n, w * CODES_PER_WORD), dtype=np.int8)
    padded[:, :k] = codes
    grouped = padded.reshape(n, w, CODES_PER_WORD)
    packed = np.zeros((n, w), dtype=np.uint32)
    for j in range(CODES_PER_WORD):
        nz_bit, sign_bit = bit_positions(j)
        c = grouped[:, :, j]
        packed |= (c != 0).astype(np.uint32) << np.uint32(nz_bit)
        packed |= (c < 0).astype(np.uint32) << np.uint32(sign_bit)
    row_sum = codes.sum(axis=1, dtype=np.int64).astype(np.int32)
    return packed, row_sum, stats[:3].copy()


def unpack(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of pack: uint32 [n, W] -> int8 codes [n, k].

    Raises ValueError on a field with sign=1 and nonzero=0, on a row length
    that does not match k, or on a nonzero padding code.
    """
    packed = np.asarray(packed)
    if packed.ndim != 2 or packed.dtype != np.uint32:
        raise ValueError("packed must be a 2-D uint32 array")
    n, w = packed.shape
    if w != words_per_row(k):
        raise ValueError(f"row holds {w} words, k={k} needs {words_per_row(k)}")
    out = np.zeros((n, w, CODES_PER_WORD), dtype=np.int8)
    for j in range(CODES_PER_WORD):
        nz_bit, sign_bit = bit_positions(j)
        nz = (packed >> np.uint32(nz_bit)) & np.uint32(1)
        sg = (packed >> np.uint32(sign_bit)) & np.uint32(1)
        if np.any(sg & ~nz & np.uint32(1)):
            raise ValueError("field with sign set and nonzero clear")
        out[:, :, j] = nz.astype(np.int8) * (1 - 2 * sg.astype(np.int8))
    flat = out.reshape(n, w * CODES_PER_WORD)
    if np.any(flat[:, k:]):
        raise ValueError("nonzero padding code")
    return flat[:, :k].copy()


def _as_rows(x: np.ndarray, k: int) -> np.ndarray:
    """fp16 activations [k] or [m, k] widened exactly to fp64 rows [m, k].

    Activations must be finite: a product against them is defined only for
    finite values here (a zero code against Inf would otherwise have to pick
    between 0 and NaN, and the pages say nothing about it), so Inf or NaN is
    rejected with ValueError rather than given a meaning.
    """
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise ValueError("activations are fp16")
    if x.ndim == 1:
        x = x[None, :]
    if x.ndim != 2 or x.shape[1] != k:
        raise ValueError(f"activations must be [m, {k}]")
    if not np.all(np.isfinite(x)):
        raise ValueError("activations must be finite")
    return x.astype(np.float64)


def ternary_gemm_small(packed: np.ndarray, scale: np.ndarray, k: int, x: np.ndarray,
                       row_block: int = 16384) -> np.ndarray:
    """Y[m, r] = s_r * sum_j c_rj * X[m, j] in fp64, for M activation rows.

    Unpacks the codes (in row blocks to bound memory), widens them and X to
    fp64, multiplies, then applies the per-row scale.
    """
    xs = _as_rows(x, k)
    scale = np.asarray(scale)
    if scale.dtype != np.float32 or scale.shape != (packed.shape[0],):
        raise ValueError("scale must be fp32 [n]")
    n = packed.shape[0]
    y = np.empty((xs.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        c = unpack(packed[r0:r1], k).astype(np.float64)
        sums = xs @ c.T
        y[:, r0:r1] = sums * scale[r0:r1].astype(np.float64)[None, :]
    return y


def ternary_gemv(packed: np.ndarray, scale: np.ndarray, k: int, x: np.ndarray) -> np.ndarray:
    """y_r = s_r * sum_j c_rj * x_j in fp64 (one activation row, M = 1)."""
    x = np.asarray(x)
    if x.ndim != 1:
        raise ValueError("ternary_gemv takes one activation row")
    return ternary_gemm_small(packed, scale, k, x[None, :])[0]


def int8_head_gemv(w: np.ndarray, scale: np.ndarray, x: np.ndarray, row_block: int = 8192) -> np.ndarray:
    """Y[m, v] = s_v * sum_j w_vj * X[m, j] in fp64 (int8 head with per-row scales)."""
    w = np.asarray(w)
    if w.ndim != 2 or w.dtype != np.int8:
        raise ValueError("head weights must be a 2-D int8 array")
    n, k = w.shape
    xs = _as_rows(x, k)
    scale = np.asarray(scale)
    if scale.dtype != np.float32 or scale.shape != (n,):
        raise ValueError("scale must be fp32 [n]")
    y = np.empty((xs.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        sums = xs @ w[r0:r1].astype(np.float64).T
        y[:, r0:r1] = sums * scale[r0:r1].astype(np.float64)[None, :]
    return y


def int8_head_argmax(w: np.ndarray, scale: np.ndarray, x: np.ndarray):
    """Greedy token of each activation row: (argmax_v y[m, v] with the lowest
    index among equal maxima, the fp64 logits y [m, n])."""
    y = int8_head_gemv(w, scale, x)
    return np.argmax(y, axis=1).astype(np.int64), y


def embedding_gather(table: np.ndarray, scale: np.ndarray, tokens: np.ndarray) -> np.ndarray:
    """Rows s_t * w_t of an int8 table with per-row scales, for token ids t.

    The product of an fp32 scale and an int8 value is exact in fp64; it is
    rounded once to fp32. Token ids outside [0, n) give a row of NaN.
    """
    table = np.asarray(table)
    if table.ndim != 2 or table.dtype != np.int8:
        raise ValueError("table must be a 2-D int8 array")
    n, k = table.shape
    scale = np.asarray(scale)
    if scale.dtype != np.float32 or scale.shape != (n,):
        raise ValueError("scale must be fp32 [n]")
    tokens = np.asarray(tokens).astype(np.int64).reshape(-1)
    out = np.full((tokens.size, k), np.nan, dtype=np.float32)
    for i, t in enumerate(tokens):
        if 0 <= t < n:
            out[i] = (np.float64(scale[t]) * table[t].astype(np.float64)).astype(np.float32)
    return out


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) in fp64, written so that neither branch overflows."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    e = np.exp(z[~pos])
    out[~pos] = z[~pos] * e / (1.0 + e)
    return out


def ffn_swiglu(gate_packed: np.ndarray, gate_scale: np.ndarray, up_packed: np.ndarray, up_scale: np.ndarray,
               down_packed: np.ndarray, down_scale: np.ndarray, d_model: int, x: np.ndarray):
    """The gated feed-forward block of one layer on M activation rows.

    The geometry table of the Neutrino-1 8B model page gives the feed-forward
    block as gated (SwiGLU) with three linears per layer. Read as usual:
    g = gate x, u = up x (both ternary linears with per-row scales),
    h = silu(g) * u, y = down h. h is the activation the down linear
    consumes, so it is rounded once to fp16 like every other linear input.
    Returns (h fp16 [m, d_ff], y fp64 [m, d_model]).
    """
    d_ff = gate_packed.shape[0]
    if up_packed.shape[0] != d_ff or down_packed.shape[0] != d_model:
        raise ValueError("gate and up are [d_ff, .], down is [d_model, .]")
    g = ternary_gemm_small(gate_packed, gate_scale, d_model, x)
    u = ternary_gemm_small(up_packed, up_scale, d_model, x)
    h = (silu(g) * u).astype(np.float16)
    y = ternary_gemm_small(down_packed, down_scale, d_ff, h)
    return h, y


# --------------------------------------------------------------------------
# The 3-bit variant: five-level codes as a sign/nonzero plane (the 2-bit
# layout) followed by a magnitude plane.
# --------------------------------------------------------------------------
CODES_PER_MAG_WORD = 32


def words_per_row3(k: int) -> int:
    """Words per 3-bit row: 12 * ceil(k / 128) (3 bits per code, 128-code groups)."""
    if k <= 0:
        raise ValueError("k must be positive")
    return 12 * math.ceil(k / 128)


def mag_bit_position(j: int) -> int:
    """Bit of code j (0..31) inside its magnitude word."""
    if not 0 <= j < CODES_PER_MAG_WORD:
        raise ValueError("code index within a magnitude word is 0..31")
    i, rest = divmod(j, 16)
    t, h = divmod(rest, 2)
    return 16 * h + 8 * i + t


def count_codes3(codes: np.ndarray) -> np.ndarray:
    """[n(-2), n(-1), n(0), n(+1), n(+2), n_invalid] over a code tensor (int64)."""
    c = np.asarray(codes)
    counts = [int(np.count_nonzero(c == v)) for v in (-2, -1, 0, 1, 2)]
    return np.array(counts + [c.size - sum(counts)], dtype=np.int64)


def pack3(codes: np.ndarray):
    """Pack int8 codes [n, k] with values -2..+2 into the 3-bit layout.

    Returns (packed uint32 [n, words_per_row3(k)], row_sum int32 [n],
    counts int64[5] of -2, -1, 0, +1, +2). Raises ValueError on any other value.
    """
    codes = np.asarray(codes)
    if codes.ndim != 2 or codes.dtype != np.int8:
        raise ValueError("codes must be a 2-D int8 array")
    n, k = codes.shape
    stats = count_codes3(codes)
    if stats[5] != 0:
        raise ValueError(f"{stats[5]} codes outside -2..+2")
    k128 = 128 * math.ceil(k / 128)
    padded = np.zeros((n, k128), dtype=np.int8)
    padded[:, :k] = codes
    # sign/nonzero plane: the 2-bit layout of sign(c) (magnitude 2 written as 1)
    sign_nz = np.sign(padded).astype(np.int8)
    plane2 = np.zeros((n, k128 // CODES_PER_WORD), dtype=np.uint32)
    grouped = sign_nz.reshape(n, -1, CODES_PER_WORD)
    for j in range(CODES_PER_WORD):
        nz_bit, sign_bit = bit_positions(j)
        c = grouped[:, :, j]
        plane2 |= (c != 0).astype(np.uint32) << np.uint32(nz_bit)
        plane2 |= (c < 0).astype(np.uint32) << np.uint32(sign_bit)
    # magnitude plane
    plane_m = np.zeros((n, k128 // CODES_PER_MAG_WORD), dtype=np.uint32)
    big = (np.abs(padded) == 2).reshape(n, -1, CODES_PER_MAG_WORD)
    for j in range(CODES_PER_MAG_WORD):
        plane_m |= big[:, :, j].astype(np.uint32) << np.uint32(mag_bit_position(j))
    packed = np.concatenate([plane2, plane_m], axis=1)
    assert packed.shape[1] == words_per_row3(k)
    row_sum = codes.sum(axis=1, dtype=np.int64).astype(np.int32)
    return packed, row_sum, stats[:5].copy()


def unpack3(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of pack3: uint32 [n, words_per_row3(k)] -> int8 codes [n, k].

    Raises ValueError on a sign or magnitude bit without its nonzero bit, on a
    row length that does not match k, or on a nonzero padding code.
    """
    packed = np.asarray(packed)
    if packed.ndim != 2 or packed.dtype != np.uint32:
        raise ValueError("packed must be a 2-D uint32 array")
    n, w = packed.shape
    if w != words_per_row3(k):
        raise ValueError(f"row holds {w} words, k={k} needs {words_per_row3(k)}")
    k128 = 128 * math.ceil(k / 128)
    w2 = k128 // CODES_PER_WORD
    # the sign/nonzero plane is the 2-bit layout; unpack() checks its fields
    ternary = unpack(packed[:, :w2], w2 * CODES_PER_WORD)
    plane_m = packed[:, w2:]
    big = np.zeros((n, plane_m.shape[1], CODES_PER_MAG_WORD), dtype=bool)
    for j in range(CODES_PER_MAG_WORD):
        big[:, :, j] = ((plane_m >> np.uint32(mag_bit_position(j))) & np.uint32(1)).astype(bool)
    big = big.reshape(n, k128)
    if np.any(big & (ternary == 0)):
        raise ValueError("magnitude bit set on a zero code")
    codes = (ternary.astype(np.int16) * np.where(big, 2, 1)).astype(np.int8)
    if np.any(codes[:, k:]):
        raise ValueError("nonzero padding code")
    return codes[:, :k].copy()


def ternary3_gemm_small(packed: np.ndarray, scale: np.ndarray, k: int, x: np.ndarray,
                        row_block: int = 16384) -> np.ndarray:
    """Y[m, r] = s_r * sum_j c_rj * X[m, j] in fp64 for five-level codes."""
    xs = _as_rows(x, k)
    scale = np.asarray(scale)
    if scale.dtype != np.float32 or scale.shape != (packed.shape[0],):
        raise ValueError("scale must be fp32 [n]")
    n = packed.shape[0]
    y = np.empty((xs.shape[0], n), dtype=np.float64)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        c = unpack3(packed[r0:r1], k).astype(np.float64)
        y[:, r0:r1] = (xs @ c.T) * scale[r0:r1].astype(np.float64)[None, :]
    return y


def ternary3_gemv(packed: np.ndarray, scale: np.ndarray, k: int, x: np.ndarray) -> np.ndarray:
    """y_r = s_r * sum_j c_rj * x_j in fp64 (one activation row) for five-level codes."""
    x = np.asarray(x)
    if x.ndim != 1:
        raise ValueError("ternary3_gemv takes one activation row")
    return ternary3_gemm_small(packed, scale, k, x[None, :])[0]


def ffn3_swiglu(gate_packed: np.ndarray, gate_scale: np.ndarray, up_packed: np.ndarray, up_scale: np.ndarray,
                down_packed: np.ndarray, down_scale: np.ndarray, d_model: int, x: np.ndarray):
    """ffn_swiglu with the three linears in the 3-bit layout: g = gate x,
    u = up x, h = fp16(silu(g) * u), y = down h, each linear five-level with
    per-row scales (Neutrino-1 8B model page: geometry table for the block,
    "Where the bytes live" for the 3-bit coded lane). Returns (h fp16 [m, d_ff],
    y fp64 [m, d_model]).
    """
    d_ff = gate_packed.shape[0]
    if up_packed.shape[0] != d_ff or down_packed.shape[0] != d_model:
        raise ValueError("gate and up are [d_ff, .], down is [d_model, .]")
    g = ternary3_gemm_small(gate_packed, gate_scale, d_model, x)
    u = ternary3_gemm_small(up_packed, up_scale, d_model, x)
    h = (silu(g) * u).astype(np.float16)
    y = ternary3_gemm_small(down_packed, down_scale, d_ff, h)
    return h, y
