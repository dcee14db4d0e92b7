"""Seeded synthetic inputs for the packed ternary GEMV path.

This module only draws inputs: ternary codes, per-row scales, fp16 activation
rows and int8 head weights, with the shapes and value statistics the Neutrino-1
8B model page gives (geometry table; "Inside the coded lane" for the code
distribution; "Where the bytes live" for the int8 head and its per-row scales).
It holds none of the method's arithmetic: no packing, no decoding, no dot
products. Both the CPU oracle side and the GPU side start from what it returns.

Two generator families:

* NumPy ``Generator(PCG64(seed))`` for every size the oracle handles (tests).
* ``torch.Generator`` on a CUDA device for the multi-GB weight streams of the
  benchmark and the full-size sampled parity tests; torch is only the random
  number source there, the codes it yields are handed to both sides.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# --------------------------------------------------------------------------
# Geometry (Neutrino-1 8B model page, geometry table): hidden 4,096; 32 query
# heads and 8 key-value heads of width 128; SwiGLU feed-forward width 12,288;
# 36 decoder layers; vocabulary 151,936 with an untied int8 output head.
# Shapes are (rows N = output features, columns K = input features).
# --------------------------------------------------------------------------
HIDDEN = 4096
FFN = 12288
HEAD_DIM = 128
N_Q_HEADS = 32
N_KV_HEADS = 8
N_LAYERS = 36
VOCAB = 151936

PROJECTIONS = ("q", "k", "v", "o", "gate", "up", "down")
SHAPES = {
    "q": (N_Q_HEADS * HEAD_DIM, HIDDEN),
    "k": (N_KV_HEADS * HEAD_DIM, HIDDEN),
    "v": (N_KV_HEADS * HEAD_DIM, HIDDEN),
    "o": (HIDDEN, N_Q_HEADS * HEAD_DIM),
    "gate": (FFN, HIDDEN),
    "up": (FFN, HIDDEN),
    "down": (HIDDEN, FFN),
}
HEAD_SHAPE = (VOCAB, HIDDEN)

# Code statistics ("Inside the coded lane"): 62.63 % zero, 18.68 % +1,
# 18.69 % -1 over all coded weights; gate and down reach 70-72 % zeros in
# layers 1-3 (0-based), attention stays near 62 % at every depth.
P_ZERO = 0.6263
P_PLUS = 0.1868
P_MINUS = 0.1869
P_ZERO_EARLY_FFN = 0.71
EARLY_FFN_LAYERS = (1, 2, 3)

# Seeds of the synthetic model.
SEED_BASE = 20260727
SEED_HEAD = SEED_BASE + 252
SEED_X_BASE = 20261727
SEED_SCALE_OFFSET = 1_000_003


@dataclasses.dataclass(frozen=True)
class CodeDist:
    """Probabilities of the codes 0, +1, -1 of one coded tensor."""

    p_zero: float
    p_plus: float
    p_minus: float


def balanced(p_zero: float) -> CodeDist:
    """Sign-balanced distribution with the given zero share."""
    half = (1.0 - p_zero) / 2.0
    return CodeDist(p_zero, half, half)


GLOBAL_DIST = CodeDist(P_ZERO, P_PLUS, P_MINUS)


def code_dist(layer: int, proj: str) -> CodeDist:
    """Code distribution of one linear of the synthetic 36-layer model."""
    if proj in ("gate", "down") and layer in EARLY_FFN_LAYERS:
        return balanced(P_ZERO_EARLY_FFN)
    return GLOBAL_DIST


def tensor_seed(layer: int, proj: str) -> int:
    return SEED_BASE + 7 * layer + PROJECTIONS.index(proj)


def x_seed(m: int) -> int:
    return SEED_X_BASE + m


def words_bytes(n: int, k: int) -> int:
    """Bytes of one packed 2-bit tensor: rows of 4*ceil(k/64) uint32 words."""
    return n * 4 * (4 * math.ceil(k / 64))


# --------------------------------------------------------------------------
# NumPy generators (sizes the oracle handles).
# --------------------------------------------------------------------------
def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def ternary_codes(seed: int, n: int, k: int, dist: CodeDist = GLOBAL_DIST) -> np.ndarray:
    """int8 codes [n, k]: u ~ U[0,1); 0 if u < p0, +1 if u < p0 + p+, else -1."""
    u = _rng(seed).random((n, k))
    codes = np.full((n, k), -1, dtype=np.int8)
    codes[u < dist.p_zero + dist.p_plus] = 1
    codes[u < dist.p_zero] = 0
    return codes


# Five-level codes of the 3-bit variant: the page gives only the split into
# zero, plus and minus ("Inside the coded lane"); the share of magnitude 2
# among nonzero codes is this project's choice (a quarter). One uniform draw
# u per code: 0 if u < p0; +2 if u < p0 + P_BIG * p+, +1 if u < p0 + p+;
# -2 if u < p0 + p+ + P_BIG * p-, else -1.
P_BIG = 0.25


def ternary3_codes(seed: int, n: int, k: int, dist: CodeDist = GLOBAL_DIST, p_big: float = P_BIG) -> np.ndarray:
    """int8 five-level codes [n, k] (-2..+2) by the thresholds above."""
    u = _rng(seed).random((n, k))
    p0, pp = dist.p_zero, dist.p_plus
    codes = np.full((n, k), -1, dtype=np.int8)
    codes[u < p0 + pp + p_big * dist.p_minus] = -2
    codes[u < p0 + pp] = 1
    codes[u < p0 + p_big * pp] = 2
    codes[u < p0] = 0
    return codes


def row_scales(seed: int, n: int, lo: float = 0.01, hi: float = 0.05) -> np.ndarray:
    """fp32 per-row scales ~ U[lo, hi)."""
    return _rng(seed + SEED_SCALE_OFFSET).uniform(lo, hi, size=n).astype(np.float32)


def activations(seed: int, m: int, k: int) -> np.ndarray:
    """fp16 activation rows [m, k] ~ N(0, 1), rounded to fp16."""
    return _rng(seed).standard_normal((m, k)).astype(np.float16)


def head_weights(seed: int, n: int, k: int) -> np.ndarray:
    """int8 head weights clip(round(N(0, 32)), -127, 127)."""
    w = np.rint(_rng(seed).standard_normal((n, k)) * 32.0)
    return np.clip(w, -127, 127).astype(np.int8)


def int8_full_range(seed: int, n: int, k: int) -> np.ndarray:
    """int8 weights uniform over the whole range -128..127 (edge-case input)."""
    return _rng(seed).integers(-128, 128, size=(n, k), dtype=np.int8)


def probe_activations(seed: int, m: int, k: int, vmax: int = 8) -> np.ndarray:
    """fp16 rows of integers drawn from +-{1..vmax} (exact-arithmetic probes)."""
    rng = _rng(seed)
    mag = rng.integers(1, vmax + 1, size=(m, k))
    sgn = rng.choice(np.array([-1, 1]), size=(m, k))
    return (mag * sgn).astype(np.float16)


def pow2_scales(seed: int, n: int, lo: int = -3, hi: int = 3) -> np.ndarray:
    """fp32 per-row scales 2**e, e uniform in [lo, hi] (exact-arithmetic probes)."""
    e = _rng(seed + SEED_SCALE_OFFSET).integers(lo, hi + 1, size=n)
    return np.ldexp(np.ones(n, dtype=np.float32), e.astype(np.int32)).astype(np.float32)


# --------------------------------------------------------------------------
# Device generators (multi-GB weight streams). torch is imported lazily so
# the CPU-only parts of the suite do not need it.
# --------------------------------------------------------------------------
def ternary_codes_device(seed: int, n: int, k: int, dist: CodeDist, device, row_block: int = 4096):
    """int8 codes [n, k] on ``device``; same thresholding rule as ternary_codes."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((n, k), dtype=torch.int8, device=device)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        u = torch.rand((r1 - r0, k), generator=g, device=device)
        c = torch.full_like(u, -1, dtype=torch.int8)
        c[u < dist.p_zero + dist.p_plus] = 1
        c[u < dist.p_zero] = 0
        out[r0:r1] = c
        del u, c
    return out


def ternary3_codes_device(seed: int, n: int, k: int, dist: CodeDist, device, p_big: float = P_BIG,
                          row_block: int = 4096):
    """int8 five-level codes [n, k] on ``device``; same thresholds as ternary3_codes."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((n, k), dtype=torch.int8, device=device)
    p0, pp = dist.p_zero, dist.p_plus
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        u = torch.rand((r1 - r0, k), generator=g, device=device)
        c = torch.full_like(u, -1, dtype=torch.int8)
        c[u < p0 + pp + p_big * dist.p_minus] = -2
        c[u < p0 + pp] = 1
        c[u < p0 + p_big * pp] = 2
        c[u < p0] = 0
        out[r0:r1] = c
        del u, c
    return out


def words3_bytes(n: int, k: int) -> int:
    """Bytes of one packed 3-bit tensor: rows of 12*ceil(k/128) uint32 words."""
    return n * 4 * (12 * math.ceil(k / 128))


def head_weights_device(seed: int, n: int, k: int, device, row_block: int = 16384):
    """int8 head weights clip(round(N(0, 32)), +-127) on ``device``."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = torch.empty((n, k), dtype=torch.int8, device=device)
    for r0 in range(0, n, row_block):
        r1 = min(n, r0 + row_block)
        z = torch.randn((r1 - r0, k), generator=g, device=device)
        out[r0:r1] = torch.clamp(torch.round(z * 32.0), -127, 127).to(torch.int8)
        del z
    return out


def row_scales_device(seed: int, n: int, device, lo: float = 0.01, hi: float = 0.05):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed + SEED_SCALE_OFFSET)
    return (torch.rand(n, generator=g, device=device) * (hi - lo) + lo).to(torch.float32)
