"""GPU parity of the 3-bit (five-level) variant through the C ABI against the
CPU oracle.

* pack_ternary3: words, row sums and the six counts bit for bit (hand-derived
  golden rows, ragged and unaligned sources, invalid bytes, the full gate
  shape).
* ternary3_gemv / ternary3_gemm_small on exact probes (integer activations,
  power-of-two scales, codes -2..+2: every fp32 partial sum is an exact
  integer, so any summation order gives the oracle's value bit for bit) at
  shapes that hit every launch shape and the element-guarded kernel, and on
  seeded workloads within |y - y_ref| <= 1e-3 * s_r * sum_j |c_rj| |x_j|;
  full-size gate and down tensors on sampled rows.
* Maximum sizes: k = 2^24 and n = 2^24, exact.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within, digit_probes, read_digits, read_format3_words, ternary3_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pbg(gpu):
    import packed_bit_gemv_amd as m

    m.lib()
    return m


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host_words(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def gpu_pack3(pbg, codes: np.ndarray):
    packed, row_sum, stats = pbg.pack_ternary3(dev(codes))
    return packed, row_sum.cpu().numpy(), stats.cpu().numpy()


SHAPES3 = [(1, 1), (3, 5), (7, 33), (5, 127), (9, 128), (4, 129), (17, 4096), (33, 4100), (40, 8200), (12, 12288)]


@pytest.mark.parametrize("n,k", SHAPES3 + [(1024, 4096)])
def test_pack3_bit_exact(pbg, n, k):
    say(f"pack3 n={n} k={k}")
    codes = synth.ternary3_codes(5000 + n + k, n, k)
    packed, row_sum, stats = gpu_pack3(pbg, codes)
    ref_p, ref_rs, ref_c = oracle.pack3(codes)
    assert np.array_equal(host_words(packed), ref_p)
    assert np.array_equal(row_sum, ref_rs)
    assert stats.tolist() == ref_c.tolist() + [0]


@pytest.mark.parametrize("case", range(len(read_format3_words())))
def test_pack3_golden_rows(pbg, case):
    k, codes, words = read_format3_words()[case]
    packed, row_sum, _ = gpu_pack3(pbg, codes[None, :])
    assert [f"{v:08X}" for v in host_words(packed)[0]] == [f"{v:08X}" for v in words]
    assert row_sum[0] == int(codes.astype(np.int64).sum())


def test_pack3_gate_full(pbg):
    n, k = synth.SHAPES["gate"]
    say("pack3 full gate")
    codes = synth.ternary3_codes(5100, n, k, synth.code_dist(1, "gate"))
    packed, row_sum, stats = gpu_pack3(pbg, codes)
    ref_p, ref_rs, ref_c = oracle.pack3(codes)
    assert np.array_equal(host_words(packed), ref_p)
    assert np.array_equal(row_sum, ref_rs)
    assert stats.tolist() == ref_c.tolist() + [0]


def test_pack3_unaligned_source(pbg):
    n, k = 37, 4096
    codes = synth.ternary3_codes(5200, n, k)
    buf = torch.zeros(n * k + 16, dtype=torch.int8, device="cuda:0")
    view = buf[3:3 + n * k].view(n, k)
    view.copy_(dev(codes))
    packed, row_sum, stats = pbg.pack_ternary3(view)
    ref_p, ref_rs, ref_c = oracle.pack3(codes)
    assert np.array_equal(host_words(packed), ref_p)
    assert np.array_equal(row_sum.cpu().numpy(), ref_rs)


@pytest.mark.parametrize("n,k", [(6, 96), (5, 4096), (3, 12300)])
def test_pack3_invalid_codes(pbg, n, k):
    """Bytes outside -2..+2 pack as 0, add nothing to the row sum and are counted."""
    codes = synth.ternary3_codes(5300 + k, n, k)
    bad_vals = np.array([3, -3, 4, -4, 127, -128, 100, -100], dtype=np.int8)
    rng = np.random.Generator(np.random.PCG64(5301 + k))
    pos = rng.choice(n * k, size=24, replace=False)
    bad = codes.copy().reshape(-1)
    bad[pos] = bad_vals[np.arange(24) % 8]
    bad = bad.reshape(n, k)
    clean = bad.copy().reshape(-1)
    clean[pos] = 0
    clean = clean.reshape(n, k)
    with pytest.raises(pbg.PbgError) as e:
        pbg.pack_ternary3(dev(bad))
    assert e.value.code == -4
    packed, row_sum, stats = pbg.pack_ternary3(dev(bad), check=False)
    ref_p, ref_rs, ref_c = oracle.pack3(clean)
    assert np.array_equal(host_words(packed), ref_p)
    assert np.array_equal(row_sum.cpu().numpy(), ref_rs)
    expect = ref_c.tolist()
    expect[2] -= 24  # the replaced positions are invalid, not zero
    assert stats.cpu().numpy().tolist() == expect + [24]


GEMV3_SHAPES = [(5, 16), (17, 100), (40, 4096), (33, 4100), (21, 8200), (64, 12288), (9000, 4096), (2100, 4096),
                (700, 4040), (1500, 8000), (300, 16384), (50, 16500), (3000, 12288)]


@pytest.mark.parametrize("n,k", GEMV3_SHAPES)
def test_gemv3_exact_probe(pbg, n, k):
    say(f"gemv3 exact n={n} k={k}")
    codes = synth.ternary3_codes(5400 + n + k, n, k)
    x = synth.probe_activations(5401 + k, 1, k)[0]
    s = synth.pow2_scales(5402 + n, n)
    packed, _, _ = gpu_pack3(pbg, codes)
    ref = oracle.ternary3_gemv(oracle.pack3(codes)[0], s, k, x)
    y = pbg.ternary3_gemv(packed, dev(s), k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref), np.argwhere(y != ref)[:5].tolist()


@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("n,k", [(5, 16), (40, 4096), (33, 4100), (64, 12288), (700, 8192), (2100, 4096),
                                 (9000, 4096), (6000, 4096), (300, 16384), (77, 4000)])
def test_gemm3_small_exact_probe(pbg, m, n, k):
    say(f"gemm3 exact m={m} n={n} k={k}")
    codes = synth.ternary3_codes(5500 + n + k, n, k)
    x = synth.probe_activations(5501 + m + k, m, k)
    s = synth.pow2_scales(5502 + n, n)
    packed, _, _ = gpu_pack3(pbg, codes)
    ref = oracle.ternary3_gemm_small(oracle.pack3(codes)[0], s, k, x)
    y = pbg.ternary3_gemm_small(packed, dev(s), k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref), (m, np.argwhere(y != ref)[:5].tolist())


@pytest.mark.parametrize("proj", ["k", "q", "gate", "down"])
@pytest.mark.parametrize("m", [1, 4, 8])
def test_gemm3_config_shapes_seeded(pbg, proj, m):
    n, k = synth.SHAPES[proj]
    say(f"gemm3 seeded {proj} m={m}")
    seed = synth.tensor_seed(1, proj)
    codes = synth.ternary3_codes(seed, n, k, synth.code_dist(1, proj))
    s = synth.row_scales(seed, n)
    x = synth.activations(synth.x_seed(0), m, k)
    packed, _, _ = gpu_pack3(pbg, codes)
    ref = oracle.ternary3_gemm_small(oracle.pack3(codes)[0], s, k, x)
    if m == 1:
        y = pbg.ternary3_gemv(packed, dev(s), k, dev(x[0])).cpu().numpy()[None, :]
    else:
        y = pbg.ternary3_gemm_small(packed, dev(s), k, dev(x)).cpu().numpy()
    assert_within(y, ref, ternary3_bound(codes, s, x), f"{proj} m={m}")


def test_gemv3_unaligned_x(pbg):
    n, k = 300, 4096
    codes = synth.ternary3_codes(5600, n, k)
    s = synth.pow2_scales(5601, n)
    x = synth.probe_activations(5602, 1, k)[0]
    buf = torch.zeros(k + 8, dtype=torch.float16, device="cuda:0")
    xv = buf[1:1 + k]
    xv.copy_(dev(x))
    packed, _, _ = gpu_pack3(pbg, codes)
    y = pbg.ternary3_gemv(packed, dev(s), k, xv).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, oracle.ternary3_gemv(oracle.pack3(codes)[0], s, k, x))


def test_gemv3_ternary_codes_match_2bit(pbg):
    """Codes in {-1, 0, +1} through the 3-bit path give the 2-bit path's bits
    (the same operands in the same order; the magnitude plane is zero)."""
    for proj in ("gate", "down", "k"):
        n, k = synth.SHAPES[proj]
        codes = dev(synth.ternary_codes(5700, n, k))
        s = dev(synth.row_scales(5701, n))
        x = dev(synth.activations(5702, 1, k)[0])
        y2 = pbg.ternary_gemv(pbg.pack_ternary(codes)[0], s, k, x)
        y3 = pbg.ternary3_gemv(pbg.pack_ternary3(codes)[0], s, k, x)
        assert torch.equal(y2, y3), proj


@pytest.mark.parametrize("n,k", [(37, 56), (300, 4100), (1000, 12288)])
def test_gemv3_digit_readback(pbg, n, k):
    """Every five-level code read back through the kernels' arithmetic: x =
    5^i on the 5 columns of one block and unit scales make y_r that block's
    codes as a balanced base-5 integer; over all blocks the digits must equal
    the codes, through ternary3_gemv and ternary3_gemm_small."""
    say(f"digit readback 3-bit n={n} k={k}")
    codes = synth.ternary3_codes(2400 + n + k, n, k)
    packed, _, _ = gpu_pack3(pbg, codes)
    s = dev(np.ones(n, dtype=np.float32))
    x, nd = digit_probes(k, 5)
    xd = dev(x)
    y1 = torch.stack([pbg.ternary3_gemv(packed, s, k, xd[b]) for b in range(len(x))]).cpu().numpy()
    assert np.array_equal(read_digits(y1, 5, nd, k), codes)
    y8 = torch.cat([pbg.ternary3_gemm_small(packed, s, k, xd[b:b + 8]) for b in range(0, len(x), 8)]).cpu().numpy()
    assert np.array_equal(read_digits(y8, 5, nd, k), codes)


@pytest.mark.parametrize("proj", ["gate", "down"])
def test_gemv3_full_size_sampled(pbg, proj):
    """Device-generated five-level codes at full size, packed on the GPU; the
    launch configuration the bench times; sampled rows against the oracle."""
    n, k = synth.SHAPES[proj]
    say(f"gemv3 full {proj}")
    seed = synth.tensor_seed(2, proj)
    codes = synth.ternary3_codes_device(seed, n, k, synth.code_dist(2, proj), "cuda:0")
    packed, _, stats = pbg.pack_ternary3(codes)
    s = synth.row_scales_device(seed, n, "cuda:0")
    x = synth.activations(synth.x_seed(0), 1, k)[0]
    y = pbg.ternary3_gemv(packed, s, k, dev(x)).cpu().numpy()
    rows = np.unique(np.concatenate([[0, 1, n - 1], np.random.Generator(np.random.PCG64(5800)).choice(n, 253)]))
    c_rows = codes[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    s_rows = s.cpu().numpy()[rows]
    ref = oracle.ternary3_gemv(oracle.pack3(c_rows)[0], s_rows, k, x)
    assert_within(y[rows][None, :], ref[None, :], ternary3_bound(c_rows, s_rows, x), proj)
    assert np.array_equal(host_words(packed[torch.from_numpy(rows).to("cuda:0")]), oracle.pack3(c_rows)[0])
    assert int(stats[5]) == 0 and int(stats.sum()) == n * k


# --------------------------------------------------------------------------
# Maximum sizes (PBG_MAX_K, PBG_MAX_N): the largest row and the largest grids
# --------------------------------------------------------------------------
def test_gemv3_max_k(pbg):
    """k = 2^24 (6 MiB per row, the element-guarded kernels): exact probe with
    99 % zeros, so that every fp32 partial sum (in units of 2 c x) stays an
    exact integer; one activation row and two."""
    n, k = 3, 1 << 24
    say(f"gemv3 max k n={n} k={k}")
    codes = synth.ternary3_codes(41, n, k, synth.balanced(0.99))
    x = synth.probe_activations(42, 2, k)
    s = synth.pow2_scales(43, n)
    assert np.all(np.abs(codes).sum(axis=1, dtype=np.int64) * 8 * 2 < 2 ** 24)
    ref_p = oracle.pack3(codes)[0]
    p, _, _ = gpu_pack3(pbg, codes)
    assert np.array_equal(host_words(p), ref_p)
    y = pbg.ternary3_gemv(p, dev(s), k, dev(x[0])).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, oracle.ternary3_gemv(ref_p, s, k, x[0]))
    y2 = pbg.ternary3_gemm_small(p, dev(s), k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y2, oracle.ternary3_gemm_small(ref_p, s, k, x))


def test_gemv3_max_n(pbg):
    """n = 2^24 rows (the largest grids of the 3-bit GEMV and of its matrix-core
    m-row kernel): exact probes on sampled rows, the last rows included."""
    n, k = 1 << 24, 16
    say(f"gemv3 max n n={n} k={k}")
    codes = synth.ternary3_codes_device(44, n, k, synth.GLOBAL_DIST, "cuda:0")
    x = synth.probe_activations(45, 8, k)
    s_host = synth.pow2_scales(46, 4096)
    s = dev(np.resize(s_host, n))  # scales repeat every 4,096 rows
    p, _, st = pbg.pack_ternary3(codes)
    assert int(st.cpu()[:5].sum()) == n * k
    rng = np.random.Generator(np.random.PCG64(47))
    rows = np.unique(np.concatenate([rng.choice(n, size=4096, replace=False), np.arange(n - 16, n)]))
    idx = torch.from_numpy(rows).to("cuda:0")
    c_rows = codes[idx].cpu().numpy()
    del codes
    s_rows = s_host[rows % 4096]
    ref_p = oracle.pack3(c_rows)[0]
    y = pbg.ternary3_gemv(p, s, k, dev(x[0])).cpu().numpy().astype(np.float64)
    assert np.array_equal(y[rows], oracle.ternary3_gemv(ref_p, s_rows, k, x[0]))
    del y
    y8 = pbg.ternary3_gemm_small(p, s, k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y8[:, rows], oracle.ternary3_gemm_small(ref_p, s_rows, k, x))
