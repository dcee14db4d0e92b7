"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer and byte work is compared bit for bit (packed words, row sums, code
counts). Floating-point outputs are compared
  * bit for bit on exact-arithmetic probes (integer activations, power-of-two
    scales: every fp32 partial sum is an exact small integer, so
    any summation order gives the oracle's value), which catches any single
    wrong code, sign or index;
  * within |y - y_ref| <= 1e-3 * s_r * sum_j |x_j| (ternary) or
    1e-3 * s_v * sum_j |w_vj| |x_j| (head) on the seeded workloads.
"""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within, digit_probes, head_bound, read_digits, ternary_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pbg(gpu):
    import packed_bit_gemv_amd as m

    m.lib()
    return m


def dev(a: np.ndarray, device="cuda:0"):
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def host_words(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def gpu_pack(pbg, codes: np.ndarray):
    packed, row_sum, stats = pbg.pack_ternary(dev(codes))
    return packed, row_sum, stats


SHAPES_SMALL = [(1, 1), (3, 7), (5, 16), (4, 64), (17, 65), (9, 100), (33, 1000), (40, 4096), (50, 4097),
                (21, 8200), (64, 12288), (7, 20000)]


# --------------------------------------------------------------------------
# pack_ternary
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n,k", SHAPES_SMALL + [(1024, 4096)])
def test_pack_bit_exact(pbg, n, k):
    say(f"pack n={n} k={k}")
    codes = synth.ternary_codes(1000 + n + k, n, k)
    ref_p, ref_rs, ref_c = oracle.pack(codes)
    p, rs, st = gpu_pack(pbg, codes)
    torch.cuda.synchronize()
    assert np.array_equal(host_words(p), ref_p)
    assert np.array_equal(rs.cpu().numpy(), ref_rs)
    assert st.cpu().numpy().tolist() == ref_c.tolist() + [0]


def test_pack_gate_full(pbg):
    say("pack gate 12288x4096")
    codes = synth.ternary_codes(synth.tensor_seed(1, "gate"), 12288, 4096, synth.code_dist(1, "gate"))
    ref_p, ref_rs, ref_c = oracle.pack(codes)
    p, rs, st = gpu_pack(pbg, codes)
    assert np.array_equal(host_words(p), ref_p)
    assert np.array_equal(rs.cpu().numpy(), ref_rs)
    assert st.cpu().numpy().tolist() == ref_c.tolist() + [0]


def test_pack_unaligned_source(pbg):
    """Codes starting at an odd address take the byte-wise path."""
    n, k = 6, 160
    codes = synth.ternary_codes(77, n, k)
    buf = torch.zeros(n * k + 1, dtype=torch.int8, device="cuda:0")
    buf[1:] = dev(codes.reshape(-1))
    view = buf[1:].view(n, k)
    p, rs, st = pbg.pack_ternary(view)
    ref_p, ref_rs, ref_c = oracle.pack(codes)
    assert np.array_equal(host_words(p), ref_p)
    assert np.array_equal(rs.cpu().numpy(), ref_rs)


def test_pack_invalid_codes(pbg):
    codes = synth.ternary_codes(78, 8, 300)
    codes[2, 5] = 2
    codes[7, 299] = -128
    with pytest.raises(pbg.PbgError) as e:
        gpu_pack(pbg, codes)
    assert e.value.code == -4
    _, _, st = pbg.pack_ternary(dev(codes), check=False)
    assert st.cpu().numpy()[3] == 2


@pytest.mark.parametrize("n,k", [(8, 320), (5, 4096), (3, 12288)])
def test_pack_invalid_codes_whole_chunks(pbg, n, k):
    """Rows of whole 16-byte chunks (four code bytes packed at a time) with every kind of invalid byte at
    several places in a word: each packs as 0 and adds nothing to the row sum; the counts split exactly."""
    say(f"pack invalid whole chunks n={n} k={k}")
    codes = synth.ternary_codes(79 + k, n, k)
    rng = np.random.default_rng(80 + k)
    bad_vals = np.array([2, 3, 126, 127, -2, -3, -127, -128], dtype=np.int8)
    cells = rng.choice(n * k, size=64, replace=False)
    raw = codes.copy().reshape(-1)
    raw[cells] = bad_vals[np.arange(64) % len(bad_vals)]
    raw = raw.reshape(n, k)
    valid = codes.copy().reshape(-1)
    valid[cells] = 0
    valid = valid.reshape(n, k)
    p, rs, st = pbg.pack_ternary(dev(raw), check=False)
    ref_p, ref_rs, _ = oracle.pack(valid)
    assert np.array_equal(host_words(p), ref_p)
    assert np.array_equal(rs.cpu().numpy(), ref_rs)
    inval = np.zeros(n * k, dtype=bool)
    inval[cells] = True
    inval = inval.reshape(n, k)
    expect = [int(((raw == -1) & ~inval).sum()), int(((raw == 0) & ~inval).sum()), int(((raw == 1) & ~inval).sum()), 64]
    assert st.cpu().numpy().tolist() == expect


# --------------------------------------------------------------------------
# ternary_gemv (M = 1)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("n,k", SHAPES_SMALL)
def test_gemv_exact_probe(pbg, n, k):
    say(f"gemv exact n={n} k={k}")
    codes = synth.ternary_codes(2000 + n + k, n, k)
    x = synth.probe_activations(3000 + k, 1, k)[0]
    s = synth.pow2_scales(4000 + n, n)
    ref = oracle.ternary_gemv(oracle.pack(codes)[0], s, k, x)
    p, _, _ = gpu_pack(pbg, codes)
    y = pbg.ternary_gemv(p, dev(s), k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref)


# one shape per M = 1 launch configuration (chunks per lane 1..4, small and large n),
# several with a partial last chunk
@pytest.mark.parametrize("n,k", [(9000, 4096), (2100, 4096), (700, 4040), (2100, 8192), (1500, 8000),
                                 (2049, 12296), (333, 12288), (2050, 16000), (300, 16384)])
def test_gemv_launch_shapes_exact(pbg, n, k):
    say(f"gemv launch shape n={n} k={k}")
    codes = synth.ternary_codes(2500 + n + k, n, k)
    x = synth.probe_activations(3500 + k, 1, k)[0]
    s = synth.pow2_scales(4500 + n, n)
    ref = oracle.ternary_gemv(oracle.pack(codes)[0], s, k, x)
    p, _, _ = gpu_pack(pbg, codes)
    y = pbg.ternary_gemv(p, dev(s), k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("n,k", SHAPES_SMALL)
def test_gemv_random_tolerance(pbg, n, k):
    say(f"gemv random n={n} k={k}")
    codes = synth.ternary_codes(5000 + n + k, n, k)
    x = synth.activations(6000 + k, 1, k)[0]
    s = synth.row_scales(7000 + n, n)
    ref = oracle.ternary_gemv(oracle.pack(codes)[0], s, k, x)
    p, _, _ = gpu_pack(pbg, codes)
    y = pbg.ternary_gemv(p, dev(s), k, dev(x)).cpu().numpy()
    assert_within(y[None], ref[None], ternary_bound(s, x), f"gemv {n}x{k}")


@pytest.mark.parametrize("proj", ["k", "q", "gate", "up", "down"])
def test_gemv_config_shapes(pbg, proj):
    """Full config shapes at M = 1 (seeded as in the benchmark's numpy recipe)."""
    n, k = synth.SHAPES[proj]
    layer = 1
    say(f"gemv config {proj} {n}x{k}")
    codes = synth.ternary_codes(synth.tensor_seed(layer, proj), n, k, synth.code_dist(layer, proj))
    s = synth.row_scales(synth.tensor_seed(layer, proj), n)
    x = synth.activations(synth.x_seed(0), 1, k)[0]
    ref = oracle.ternary_gemv(oracle.pack(codes)[0], s, k, x)
    p, _, _ = gpu_pack(pbg, codes)
    y = pbg.ternary_gemv(p, dev(s), k, dev(x)).cpu().numpy()
    assert_within(y[None], ref[None], ternary_bound(s, x), f"{proj}")
    # bitwise repeatable
    y2 = pbg.ternary_gemv(p, dev(s), k, dev(x)).cpu().numpy()
    assert np.array_equal(y, y2)


def test_gemv_special_cases(pbg):
    n = k = 300
    x = synth.activations(11, 1, k)[0]
    s = synth.row_scales(12, n)
    xd, sd = dev(x), dev(s)
    zero = np.zeros((n, k), dtype=np.int8)
    y0 = pbg.ternary_gemv(gpu_pack(pbg, zero)[0], sd, k, xd).cpu().numpy()
    assert np.all(y0 == 0.0)
    eye = np.eye(n, k, dtype=np.int8)
    ye = pbg.ternary_gemv(gpu_pack(pbg, eye)[0], sd, k, xd).cpu().numpy()
    assert np.array_equal(ye.astype(np.float64), (s.astype(np.float64) * x.astype(np.float64)).astype(np.float32))
    codes = synth.ternary_codes(13, n, k)
    y = pbg.ternary_gemv(gpu_pack(pbg, codes)[0], sd, k, xd).cpu().numpy()
    yn = pbg.ternary_gemv(gpu_pack(pbg, -codes)[0], sd, k, xd).cpu().numpy()
    assert np.array_equal(yn, -y)


@pytest.mark.parametrize("n,k", [(37, 56), (300, 4100), (1000, 12288)])
def test_digit_readback(pbg, n, k):
    """Every code read back through the kernels' arithmetic: x = 3^i on the 7
    columns of one block and unit scales make y_r that block's codes as a
    balanced-ternary integer; over all blocks the digits must equal the codes,
    through ternary_gemv (one block per call) and ternary_gemm_small (8 blocks,
    and the remainder, per call)."""
    say(f"digit readback n={n} k={k}")
    codes = synth.ternary_codes(2300 + n + k, n, k)
    packed, _, _ = gpu_pack(pbg, codes)
    s = dev(np.ones(n, dtype=np.float32))
    x, nd = digit_probes(k, 3)
    xd = dev(x)
    y1 = torch.stack([pbg.ternary_gemv(packed, s, k, xd[b]) for b in range(len(x))]).cpu().numpy()
    assert np.array_equal(read_digits(y1, 3, nd, k), codes)
    y8 = torch.cat([pbg.ternary_gemm_small(packed, s, k, xd[b:b + 8]) for b in range(0, len(x), 8)]).cpu().numpy()
    assert np.array_equal(read_digits(y8, 3, nd, k), codes)


def test_gemv_full_size_sampled(pbg):
    """Device-generated gate and down tensors at full size (the benchmark's
    generator), checked on sampled rows against the oracle."""
    rng = np.random.Generator(np.random.PCG64(5))
    for proj, layer in (("gate", 2), ("down", 2), ("up", 5)):
        n, k = synth.SHAPES[proj]
        say(f"gemv full-size sampled {proj}")
        codes = synth.ternary_codes_device(synth.tensor_seed(layer, proj), n, k, synth.code_dist(layer, proj),
                                           "cuda:0")
        s = synth.row_scales_device(synth.tensor_seed(layer, proj), n, "cuda:0")
        x = synth.activations(synth.x_seed(0), 1, k)[0]
        p, _, st = pbg.pack_ternary(codes)
        y = pbg.ternary_gemv(p, s, k, dev(x)).cpu().numpy()
        rows = np.sort(rng.choice(n, size=256, replace=False))
        c_rows = codes[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
        s_rows = s.cpu().numpy()[rows]
        ref = oracle.ternary_gemv(oracle.pack(c_rows)[0], s_rows, k, x)
        assert_within(y[rows][None], ref[None], ternary_bound(s_rows, x), proj)
        assert np.array_equal(host_words(p)[rows], oracle.pack(c_rows)[0])


# --------------------------------------------------------------------------
# ternary_gemm_small (M <= 8)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,k", [(5, 16), (17, 65), (40, 4096), (21, 8200), (64, 12288), (8200, 4096),
                                 (1000, 12288), (3000, 4096), (100, 6000), (2100, 12280), (6144, 4096),
                                 (700, 8192), (300, 16384), (70, 13000)])
def test_small_m_exact_probe(pbg, m, n, k):
    say(f"small-m exact m={m} n={n} k={k}")
    codes = synth.ternary_codes(8000 + n + k, n, k)
    x = synth.probe_activations(9000 + m, m, k)
    s = synth.pow2_scales(9100 + n, n)
    ref = oracle.ternary_gemm_small(oracle.pack(codes)[0], s, k, x)
    p, _, _ = gpu_pack(pbg, codes)
    y = pbg.ternary_gemm_small(p, dev(s), k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref)


def _random_shapes(seed: int, count: int):
    """Seeded (n, k, m) over the dispatch's ranges: n up to 12,500, k up to
    12,800 (multiples of 8 mostly, some not), n * k below 8 million."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < count:
        n = int(rng.integers(1, 12_500))
        k = int(rng.integers(1, 1_600)) * 8 + (int(rng.integers(1, 8)) if rng.random() < 0.15 else 0)
        if n * k < 8_000_000:
            out.append((n, k, int(rng.integers(1, 9))))
    return out


@pytest.mark.parametrize("n,k,m", _random_shapes(20261203, 24))
def test_small_m_random_shapes_exact(pbg, n, k, m):
    """Random shapes across every launch shape and kernel of the dispatch, exact probes."""
    say(f"small-m random m={m} n={n} k={k}")
    codes = synth.ternary_codes(9500 + n + k, n, k)
    x = synth.probe_activations(9600 + m, m, k)
    s = synth.pow2_scales(9700 + n, n)
    ref = oracle.ternary_gemm_small(oracle.pack(codes)[0], s, k, x)
    p, _, _ = gpu_pack(pbg, codes)
    y = pbg.ternary_gemm_small(p, dev(s), k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("m", [2, 4, 7, 8])
@pytest.mark.parametrize("proj", ["k", "o", "gate", "down"])
def test_small_m_config_shapes(pbg, m, proj):
    n, k = synth.SHAPES[proj]
    say(f"small-m config m={m} {proj}")
    codes = synth.ternary_codes(synth.tensor_seed(0, proj), n, k, synth.code_dist(0, proj))
    s = synth.row_scales(synth.tensor_seed(0, proj), n)
    x = synth.activations(synth.x_seed(0), m, k)
    ref = oracle.ternary_gemm_small(oracle.pack(codes)[0], s, k, x)
    p, _, _ = gpu_pack(pbg, codes)
    y = pbg.ternary_gemm_small(p, dev(s), k, dev(x)).cpu().numpy()
    assert_within(y, ref, ternary_bound(s, x), f"{proj} m={m}")


# --------------------------------------------------------------------------
# int8_head_gemv
# --------------------------------------------------------------------------
@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("n,k", [(1, 16), (3, 5), (17, 100), (40, 4096), (33, 4112), (9, 12288), (1000, 4096),
                                 (40000, 1024), (4100, 2048), (33, 3072), (5, 4096)])
def test_head_exact_probe(pbg, m, n, k):
    say(f"head exact m={m} n={n} k={k}")
    w = synth.int8_full_range(10000 + n + k, n, k)
    x = synth.probe_activations(11000 + m, m, k)
    s = synth.pow2_scales(12000 + n, n)
    ref = oracle.int8_head_gemv(w, s, x)
    y = pbg.int8_head_gemv(dev(w), dev(s), dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("m", [1, 2, 4, 7, 8])
def test_head_random_tolerance(pbg, m):
    n, k = 4099, 4096
    say(f"head random m={m}")
    w = synth.head_weights(13000, n, k)
    x = synth.activations(14000 + m, m, k)
    s = synth.row_scales(15000, n)
    ref = oracle.int8_head_gemv(w, s, x)
    y = pbg.int8_head_gemv(dev(w), dev(s), dev(x)).cpu().numpy()
    assert_within(y, ref, head_bound(w, s, x), f"head m={m}")


@pytest.mark.parametrize("m", [1, 4, 8])
def test_head_full_size_sampled(pbg, m):
    n, k = synth.HEAD_SHAPE
    say(f"head full-size sampled m={m}")
    w = synth.head_weights_device(synth.SEED_HEAD, n, k, "cuda:0")
    s = synth.row_scales_device(synth.SEED_HEAD, n, "cuda:0")
    x = synth.activations(synth.x_seed(0), m, k)
    y = pbg.int8_head_gemv(w, s, dev(x)).cpu().numpy()
    rows = np.sort(np.random.Generator(np.random.PCG64(9)).choice(n, size=512, replace=False))
    rows = np.concatenate([rows, [0, n - 1]])
    w_rows = w[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    s_rows = s.cpu().numpy()[rows]
    ref = oracle.int8_head_gemv(w_rows, s_rows, x)
    assert_within(y[:, rows], ref, head_bound(w_rows, s_rows, x), "head full")


# --------------------------------------------------------------------------
# Error paths with real device buffers
# --------------------------------------------------------------------------
def test_device_error_paths(pbg):
    lib = pbg.lib()
    p = torch.zeros((8, 4), dtype=torch.int32, device="cuda:0")
    s = torch.ones(8, dtype=torch.float32, device="cuda:0")
    x = torch.ones(64, dtype=torch.float16, device="cuda:0")
    y = torch.empty(8, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.ternary_gemv(p.data_ptr() + 4, s.data_ptr(), 7, 64, x.data_ptr(), y.data_ptr(), stream) == -3
    assert lib.ternary_gemv(p.data_ptr(), s.data_ptr(), 8, 0, x.data_ptr(), y.data_ptr(), stream) == -2
    assert lib.ternary_gemm_small(p.data_ptr(), s.data_ptr(), 8, 64, x.data_ptr(), 9, y.data_ptr(), stream) == -2
    assert lib.ternary_gemv(p.data_ptr(), s.data_ptr(), 8, 64, x.data_ptr(), y.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 0)


def _loaded_hip_runtimes():
    """ctypes handles of every HIP runtime mapped into this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            path = line.split()[-1] if len(line.split()) >= 6 else ""
            if "libamdhip64" in os.path.basename(path):
                paths.add(path)
    return [ctypes.CDLL(p) for p in sorted(paths)]


def test_pending_hip_error_is_left_to_the_caller(pbg):
    """A HIP error left pending by earlier work (here a host-side query of a
    device that does not exist) is the caller's: an entry point then
    enqueues nothing, returns PBG_ERR_HIP and leaves the error pending."""
    lib = pbg.lib()
    p = torch.zeros((8, 4), dtype=torch.int32, device="cuda:0")
    s = torch.ones(8, dtype=torch.float32, device="cuda:0")
    x = torch.ones(64, dtype=torch.float16, device="cuda:0")
    y = torch.full((8,), 7.0, dtype=torch.float32, device="cuda:0")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    hips = _loaded_hip_runtimes()
    assert hips, "no HIP runtime mapped"
    v = ctypes.c_int(0)
    for h in hips:
        assert h.hipDeviceGetAttribute(ctypes.byref(v), 0, 9999) != 0
    pending = [h.hipPeekAtLastError() for h in hips]
    assert all(e != 0 for e in pending)
    assert lib.ternary_gemv(p.data_ptr(), s.data_ptr(), 8, 64, x.data_ptr(), y.data_ptr(), stream) == -5
    assert [h.hipPeekAtLastError() for h in hips] == pending  # still the caller's to see
    for h in hips:
        h.hipGetLastError()
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)  # nothing was enqueued
    assert lib.ternary_gemv(p.data_ptr(), s.data_ptr(), 8, 64, x.data_ptr(), y.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 0)


# --------------------------------------------------------------------------
# HIP graph capture and replay
# --------------------------------------------------------------------------
def test_graph_replay_matches_eager(pbg):
    """The GEMV entry points captured into a HIP graph give, on every replay,
    the same bits as eager calls; eager work runs between the replays."""
    n, k = 4096, 12288
    say("graph replay")
    codes = synth.ternary_codes(91, n, k)
    s = dev(synth.row_scales(92, n))
    x = dev(synth.activations(93, 8, k))
    w = dev(synth.head_weights(94, 3000, 4096))
    hs = dev(synth.row_scales(95, 3000))
    hx = dev(synth.activations(96, 4, 4096))
    p, _, _ = gpu_pack(pbg, codes)
    y1 = torch.empty(n, dtype=torch.float32, device="cuda:0")
    y4 = torch.empty((4, n), dtype=torch.float32, device="cuda:0")
    yh = torch.empty((4, 3000), dtype=torch.float32, device="cuda:0")

    def run():
        pbg.ternary_gemv(p, s, k, x[0], y1)
        pbg.ternary_gemm_small(p, s, k, x[:4], y4)
        pbg.int8_head_gemv(w, hs, hx, yh)

    run()
    torch.cuda.synchronize()
    ref = (y1.clone(), y4.clone(), yh.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        y1.fill_(float("nan"))
        y4.fill_(float("nan"))
        yh.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1, ref[0]) and torch.equal(y4, ref[1]) and torch.equal(yh, ref[2]), rep
        pbg.ternary_gemv(p, s, k, x[1], torch.empty_like(y1))  # eager work between replays
        torch.cuda.synchronize()


# --------------------------------------------------------------------------
# Greedy argmax through the head, embedding rows
# --------------------------------------------------------------------------
@pytest.mark.parametrize("m", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("n,k", [(1, 16), (17, 100), (40, 4096), (33, 4112), (2000, 4096), (9, 12288),
                                 (40000, 1024), (33, 3072)])
def test_head_argmax_exact_probe(pbg, m, n, k):
    """Integer activations, power-of-two scales, full-range int8: logits are
    exact on both sides, so the token (lowest index on ties) and its logit
    must equal the oracle's."""
    say(f"argmax exact m={m} n={n} k={k}")
    w = synth.int8_full_range(16000 + n + k, n, k)
    w[n // 2] = w[0]  # a guaranteed tie in every row of X when row 0 wins
    x = synth.probe_activations(17000 + m, m, k)
    s = synth.pow2_scales(18000 + n, n)
    s[n // 2] = s[0]
    tok_ref, y_ref = oracle.int8_head_argmax(w, s, x)
    tok, logit = pbg.int8_head_argmax(dev(w), dev(s), dev(x))
    assert tok.cpu().numpy().tolist() == tok_ref.tolist()
    assert np.array_equal(logit.cpu().numpy().astype(np.float64), y_ref[np.arange(m), tok_ref])


@pytest.mark.parametrize("m", [1, 2, 3, 8])
@pytest.mark.parametrize("n,k", [(33, 4112), (40, 4096), (2000, 4096), (40000, 1024)])
def test_head_argmax_signed_zero_tie(pbg, m, n, k):
    """A zero maximum reached as -0 by a lower row (negative scale) and as +0
    by a higher row: the two logits are equal, so the lower row is the token,
    as in the oracle. Every other logit is -k."""
    say(f"argmax signed zero m={m} n={n} k={k}")
    w = np.full((n, k), -1, dtype=np.int8)
    lo, hi = n // 3, n // 3 + 7
    w[lo] = 0
    w[hi] = 0
    x = np.ones((m, k), dtype=np.float16)
    s = np.ones(n, dtype=np.float32)
    s[lo] = -1.0
    tok_ref, y_ref = oracle.int8_head_argmax(w, s, x)
    assert tok_ref.tolist() == [lo] * m
    tok, logit = pbg.int8_head_argmax(dev(w), dev(s), dev(x))
    assert tok.cpu().numpy().tolist() == [lo] * m
    assert np.all(logit.cpu().numpy() == 0.0)


@pytest.mark.parametrize("m", [1, 2, 4, 7, 8])
def test_head_argmax_random(pbg, m):
    n, k = 5003, 4096
    say(f"argmax random m={m}")
    w = synth.head_weights(19000, n, k)
    x = synth.activations(19100 + m, m, k)
    s = synth.row_scales(19200, n)
    tok_ref, y_ref = oracle.int8_head_argmax(w, s, x)
    bound = head_bound(w, s, x)
    tok, logit = pbg.int8_head_argmax(dev(w), dev(s), dev(x))
    tok = tok.cpu().numpy()
    y_gpu = pbg.int8_head_gemv(dev(w), dev(s), dev(x)).cpu().numpy()
    for i in range(m):
        t = int(tok[i])
        # a valid argmax of the exact logits within the error bounds
        assert y_ref[i, t] >= np.max(y_ref[i] - bound[i]) - bound[i, t]
        # the same logit and the lowest-index maximum of the kernel's own logits
        assert logit.cpu().numpy()[i] == y_gpu[i, t]
        assert t == int(np.argmax(y_gpu[i]))
        gap = np.sort(y_ref[i])[-1] - np.sort(y_ref[i])[-2]
        if gap > 2 * bound[i].max():
            assert t == tok_ref[i]


@pytest.mark.parametrize("m", [1, 3, 7])
def test_head_argmax_full_size(pbg, m):
    n, k = synth.HEAD_SHAPE
    say(f"argmax full head m={m}")
    w = synth.head_weights_device(synth.SEED_HEAD, n, k, "cuda:0")
    s = synth.row_scales_device(synth.SEED_HEAD, n, "cuda:0")
    x = synth.activations(synth.x_seed(0), m, k)
    tok, logit = pbg.int8_head_argmax(w, s, dev(x))
    y = pbg.int8_head_gemv(w, s, dev(x)).cpu().numpy()
    tok = tok.cpu().numpy()
    for i in range(m):
        assert tok[i] == int(np.argmax(y[i]))
        assert logit.cpu().numpy()[i] == y[i, tok[i]]
    # the token against the fp64 oracle over every row of the head: a valid
    # argmax of the exact logits within their error bounds, and the oracle's
    # own token whenever its top-2 gap exceeds twice the largest bound
    w_host, s_host = w.cpu().numpy(), s.cpu().numpy()
    tok_ref, y_ref = oracle.int8_head_argmax(w_host, s_host, x)
    bound = head_bound(w_host, s_host, x)
    lg = logit.cpu().numpy()
    for i in range(m):
        t = int(tok[i])
        assert y_ref[i, t] >= np.max(y_ref[i] - bound[i]) - bound[i, t], (i, t, int(tok_ref[i]))
        assert abs(float(lg[i]) - y_ref[i, t]) <= bound[i, t]
        top = np.sort(y_ref[i])
        if top[-1] - top[-2] > 2 * bound[i].max():
            assert t == int(tok_ref[i]), (i, t, int(tok_ref[i]))
    say(f"  tokens {tok.tolist()}, oracle {tok_ref.tolist()}")


def test_head_argmax_workspace_reuse_and_graph(pbg):
    """One workspace across calls with different m: every call leaves it zero, results match the
    plain head; a captured call replayed on new activations matches eager calls."""
    n, k = 40000, 4096
    say("argmax workspace reuse")
    w = synth.head_weights_device(synth.SEED_HEAD + 1, n, k, "cuda:0")
    s = synth.row_scales_device(synth.SEED_HEAD + 1, n, "cuda:0")
    keys = torch.zeros(8 * pbg.binding.ARGMAX_KEYS_PER_ROW, dtype=torch.int64, device="cuda:0")
    for m in (8, 1, 3, 8, 2):
        x = dev(synth.activations(500 + m, m, k))
        tok, logit = pbg.int8_head_argmax(w, s, x, keys=keys)
        y = pbg.int8_head_gemv(w, s, x)
        assert torch.equal(tok.long(), torch.argmax(y, dim=1))
        assert torch.equal(logit, y.gather(1, tok.long()[:, None])[:, 0])
        assert int(torch.count_nonzero(keys)) == 0
    m = 7
    xb = dev(synth.activations(600, m, k))
    tok_b = torch.empty(m, dtype=torch.int32, device="cuda:0")
    lg_b = torch.empty(m, dtype=torch.float32, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pbg.int8_head_argmax(w, s, xb, keys, tok_b, lg_b)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pbg.int8_head_argmax(w, s, xb, keys, tok_b, lg_b)
    eager_keys = torch.zeros_like(keys)
    for rep in range(4):
        xb.copy_(dev(synth.activations(601 + rep, m, k)))
        graph.replay()
        torch.cuda.synchronize()
        tok_e, lg_e = pbg.int8_head_argmax(w, s, xb, keys=eager_keys)
        torch.cuda.synchronize()
        assert torch.equal(tok_b, tok_e) and torch.equal(lg_b, lg_e), rep
        assert int(torch.count_nonzero(keys)) == 0


def test_embedding_gather_exact(pbg):
    n, k = 777, 4100
    table = synth.int8_full_range(20000, n, k)
    s = synth.row_scales(20001, n)
    tokens = np.array([0, 776, 5, 5, 300, -1, 777, 123], dtype=np.int32)
    ref = oracle.embedding_gather(table, s, tokens)
    out = pbg.int8_embedding_gather(dev(table), dev(s), dev(tokens)).cpu().numpy()
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(out), ~ok)
    assert np.array_equal(out[ok], ref[ok])


def test_embedding_gather_full_table(pbg):
    n, k = synth.HEAD_SHAPE
    table = synth.head_weights_device(synth.SEED_HEAD + 1, n, k, "cuda:0")
    s = synth.row_scales_device(synth.SEED_HEAD + 1, n, "cuda:0")
    tokens = np.random.Generator(np.random.PCG64(21)).integers(0, n, size=64).astype(np.int32)
    tokens[:2] = [0, n - 1]
    out = pbg.int8_embedding_gather(table, s, dev(tokens)).cpu().numpy()
    rows = torch.from_numpy(tokens.astype(np.int64)).to("cuda:0")
    sub = table[rows].cpu().numpy()
    ref = oracle.embedding_gather(sub, s.cpu().numpy()[tokens], np.arange(len(tokens)))
    assert np.array_equal(out, ref)


# --------------------------------------------------------------------------
# Maximum sizes (PBG_MAX_K, PBG_MAX_N): the largest row and the largest grids
# --------------------------------------------------------------------------
def test_gemv_max_k(pbg):
    """k = 2^24 (one row per 4 MiB, the element-guarded kernel): exact probe with 99 % zeros,
    so every fp32 partial sum stays an exact integer."""
    n, k = 3, 1 << 24
    say(f"gemv max k n={n} k={k}")
    codes = synth.ternary_codes(31, n, k, synth.balanced(0.99))
    x = synth.probe_activations(32, 1, k)[0]
    s = synth.pow2_scales(33, n)
    ref_p = oracle.pack(codes)[0]
    ref = oracle.ternary_gemv(ref_p, s, k, x)
    p, _, _ = gpu_pack(pbg, codes)
    assert np.array_equal(host_words(p), ref_p)
    y = pbg.ternary_gemv(p, dev(s), k, dev(x)).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, ref)


def test_gemv_and_head_max_n(pbg):
    """n = 2^24 rows (the largest grids of the M = 1 GEMV and of the head): sampled rows, the last
    rows included, against the oracle; exact probes."""
    n, k = 1 << 24, 16
    say(f"gemv/head max n n={n} k={k}")
    codes = synth.ternary_codes_device(34, n, k, synth.GLOBAL_DIST, "cuda:0")
    x = synth.probe_activations(35, 1, k)[0]
    s_host = synth.pow2_scales(36, 4096)
    s = dev(np.resize(s_host, n))  # scales repeat every 4,096 rows
    p, _, st = pbg.pack_ternary(codes)
    y = pbg.ternary_gemv(p, s, k, dev(x)).cpu().numpy().astype(np.float64)
    rng = np.random.Generator(np.random.PCG64(37))
    rows = np.unique(np.concatenate([rng.choice(n, size=4096, replace=False), np.arange(n - 16, n)]))
    idx = torch.from_numpy(rows).to("cuda:0")
    c_rows = codes[idx].cpu().numpy()
    s_rows = s_host[rows % 4096]
    ref = oracle.ternary_gemv(oracle.pack(c_rows)[0], s_rows, k, x)
    assert np.array_equal(y[rows], ref)
    assert int(st.cpu()[0] + st.cpu()[1] + st.cpu()[2]) == n * k
    del p, y
    # the int8 head at the same row count
    w = synth.head_weights_device(38, n, k, "cuda:0")
    yh = pbg.int8_head_gemv(w, s, dev(x[None, :])).cpu().numpy()[0].astype(np.float64)
    w_rows = w[idx].cpu().numpy()
    href = oracle.int8_head_gemv(w_rows, s_rows, x[None, :])[0]
    assert np.array_equal(yh[rows], href)


def test_ffn_max_d_ff(pbg):
    """d_ff = 2^24 with d_model = 8 (the largest gate/up grid; down is one 16M-column row group):
    integer probe, h and y exact."""
    d_model, d_ff = 8, 1 << 24
    say(f"ffn max d_ff d_model={d_model} d_ff={d_ff}")
    x = np.array([1, -1, 1, 1, -1, 1, -1, -1], dtype=np.float16)
    sx = np.where(x > 0, 1, -1).astype(np.int8)
    # gate rows: sign(x) in every column (negated on rows r = 3 mod 5) and scale 8, so g = +-64;
    # up rows: one code sign(x_j) at column j = r % 8, so u = 1
    gate = np.broadcast_to(sx, (5, d_model)).copy()
    gate[3] = -sx
    g_codes = torch.from_numpy(gate).to("cuda:0").repeat((d_ff + 4) // 5, 1)[:d_ff].contiguous()
    u_codes = torch.zeros((d_ff, d_model), dtype=torch.int8, device="cuda:0")
    cols = torch.arange(d_ff, device="cuda:0") % d_model
    u_codes[torch.arange(d_ff, device="cuda:0"), cols] = torch.from_numpy(sx).to("cuda:0")[cols]
    gs = torch.full((d_ff,), 8.0, dtype=torch.float32, device="cuda:0")
    us = torch.ones(d_ff, dtype=torch.float32, device="cuda:0")
    down = synth.ternary_codes(39, d_model, d_ff, synth.balanced(0.999))
    sd = synth.pow2_scales(40, d_model)
    keep = np.arange(d_ff) % 5 != 3
    h_exp = np.where(keep, 64.0, 0.0)  # silu(64) * 1 = 64 exactly; silu(-64) * 1 rounds to 0 in fp16
    assert np.all(np.count_nonzero(down, axis=1) * 64 < 2 ** 24)  # every partial sum an exact fp32 integer
    y_exp = 64.0 * down[:, keep].sum(axis=1, dtype=np.int64).astype(np.float64) * sd.astype(np.float64)
    h, y = pbg.ternary_ffn_swiglu(pbg.pack_ternary(g_codes)[0], gs, pbg.pack_ternary(u_codes)[0], us,
                                  gpu_pack(pbg, down)[0], dev(sd), dev(x))
    assert np.array_equal(h.cpu().numpy().astype(np.float64), h_exp)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_exp)


# --------------------------------------------------------------------------
# Concurrency: no hidden shared state between calls
# --------------------------------------------------------------------------
def test_concurrent_streams_and_threads_match_sequential(pbg):
    """Calls on two streams at once, and from two host threads with a stream
    each, give the same bits as the same calls one after another (every
    kernel sums in a fixed order, the argmax workspaces are per caller, and
    the FFN block's two-slice down adds only onto the caller's own y)."""
    import threading

    say("concurrent streams")
    n, k, hn = 12288, 4096, 40000
    codes = synth.ternary_codes_device(synth.tensor_seed(2, "gate"), n, k, synth.code_dist(2, "gate"), "cuda:0")
    packed = pbg.pack_ternary(codes)[0]
    del codes
    s = synth.row_scales_device(synth.tensor_seed(2, "gate"), n, "cuda:0")
    hw = synth.head_weights_device(synth.SEED_HEAD + 2, hn, k, "cuda:0")
    hs = synth.row_scales_device(synth.SEED_HEAD + 2, hn, "cuda:0")
    x = dev(synth.activations(700, 8, k))
    codes = synth.ternary_codes_device(synth.tensor_seed(2, "down"), k, n, synth.code_dist(2, "down"), "cuda:0")
    down = pbg.pack_ternary(codes)[0]
    del codes
    sd = synth.row_scales_device(synth.tensor_seed(2, "down"), k, "cuda:0")

    def work_a():
        return (pbg.ternary_gemv(packed, s, k, x[0]), pbg.ternary_gemm_small(packed, s, k, x[:4]),
                pbg.int8_head_gemv(hw, hs, x[:3]), pbg.ternary_ffn_swiglu(packed, s, packed, s, down, sd, x[:4]))

    def work_b(keys):
        return (pbg.int8_head_argmax(hw, hs, x[:7], keys=keys), pbg.ternary_gemm_small(packed, s, k, x[:2]),
                pbg.int8_head_gemv(hw, hs, x[:1]), pbg.ternary_ffn_swiglu(packed, s, packed, s, down, sd, x[:8]))

    keys_a = torch.zeros(8 * pbg.binding.ARGMAX_KEYS_PER_ROW, dtype=torch.int64, device="cuda:0")
    keys_b = torch.zeros_like(keys_a)
    ref_a, ref_b = work_a(), work_b(keys_a)
    torch.cuda.synchronize()

    def same(got, ref):
        flat_g = [t for g in got for t in (g if isinstance(g, tuple) else (g,))]
        flat_r = [t for r in ref for t in (r if isinstance(r, tuple) else (r,))]
        return all(torch.equal(a, b) for a, b in zip(flat_g, flat_r))

    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(5):
        with torch.cuda.stream(sa):
            oa = work_a()
        with torch.cuda.stream(sb):
            ob = work_b(keys_b)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert same(oa, ref_a) and same(ob, ref_b)
    assert int(torch.count_nonzero(keys_b)) == 0

    say("concurrent threads")
    results, errors = {}, []

    def thread_body(name, fn):
        try:
            st = torch.cuda.Stream()
            st.wait_stream(torch.cuda.default_stream())
            got = []
            with torch.cuda.stream(st):
                for _ in range(5):
                    got.append(fn())
            st.synchronize()
            results[name] = got
        except Exception as e:  # reported below
            errors.append(repr(e))

    keys_t = torch.zeros_like(keys_a)
    threads = [threading.Thread(target=thread_body, args=("a", work_a)),
               threading.Thread(target=thread_body, args=("b", lambda: work_b(keys_t)))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert all(same(g, ref_a) for g in results["a"]) and all(same(g, ref_b) for g in results["b"])
    assert int(torch.count_nonzero(keys_t)) == 0
