"""GPU parity of ternary_gemm_splitk (K split across workgroups, slices added
in slice order through a caller workspace) against the CPU oracle.

* Exact probes (integer activations, power-of-two scales): every fp32 partial
  sum is an exact integer, so the result must equal the oracle bit for bit in
  any summation order; this catches a wrong code, slice offset, row or column.
  Shapes cover the 4,096 x 12,288 down projection, ragged k (a last slice of a
  few columns, k not a multiple of 64), ragged n and every m.
* Seeded workloads within |y - y_ref| <= 1e-3 * s_r * sum_j |x_j|.
* Repeated calls, graph replays and two streams with their own workspaces give
  the same bits; every call leaves the workspace all zero.
* Shapes that are not split (m = 1 among them) give exactly
  ternary_gemm_small's result.
* Activations at the fp16 extremes (+-65,504) stay exact: the fixed-point
  combine has the range the header states.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within, ternary_bound

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


def pack(pbg, codes: np.ndarray):
    return pbg.pack_ternary(dev(codes))[0]


def ws_zero(ws: torch.Tensor) -> bool:
    # every accumulator a call used is set back to zero by the slice that completed it
    return int(torch.count_nonzero(ws)) == 0


SHAPES = [(4096, 12288), (2048, 12288), (1000, 12288), (512, 12288), (37, 8200), (2047, 4104), (1024, 16384),
          (300, 16384), (130, 12280), (64, 6000)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_splitk_exact_probe(pbg, n, k):
    codes = synth.ternary_codes(3000 + n + k, n, k)
    s = synth.pow2_scales(3100 + n, n)
    packed = pack(pbg, codes)
    ref_p = oracle.pack(codes)[0]
    ws = pbg.splitk_workspace(n, k, "cuda:0")
    for m in range(1, 9):
        say(f"splitk exact n={n} k={k} m={m}")
        x = synth.probe_activations(3200 + m + k, m, k)
        ref = oracle.ternary_gemm_small(ref_p, s, k, x)
        y = pbg.ternary_gemm_splitk(packed, dev(s), k, dev(x), ws).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, ref), (m, np.argwhere(y != ref)[:5].tolist())
        if m == 1:
            y1 = pbg.ternary_gemm_splitk(packed, dev(s), k, dev(x[0]), ws).cpu().numpy().astype(np.float64)
            assert np.array_equal(y1, ref[0])
        assert ws_zero(ws)


@pytest.mark.parametrize("n,k", [(4096, 12288), (37, 8200)])
def test_splitk_alternating_m_one_workspace(pbg, n, k):
    """Calls with different m use different launch shapes (row blocks of 12
    or 48 rows); alternating them on one workspace must stay exact."""
    codes = synth.ternary_codes(3050 + n, n, k)
    s = synth.pow2_scales(3051 + n, n)
    packed = pack(pbg, codes)
    ref_p = oracle.pack(codes)[0]
    ws = pbg.splitk_workspace(n, k, "cuda:0")
    for i, m in enumerate((8, 1, 3, 1, 8, 2, 5, 1)):
        say(f"splitk alternating n={n} k={k} m={m}")
        x = synth.probe_activations(3060 + i, m, k)
        y = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
        pbg.ternary_gemm_splitk(packed, dev(s), k, dev(x), ws, y)
        assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.ternary_gemm_small(ref_p, s, k, x)), (i, m)
        assert ws_zero(ws)


@pytest.mark.parametrize("n,k", [(64, 16384), (1000, 12288)])
def test_splitk_extreme_activations_exact(pbg, n, k):
    """Every code +1 (or -1 on odd rows) against x = +-65,504: each slice's
    partial is near its largest, and the fixed-point sum must still equal the
    oracle (the exact sum, an integer times 2 ** 5)."""
    say(f"splitk extremes n={n} k={k}")
    codes = np.ones((n, k), dtype=np.int8)
    codes[1::2] = -1
    s = np.full(n, 2.0 ** -20, dtype=np.float32)
    ws = pbg.splitk_workspace(n, k, "cuda:0")
    packed = pack(pbg, codes)
    for m in (2, 8):
        x = np.full((m, k), 65504.0, dtype=np.float16)
        x[1, ::3] = -65504.0
        ref = oracle.ternary_gemm_small(oracle.pack(codes)[0], s, k, x)
        y = pbg.ternary_gemm_splitk(packed, dev(s), k, dev(x), ws).cpu().numpy().astype(np.float64)
        assert np.array_equal(y, ref), m
        assert ws_zero(ws)


@pytest.mark.parametrize("m", [1, 2, 4, 7, 8])
def test_splitk_down_seeded(pbg, m):
    n, k = synth.SHAPES["down"]
    say(f"splitk down seeded m={m}")
    seed = synth.tensor_seed(2, "down")
    codes = synth.ternary_codes(seed, n, k, synth.code_dist(2, "down"))
    s = synth.row_scales(seed, n)
    x = synth.activations(synth.x_seed(0), m, k)
    ref = oracle.ternary_gemm_small(oracle.pack(codes)[0], s, k, x)
    ws = pbg.splitk_workspace(n, k, "cuda:0")
    y = pbg.ternary_gemm_splitk(pack(pbg, codes), dev(s), k, dev(x), ws).cpu().numpy()
    assert_within(y, ref, ternary_bound(s, x), f"splitk down m={m}")


def test_splitk_repeatable_and_graph(pbg):
    n, k, m = 4096, 12288, 8
    say("splitk repeat and graph")
    codes = synth.ternary_codes(3300, n, k)
    packed = pack(pbg, codes)
    s = dev(synth.row_scales(3301, n))
    x = dev(synth.activations(3302, m, k))
    ws = pbg.splitk_workspace(n, k, "cuda:0")
    first = torch.full((m, n), float("nan"), dtype=torch.float32, device="cuda:0")
    pbg.ternary_gemm_splitk(packed, s, k, x, ws, first)
    bound = torch.from_numpy(ternary_bound(s.cpu().numpy(), x.cpu().numpy())).to("cuda:0")
    assert bool(((first - pbg.ternary_gemm_small(packed, s, k, x)).abs() <= 2 * bound).all())
    for _ in range(4):
        assert torch.equal(pbg.ternary_gemm_splitk(packed, s, k, x, ws), first)
    x1 = x[0].clone()
    first1 = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda:0")
    pbg.ternary_gemm_splitk(packed, s, k, x1, ws, first1)
    assert bool(((first1 - pbg.ternary_gemv(packed, s, k, x1)).abs() <= 2 * bound[0]).all())
    y = torch.empty_like(first)
    y1 = torch.empty_like(first1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pbg.ternary_gemm_splitk(packed, s, k, x, ws, y)
        pbg.ternary_gemm_splitk(packed, s, k, x1, ws, y1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pbg.ternary_gemm_splitk(packed, s, k, x, ws, y)
        pbg.ternary_gemm_splitk(packed, s, k, x1, ws, y1)
    for rep in range(4):
        y.fill_(float("nan"))
        y1.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, first) and torch.equal(y1, first1), rep
        assert ws_zero(ws)
        pbg.ternary_gemm_splitk(packed, s, k, x[:3], ws)  # eager work between replays
        torch.cuda.synchronize()


def test_splitk_two_streams(pbg):
    n, k = 4096, 12288
    say("splitk two streams")
    packed = pack(pbg, synth.ternary_codes(3400, n, k))
    s = dev(synth.row_scales(3401, n))
    xs = [dev(synth.activations(3402 + i, 8, k)) for i in range(2)]
    wss = [pbg.splitk_workspace(n, k, "cuda:0") for _ in range(2)]
    refs = [pbg.ternary_gemm_splitk(packed, s, k, xs[i], wss[i]) for i in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    outs = [[torch.empty_like(refs[i]) for _ in range(5)] for i in range(2)]
    for r in range(5):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                pbg.ternary_gemm_splitk(packed, s, k, xs[i], wss[i], outs[i][r])
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(5):
            assert torch.equal(outs[i][r], refs[i]), (i, r)
        assert ws_zero(wss[i])


@pytest.mark.parametrize("n,k,ms", [(500, 4096, (1, 3, 8)), (500, 1000, (1, 3, 8)), (77, 20000, (1, 3, 8)),
                                    (4096, 12288, (1, 2, 3, 4)), (4096, 16384, (2, 8)), (4097, 4104, (2, 8)),
                                    (5000, 12288, (8,))])
def test_splitk_unsplit_shapes_match_small(pbg, n, k, ms):
    """Calls the split does not take (m = 1, k <= 4,096, k > 16,384, and the
    larger n where it measured slower) give exactly ternary_gemm_small's bits."""
    say(f"splitk unsplit n={n} k={k}")
    packed = pack(pbg, synth.ternary_codes(3500 + k, n, k))
    s = dev(synth.row_scales(3501, n))
    ws = pbg.splitk_workspace(n, k, "cuda:0")
    for m in ms:
        x = dev(synth.activations(3502 + m, m, k))
        assert torch.equal(pbg.ternary_gemm_splitk(packed, s, k, x, ws), pbg.ternary_gemm_small(packed, s, k, x))
        assert ws_zero(ws)


def test_splitk_unaligned_x_falls_back(pbg):
    n, k, m = 300, 12288, 4
    say("splitk unaligned x")
    codes = synth.ternary_codes(3600, n, k)
    s = synth.pow2_scales(3601, n)
    x = synth.probe_activations(3602, m, k)
    buf = torch.zeros(m * k + 8, dtype=torch.float16, device="cuda:0")
    xv = buf[1:1 + m * k].view(m, k)
    xv.copy_(dev(x))
    ws = pbg.splitk_workspace(n, k, "cuda:0")
    y = pbg.ternary_gemm_splitk(pack(pbg, codes), dev(s), k, xv, ws).cpu().numpy().astype(np.float64)
    assert np.array_equal(y, oracle.ternary_gemm_small(oracle.pack(codes)[0], s, k, x))


def test_splitk_workspace_too_small(pbg):
    n, k = 4096, 12288
    packed = torch.zeros((n, pbg.words_per_row(k)), dtype=torch.int32, device="cuda:0")
    s = torch.ones(n, dtype=torch.float32, device="cuda:0")
    x = torch.zeros((2, k), dtype=torch.float16, device="cuda:0")
    small = torch.zeros(16, dtype=torch.int64, device="cuda:0")
    with pytest.raises(pbg.PbgError) as e:
        pbg.ternary_gemm_splitk(packed, s, k, x, small)
    assert e.value.code == -6
