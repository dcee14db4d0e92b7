"""GPU parity of ternary_ffn_swiglu (gated feed-forward block in one launch)
against the CPU oracle and against exact integer arithmetic.

* Integer probes (tests/helpers.ffn_probe): h and y are known exactly, so the
  kernel's h and y must match bit for bit; this catches any single wrong code,
  sign, row or column in all three linears.
* Seeded workloads: h within the bound that the ternary tolerance on g and u
  implies (helpers.swiglu_h_bound); y within 1e-3 * s_r * sum_j |h_j| of the
  oracle's down linear applied to the kernel's own h.
* Repeated calls and graph replays give identical results.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within, ffn_probe, swiglu_h_bound, ternary_bound

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


def h_host(h) -> np.ndarray:
    return h.cpu().numpy().astype(np.float64)


SHAPES = [(64, 64), (64, 4160), (72, 67), (128, 192), (200, 8257), (256, 8256), (4096, 128), (4088, 333),
          (192, 12288 + 64), (4096, 12288), (1024, 24576)]


@pytest.mark.parametrize("d_model,d_ff", SHAPES)
def test_ffn_exact_probe(pbg, d_model, d_ff):
    say(f"ffn exact d_model={d_model} d_ff={d_ff}")
    x, gate, up, h_exp = ffn_probe(100 + d_model + d_ff, d_model, d_ff)
    down = synth.ternary_codes(200 + d_model + d_ff, d_model, d_ff)
    sd = synth.pow2_scales(300 + d_model, d_model)
    ones = np.ones(d_ff, dtype=np.float32)
    # every partial sum of the down linear stays an exact fp32 integer
    assert np.all(np.abs(down.astype(np.int64)) @ np.abs(h_exp) < 2 ** 24)
    y_exp = (down.astype(np.int64) @ h_exp).astype(np.float64) * sd.astype(np.float64)
    h, y = pbg.ternary_ffn_swiglu(pack(pbg, gate), dev(ones), pack(pbg, up), dev(ones), pack(pbg, down), dev(sd),
                                  dev(x))
    assert np.array_equal(h_host(h), h_exp.astype(np.float64))
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_exp)
    if d_model * d_ff <= 1 << 22:
        h_ref, y_ref = oracle.ffn_swiglu(oracle.pack(gate)[0], ones, oracle.pack(up)[0], ones, oracle.pack(down)[0],
                                         sd, d_model, x)
        assert np.array_equal(h_host(h), h_ref[0].astype(np.float64))
        assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref[0])


@pytest.mark.parametrize("d_model,d_ff", [(64, 64), (128, 4160), (200, 999), (256, 1024), (4096, 12288)])
def test_ffn_random_tolerance(pbg, d_model, d_ff):
    """Seeded workload codes (early-layer gate and down, as in the benchmark), x ~ N(0, 1)."""
    say(f"ffn random d_model={d_model} d_ff={d_ff}")
    layer = 1
    gate = synth.ternary_codes(synth.tensor_seed(layer, "gate") + d_ff, d_ff, d_model, synth.code_dist(layer, "gate"))
    up = synth.ternary_codes(synth.tensor_seed(layer, "up") + d_ff, d_ff, d_model, synth.code_dist(layer, "up"))
    down = synth.ternary_codes(synth.tensor_seed(layer, "down") + d_ff, d_model, d_ff,
                               synth.code_dist(layer, "down"))
    sg, su = synth.row_scales(601, d_ff), synth.row_scales(602, d_ff)
    sd = synth.row_scales(603, d_model)
    x = synth.activations(synth.x_seed(0), 1, d_model)[0]
    gp, upk, dp = oracle.pack(gate)[0], oracle.pack(up)[0], oracle.pack(down)[0]
    h, y = pbg.ternary_ffn_swiglu(pack(pbg, gate), dev(sg), pack(pbg, up), dev(su), pack(pbg, down), dev(sd), dev(x))
    h_gpu = h.cpu().numpy()
    g_ref = oracle.ternary_gemv(gp, sg, d_model, x)
    u_ref = oracle.ternary_gemv(upk, su, d_model, x)
    h_ref, y_ref = oracle.ffn_swiglu(gp, sg, upk, su, dp, sd, d_model, x)
    tg = ternary_bound(sg, x)[0]
    tu = ternary_bound(su, x)[0]
    assert_within(h_gpu.astype(np.float64), h_ref[0].astype(np.float64),
                  swiglu_h_bound(oracle.silu(g_ref), u_ref, tg, tu), "h")
    y_down = oracle.ternary_gemv(dp, sd, d_ff, h_gpu)
    assert_within(y.cpu().numpy()[None], y_down[None], ternary_bound(sd, h_gpu), "y = down h")
    # against the oracle's own h: add what the difference in h can move y by
    dh = np.abs(h_gpu.astype(np.float64) - h_ref[0].astype(np.float64))
    extra = np.abs(down.astype(np.float64)) @ dh * sd.astype(np.float64)
    assert_within(y.cpu().numpy()[None], y_ref, ternary_bound(sd, h_gpu) + extra[None], "y")


def test_ffn_full_size_sampled(pbg):
    """Full gate/up/down tensors from the benchmark's device generator; sampled rows against the oracle."""
    d_model, d_ff = synth.SHAPES["down"]
    layer = 2
    say("ffn full-size sampled")
    codes = {p: synth.ternary_codes_device(synth.tensor_seed(layer, p), *synth.SHAPES[p], synth.code_dist(layer, p),
                                           "cuda:0") for p in ("gate", "up", "down")}
    scales = {p: synth.row_scales_device(synth.tensor_seed(layer, p), synth.SHAPES[p][0], "cuda:0")
              for p in ("gate", "up", "down")}
    x = synth.activations(synth.x_seed(0), 1, d_model)[0]
    packed = {p: pbg.pack_ternary(codes[p])[0] for p in codes}
    h, y = pbg.ternary_ffn_swiglu(packed["gate"], scales["gate"], packed["up"], scales["up"], packed["down"],
                                  scales["down"], dev(x))
    h_gpu, y_gpu = h.cpu().numpy(), y.cpu().numpy()
    rng = np.random.Generator(np.random.PCG64(9))
    rows = np.sort(rng.choice(d_ff, size=256, replace=False))
    idx = torch.from_numpy(rows).to("cuda:0")
    sg, su = scales["gate"].cpu().numpy()[rows], scales["up"].cpu().numpy()[rows]
    gp = oracle.pack(codes["gate"][idx].cpu().numpy())[0]
    upk = oracle.pack(codes["up"][idx].cpu().numpy())[0]
    g_ref = oracle.ternary_gemv(gp, sg, d_model, x)
    u_ref = oracle.ternary_gemv(upk, su, d_model, x)
    h_ref = (oracle.silu(g_ref) * u_ref).astype(np.float16)
    assert_within(h_gpu[rows].astype(np.float64), h_ref.astype(np.float64),
                  swiglu_h_bound(oracle.silu(g_ref), u_ref, ternary_bound(sg, x)[0], ternary_bound(su, x)[0]), "h")
    drows = np.sort(rng.choice(d_model, size=256, replace=False))
    didx = torch.from_numpy(drows).to("cuda:0")
    sd = scales["down"].cpu().numpy()[drows]
    y_down = oracle.ternary_gemv(oracle.pack(codes["down"][didx].cpu().numpy())[0], sd, d_ff, h_gpu)
    assert_within(y_gpu[drows][None], y_down[None], ternary_bound(sd, h_gpu), "y")


def test_ffn_repeat(pbg):
    d_model, d_ff = 4096, 12288
    say("ffn repeat")
    g = pbg.pack_ternary(synth.ternary_codes_device(11, d_ff, d_model, synth.GLOBAL_DIST, "cuda:0"))[0]
    u = pbg.pack_ternary(synth.ternary_codes_device(12, d_ff, d_model, synth.GLOBAL_DIST, "cuda:0"))[0]
    d = pbg.pack_ternary(synth.ternary_codes_device(13, d_model, d_ff, synth.GLOBAL_DIST, "cuda:0"))[0]
    sg = synth.row_scales_device(14, d_ff, "cuda:0")
    su = synth.row_scales_device(15, d_ff, "cuda:0")
    sd = synth.row_scales_device(16, d_model, "cuda:0")
    x = dev(synth.activations(17, 1, d_model)[0])
    h0, y0 = pbg.ternary_ffn_swiglu(g, sg, u, su, d, sd, x)
    for i in range(5):
        h1, y1 = pbg.ternary_ffn_swiglu(g, sg, u, su, d, sd, x)
        assert torch.equal(h0, h1) and torch.equal(y0, y1)
    assert torch.isfinite(y0).all()
    # h is exactly the input the down GEMV sees: the M = 1 GEMV on it gives y bit for bit,
    # and the gate/up launch alone gives the same h
    assert torch.equal(pbg.ternary_gemv(d, sd, d_ff, h0), y0)
    assert torch.equal(pbg.ternary_swiglu_gate_up(g, sg, u, su, d_model, x), h0)


def test_ffn_graph_replay(pbg):
    """Captured once, replayed with new activations between replays: every replay equals an eager call."""
    d_model, d_ff = 4096, 12288
    say("ffn graph replay")
    g = pbg.pack_ternary(synth.ternary_codes_device(21, d_ff, d_model, synth.GLOBAL_DIST, "cuda:0"))[0]
    u = pbg.pack_ternary(synth.ternary_codes_device(22, d_ff, d_model, synth.GLOBAL_DIST, "cuda:0"))[0]
    d = pbg.pack_ternary(synth.ternary_codes_device(23, d_model, d_ff, synth.GLOBAL_DIST, "cuda:0"))[0]
    sg = synth.row_scales_device(24, d_ff, "cuda:0")
    su = synth.row_scales_device(25, d_ff, "cuda:0")
    sd = synth.row_scales_device(26, d_model, "cuda:0")
    x = torch.empty(d_model, dtype=torch.float16, device="cuda:0")
    h = torch.empty(d_ff, dtype=torch.float16, device="cuda:0")
    y = torch.empty(d_model, dtype=torch.float32, device="cuda:0")
    x.copy_(dev(synth.activations(27, 1, d_model)[0]))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        pbg.ternary_ffn_swiglu(g, sg, u, su, d, sd, x, h, y)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pbg.ternary_ffn_swiglu(g, sg, u, su, d, sd, x, h, y)
    for rep in range(4):
        x.copy_(dev(synth.activations(30 + rep, 1, d_model)[0]))
        graph.replay()
        torch.cuda.synchronize()
        h_g, y_g = h.clone(), y.clone()
        h_e, y_e = pbg.ternary_ffn_swiglu(g, sg, u, su, d, sd, x)
        torch.cuda.synchronize()
        assert torch.equal(h_g, h_e) and torch.equal(y_g, y_e), rep


def test_ffn_errors(pbg):
    d_model, d_ff = 128, 256
    g = pack(pbg, np.zeros((d_ff, d_model), dtype=np.int8))
    d = pack(pbg, np.zeros((d_model, d_ff), dtype=np.int8))
    sg = dev(np.ones(d_ff, dtype=np.float32))
    sd = dev(np.ones(d_model, dtype=np.float32))
    x = dev(np.ones(d_model, dtype=np.float16))
    lib = pbg.lib()
    stream = torch.cuda.current_stream().cuda_stream
    hbuf = torch.zeros(d_ff + 8, dtype=torch.float16, device="cuda:0")
    y = torch.full((d_model,), 7.0, dtype=torch.float32, device="cuda:0")
    args = [g.data_ptr(), sg.data_ptr(), g.data_ptr(), sg.data_ptr(), d.data_ptr(), sd.data_ptr()]
    assert lib.ternary_ffn_swiglu(*args, d_model, d_ff, x.data_ptr(), hbuf.data_ptr(), y.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 0)  # zero codes
    assert lib.ternary_ffn_swiglu(*args, d_model, d_ff, x.data_ptr(), hbuf.data_ptr() + 2, y.data_ptr(), stream) == -3
    assert lib.ternary_ffn_swiglu(*args, d_model, d_ff, x.data_ptr() + 8, hbuf.data_ptr(), y.data_ptr(), stream) == -3
    assert lib.ternary_ffn_swiglu(*args, d_model, d_ff, x.data_ptr(), None, y.data_ptr(), stream) == -1
    for dm, dff in ((100, d_ff), (4104, d_ff), (0, d_ff), (d_model, 0), (d_model, 2 ** 24 + 1)):
        assert lib.ternary_ffn_swiglu(*args, dm, dff, x.data_ptr(), hbuf.data_ptr(), y.data_ptr(), stream) == -2


# --------------------------------------------------------------------------
# The block for 2 <= m <= 8 activation rows (speculative verify)
# --------------------------------------------------------------------------
SMALL_SHAPES = [(64, 64), (128, 4160), (256, 1024), (96, 8200), (192, 12288 + 64), (4096, 12288)]


@pytest.mark.parametrize("m", [2, 3, 5, 8])
@pytest.mark.parametrize("d_model,d_ff", SMALL_SHAPES)
def test_ffn_small_exact_probe(pbg, m, d_model, d_ff):
    """Row i of x is c_i times the integer probe x0 with c_i in {1, -1, 2, -2}: every gate sum is 0 or
    |g| >= 40, where silu(g) is g or rounds h to zero, so h and y are exact on both sides and equal
    the oracle bit for bit (the down sums stay below 2^24, checked)."""
    say(f"ffn small exact m={m} d_model={d_model} d_ff={d_ff}")
    x0, gate, up, _ = ffn_probe(100 + d_model + d_ff, d_model, d_ff)
    down = synth.ternary_codes(200 + d_model + d_ff, d_model, d_ff)
    sd = synth.pow2_scales(300 + d_model, d_model)
    ones = np.ones(d_ff, dtype=np.float32)
    gp, upk, dp = oracle.pack(gate)[0], oracle.pack(up)[0], oracle.pack(down)[0]
    for coef in ([1, -1, 2, -2, 1, 2, -1, -2], [1, -1, 1, -1, -1, 1, 1, -1]):
        c = np.array(coef[:m], dtype=np.float64)
        x = (c[:, None] * x0.astype(np.float64)[None, :]).astype(np.float16)
        h_ref, y_ref = oracle.ffn_swiglu(gp, ones, upk, ones, dp, sd, d_model, x)
        if np.all(np.abs(down.astype(np.float64)) @ np.abs(h_ref.astype(np.float64)).T < 2 ** 24):
            break
    else:
        pytest.fail("probe sums exceed 2^24")
    h, y = pbg.ternary_ffn_swiglu(pack(pbg, gate), dev(ones), pack(pbg, up), dev(ones), pack(pbg, down), dev(sd),
                                  dev(x))
    assert tuple(h.shape) == (m, d_ff) and tuple(y.shape) == (m, d_model)
    assert np.array_equal(h_host(h), h_ref.astype(np.float64))
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)
    h2 = pbg.ternary_swiglu_gate_up(pack(pbg, gate), dev(ones), pack(pbg, up), dev(ones), d_model, dev(x))
    assert torch.equal(h2, h)


@pytest.mark.parametrize("m", [2, 4, 7, 8])
@pytest.mark.parametrize("d_model,d_ff", [(128, 4160), (200, 999), (4096, 12288)])
def test_ffn_small_random_tolerance(pbg, m, d_model, d_ff):
    """Seeded workload codes and x ~ N(0, 1) rows against the oracle, row by row, with the m = 1 bounds."""
    say(f"ffn small random m={m} d_model={d_model} d_ff={d_ff}")
    layer = 1
    gate = synth.ternary_codes(synth.tensor_seed(layer, "gate") + d_ff, d_ff, d_model, synth.code_dist(layer, "gate"))
    up = synth.ternary_codes(synth.tensor_seed(layer, "up") + d_ff, d_ff, d_model, synth.code_dist(layer, "up"))
    down = synth.ternary_codes(synth.tensor_seed(layer, "down") + d_ff, d_model, d_ff,
                               synth.code_dist(layer, "down"))
    sg, su, sd = synth.row_scales(611, d_ff), synth.row_scales(612, d_ff), synth.row_scales(613, d_model)
    x = synth.activations(synth.x_seed(0), m, d_model)
    gp, upk, dp = oracle.pack(gate)[0], oracle.pack(up)[0], oracle.pack(down)[0]
    h, y = pbg.ternary_ffn_swiglu(pack(pbg, gate), dev(sg), pack(pbg, up), dev(su), pack(pbg, down), dev(sd), dev(x))
    h_gpu = h.cpu().numpy()
    g_ref = oracle.ternary_gemm_small(gp, sg, d_model, x)
    u_ref = oracle.ternary_gemm_small(upk, su, d_model, x)
    h_ref = (oracle.silu(g_ref) * u_ref).astype(np.float16)
    assert_within(h_gpu.astype(np.float64), h_ref.astype(np.float64),
                  swiglu_h_bound(oracle.silu(g_ref), u_ref, ternary_bound(sg, x), ternary_bound(su, x)), "h")
    y_down = oracle.ternary_gemm_small(dp, sd, d_ff, h_gpu)
    assert_within(y.cpu().numpy(), y_down, ternary_bound(sd, h_gpu), "y = down h")


def test_ffn_small_graph_replay(pbg):
    """The m = 8 block captured once and replayed on fresh activations equals eager calls."""
    d_model, d_ff, m = 4096, 12288, 8
    say("ffn small graph replay")
    layer = 3
    t = {p: pbg.pack_ternary(synth.ternary_codes_device(synth.tensor_seed(layer, p), *synth.SHAPES[p],
                                                         synth.code_dist(layer, p), "cuda:0"))[0]
         for p in ("gate", "up", "down")}
    s = {p: synth.row_scales_device(synth.tensor_seed(layer, p), synth.SHAPES[p][0], "cuda:0")
         for p in ("gate", "up", "down")}
    x = dev(synth.activations(801, m, d_model))
    h = torch.empty((m, d_ff), dtype=torch.float16, device="cuda:0")
    y = torch.empty((m, d_model), dtype=torch.float32, device="cuda:0")
    args = (t["gate"], s["gate"], t["up"], s["up"], t["down"], s["down"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pbg.ternary_ffn_swiglu(*args, x, h, y)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pbg.ternary_ffn_swiglu(*args, x, h, y)
    for rep in range(4):
        x.copy_(dev(synth.activations(802 + rep, m, d_model)))
        graph.replay()
        torch.cuda.synchronize()
        h_e, y_e = pbg.ternary_ffn_swiglu(*args, x)
        torch.cuda.synchronize()
        assert torch.equal(h, h_e) and torch.equal(y, y_e), rep


@pytest.mark.parametrize("m", [2, 8])
@pytest.mark.parametrize("d_model,d_ff", [(4096, 12288), (96, 8200), (128, 4160)])
def test_ffn_small_y_contents_ignored(pbg, m, d_model, d_ff):
    """The block's down linear adds its K-slices onto y after the gate|up launch
    has cleared it: whatever y held before (NaN here) does not reach the result,
    and repeated calls give the same bits."""
    say(f"ffn small y reuse m={m} d_model={d_model} d_ff={d_ff}")
    layer = 2
    gate = synth.ternary_codes(synth.tensor_seed(layer, "gate") + d_ff, d_ff, d_model, synth.code_dist(layer, "gate"))
    up = synth.ternary_codes(synth.tensor_seed(layer, "up") + d_ff, d_ff, d_model, synth.code_dist(layer, "up"))
    down = synth.ternary_codes(synth.tensor_seed(layer, "down") + d_ff, d_model, d_ff,
                               synth.code_dist(layer, "down"))
    sg, su, sd = synth.row_scales(621, d_ff), synth.row_scales(622, d_ff), synth.row_scales(623, d_model)
    x = dev(synth.activations(synth.x_seed(1), m, d_model))
    args = (pack(pbg, gate), dev(sg), pack(pbg, up), dev(su), pack(pbg, down), dev(sd))
    h0, y0 = pbg.ternary_ffn_swiglu(*args, x)
    h = torch.empty_like(h0)
    y = torch.full_like(y0, float("nan"))
    for _ in range(3):
        pbg.ternary_ffn_swiglu(*args, x, h, y)
        assert torch.equal(h, h0) and torch.equal(y, y0)
        y.fill_(float("nan"))
    h_gpu = h0.cpu().numpy()
    y_down = oracle.ternary_gemm_small(oracle.pack(down)[0], sd, d_ff, h_gpu)
    assert_within(y0.cpu().numpy(), y_down, ternary_bound(sd, h_gpu), "y = down h")

