"""GPU parity of the SwiGLU feed-forward block with 3-bit linears
(ternary3_ffn_swiglu, ternary3_swiglu_gate_up and their m-row forms) against
the CPU oracle (oracle.ffn3_swiglu) and exact integer arithmetic.

* Five-level integer probes: the 2-bit block's probe (helpers.ffn_probe) with
  the gate codes of rows r = 0 mod 3 and the up codes of rows r = 1 mod 4
  doubled, and five-level down codes. g = +-size or +-2 size (|g| >= 40), u is
  an integer, so h = fp16(g * u) or 0 on both sides and y is an exact integer
  sum: the kernels' h and y must match bit for bit, which catches a wrong
  code, sign, magnitude, row or column in any of the three linears.
* Seeded workload codes: h within the bound that the five-level tolerance on
  g and u implies; y within 1e-3 * s_r * sum_j |c_rj| |h_j| of the oracle's down
  linear on the kernel's own h.
* Repeats and graph replays are bitwise identical to eager calls.
* d_ff = 2^24 (the largest grid), exact.
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import pytest

import oracle
import synth
from helpers import assert_within, ffn_probe, swiglu_h_bound, ternary3_bound

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


def pack3(pbg, codes: np.ndarray):
    return pbg.pack_ternary3(dev(codes))[0]


def probe3(seed: int, d_model: int, d_ff: int):
    """Five-level probe: (x, gate3, up3, down3, h_exp fp16 values as fp64)."""
    x, gate, up, h2 = ffn_probe(seed, d_model, d_ff)
    r = np.arange(d_ff)
    gmul = np.where(r % 3 == 0, 2, 1)
    umul = np.where(r % 4 == 1, 2, 1)
    gate3 = (gate.astype(np.int16) * gmul[:, None]).astype(np.int8)
    up3 = (up.astype(np.int16) * umul[:, None]).astype(np.int8)
    h_exp = (h2 * gmul * umul).astype(np.float16).astype(np.float64)
    down3 = synth.ternary3_codes(seed + 7, d_model, d_ff)
    return x, gate3, up3, down3, h_exp


SHAPES = [(64, 64), (64, 4160), (128, 192), (200 - 8, 8257), (256, 8256), (4096, 128), (192, 12288 + 64),
          (4096, 12288)]


@pytest.mark.parametrize("d_model,d_ff", SHAPES)
def test_ffn3_exact_probe(pbg, d_model, d_ff):
    say(f"ffn3 exact d_model={d_model} d_ff={d_ff}")
    x, gate, up, down, h_exp = probe3(500 + d_model + d_ff, d_model, d_ff)
    sd = synth.pow2_scales(600 + d_model, d_model)
    ones = np.ones(d_ff, dtype=np.float32)
    # every partial sum of the down linear stays an exact fp32 integer
    assert np.all(np.abs(down.astype(np.int64)) @ np.abs(h_exp.astype(np.int64)) < 2 ** 24)
    y_exp = (down.astype(np.int64) @ h_exp.astype(np.int64)).astype(np.float64) * sd.astype(np.float64)
    h, y = pbg.ternary3_ffn_swiglu(pack3(pbg, gate), dev(ones), pack3(pbg, up), dev(ones), pack3(pbg, down), dev(sd),
                                   dev(x))
    assert np.array_equal(h.cpu().numpy().astype(np.float64), h_exp)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_exp)
    if d_model * d_ff <= 1 << 22:
        h_ref, y_ref = oracle.ffn3_swiglu(oracle.pack3(gate)[0], ones, oracle.pack3(up)[0], ones,
                                          oracle.pack3(down)[0], sd, d_model, x)
        assert np.array_equal(h.cpu().numpy(), h_ref[0]) and np.array_equal(y.cpu().numpy().astype(np.float64),
                                                                            y_ref[0])


@pytest.mark.parametrize("m", [2, 3, 5, 8])
@pytest.mark.parametrize("d_model,d_ff", [(64, 64), (128, 4160), (96, 8256), (192, 12288 + 64), (4096, 12288)])
def test_ffn3_small_exact_probe(pbg, m, d_model, d_ff):
    """Row i of x is c_i times the probe's x with c_i in {1, -1, 2, -2}; each row's h and y are exact."""
    say(f"ffn3 small exact m={m} d_model={d_model} d_ff={d_ff}")
    x0, gate, up, down, _ = probe3(700 + d_model + d_ff, d_model, d_ff)
    sd = synth.pow2_scales(800 + d_model, d_model)
    ones = np.ones(d_ff, dtype=np.float32)
    gp, upk, dp = oracle.pack3(gate)[0], oracle.pack3(up)[0], oracle.pack3(down)[0]
    for coef in ([1, -1, 2, -2, 1, 2, -1, -2], [1, -1, 1, -1, -1, 1, 1, -1]):
        c = np.array(coef[:m], dtype=np.float64)
        x = (c[:, None] * x0.astype(np.float64)[None, :]).astype(np.float16)
        h_ref, y_ref = oracle.ffn3_swiglu(gp, ones, upk, ones, dp, sd, d_model, x)
        if np.all(np.abs(down.astype(np.float64)) @ np.abs(h_ref.astype(np.float64)).T < 2 ** 24):
            break
    else:
        pytest.fail("probe sums exceed 2^24")
    h, y = pbg.ternary3_ffn_swiglu(pack3(pbg, gate), dev(ones), pack3(pbg, up), dev(ones), pack3(pbg, down), dev(sd),
                                   dev(x))
    assert tuple(h.shape) == (m, d_ff) and tuple(y.shape) == (m, d_model)
    assert np.array_equal(h.cpu().numpy(), h_ref)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_ref)
    h2 = pbg.ternary3_swiglu_gate_up(pack3(pbg, gate), dev(ones), pack3(pbg, up), dev(ones), d_model, dev(x))
    assert torch.equal(h2, h)


@functools.lru_cache(maxsize=6)
def _workload(layer: int, d_model: int, d_ff: int):
    """Seeded five-level codes of the block and their oracle packs (cached across the m cases)."""
    gate = synth.ternary3_codes(synth.tensor_seed(layer, "gate") + d_ff, d_ff, d_model, synth.code_dist(layer, "gate"))
    up = synth.ternary3_codes(synth.tensor_seed(layer, "up") + d_ff, d_ff, d_model, synth.code_dist(layer, "up"))
    down = synth.ternary3_codes(synth.tensor_seed(layer, "down") + d_ff, d_model, d_ff,
                                synth.code_dist(layer, "down"))
    return gate, up, down, oracle.pack3(gate)[0], oracle.pack3(up)[0], oracle.pack3(down)[0]


@pytest.mark.parametrize("d_model,d_ff", [(64, 64), (72, 67), (128, 4160), (200, 999), (4088, 333), (4096, 12288)])
@pytest.mark.parametrize("m", [1, 2, 4, 7, 8])
def test_ffn3_random_tolerance(pbg, m, d_model, d_ff):
    """Seeded five-level workload codes, x ~ N(0, 1) rows, against the oracle row by row."""
    say(f"ffn3 random m={m} d_model={d_model} d_ff={d_ff}")
    gate, up, down, gp, upk, dp = _workload(1, d_model, d_ff)
    sg, su, sd = synth.row_scales(611, d_ff), synth.row_scales(612, d_ff), synth.row_scales(613, d_model)
    x = synth.activations(synth.x_seed(0), m, d_model)
    xin = dev(x[0]) if m == 1 else dev(x)
    h, y = pbg.ternary3_ffn_swiglu(pack3(pbg, gate), dev(sg), pack3(pbg, up), dev(su), pack3(pbg, down), dev(sd), xin)
    h_gpu = np.atleast_2d(h.cpu().numpy())
    y_gpu = np.atleast_2d(y.cpu().numpy())
    g_ref = oracle.ternary3_gemm_small(gp, sg, d_model, x)
    u_ref = oracle.ternary3_gemm_small(upk, su, d_model, x)
    h_ref = (oracle.silu(g_ref) * u_ref).astype(np.float16)
    assert_within(h_gpu.astype(np.float64), h_ref.astype(np.float64),
                  swiglu_h_bound(oracle.silu(g_ref), u_ref, ternary3_bound(gate, sg, x), ternary3_bound(up, su, x)),
                  "h")
    y_down = oracle.ternary3_gemm_small(dp, sd, d_ff, h_gpu)
    assert_within(y_gpu, y_down, ternary3_bound(down, sd, h_gpu.astype(np.float64)), "y = down h")


def test_ffn3_repeat_and_parts(pbg):
    """Repeated calls are bitwise identical; h is exactly what the gate|up launch gives alone, and y is the
    3-bit GEMV of down on it (m = 1, same bits) or the small-M GEMM (m = 8: down is split over K in two
    slices added onto y, so the sums round differently; within 1e-3 * s_r * 2 * sum_j |h_j|)."""
    d_model, d_ff = 4096, 12288
    say("ffn3 repeat")
    t = {p: pbg.pack_ternary3(synth.ternary3_codes_device(40 + i, *synth.SHAPES[p], synth.GLOBAL_DIST, "cuda:0"))[0]
         for i, p in enumerate(("gate", "up", "down"))}
    s = {p: synth.row_scales_device(50 + i, synth.SHAPES[p][0], "cuda:0") for i, p in enumerate(("gate", "up", "down"))}
    args = (t["gate"], s["gate"], t["up"], s["up"], t["down"], s["down"])
    for m in (1, 8):
        x = dev(synth.activations(60 + m, m, d_model)[0] if m == 1 else synth.activations(60 + m, m, d_model))
        h0, y0 = pbg.ternary3_ffn_swiglu(*args, x)
        for _ in range(3):
            h1, y1 = pbg.ternary3_ffn_swiglu(*args, x)
            assert torch.equal(h0, h1) and torch.equal(y0, y1)
        assert torch.isfinite(y0).all()
        assert torch.equal(pbg.ternary3_swiglu_gate_up(t["gate"], s["gate"], t["up"], s["up"], d_model, x), h0)
        if m == 1:
            assert torch.equal(pbg.ternary3_gemv(t["down"], s["down"], d_ff, h0), y0)
        else:
            y_gemm = pbg.ternary3_gemm_small(t["down"], s["down"], d_ff, h0)
            bound = 1e-3 * s["down"].abs()[None, :] * 2 * h0.float().abs().sum(dim=1, keepdim=True)
            assert bool(((y0 - y_gemm).abs() <= bound).all())


@pytest.mark.parametrize("m", [1, 8])
def test_ffn3_graph_replay(pbg, m):
    """Captured once, replayed with new activations between replays: every replay equals an eager call."""
    d_model, d_ff = 4096, 12288
    say(f"ffn3 graph replay m={m}")
    layer = 3
    t = {p: pbg.pack_ternary3(synth.ternary3_codes_device(synth.tensor_seed(layer, p), *synth.SHAPES[p],
                                                           synth.code_dist(layer, p), "cuda:0"))[0]
         for p in ("gate", "up", "down")}
    s = {p: synth.row_scales_device(synth.tensor_seed(layer, p), synth.SHAPES[p][0], "cuda:0")
         for p in ("gate", "up", "down")}
    args = (t["gate"], s["gate"], t["up"], s["up"], t["down"], s["down"])
    shape_x = (d_model,) if m == 1 else (m, d_model)
    x = torch.empty(shape_x, dtype=torch.float16, device="cuda:0")
    h = torch.empty(shape_x[:-1] + (d_ff,), dtype=torch.float16, device="cuda:0")
    y = torch.empty(shape_x, dtype=torch.float32, device="cuda:0")

    def fresh(seed):
        a = synth.activations(seed, m, d_model)
        x.copy_(dev(a[0] if m == 1 else a))

    fresh(900)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pbg.ternary3_ffn_swiglu(*args, x, h, y)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pbg.ternary3_ffn_swiglu(*args, x, h, y)
    for rep in range(4):
        fresh(901 + rep)
        graph.replay()
        torch.cuda.synchronize()
        h_g, y_g = h.clone(), y.clone()
        h_e, y_e = pbg.ternary3_ffn_swiglu(*args, x)
        torch.cuda.synchronize()
        assert torch.equal(h_g, h_e) and torch.equal(y_g, y_e), rep


@pytest.mark.parametrize("m", [2, 8])
@pytest.mark.parametrize("d_model,d_ff", [(4096, 12288), (96, 8256)])
def test_ffn3_small_y_contents_ignored(pbg, m, d_model, d_ff):
    """As for the 2-bit block: down's two K-slices add onto y after the gate|up launch has cleared it, so
    y's earlier contents (NaN) do not reach the result, and repeated calls give the same bits."""
    say(f"ffn3 small y reuse m={m} d_model={d_model} d_ff={d_ff}")
    gate, up, down, gp, upk, dp = _workload(2, d_model, d_ff)
    sg, su, sd = synth.row_scales(631, d_ff), synth.row_scales(632, d_ff), synth.row_scales(633, d_model)
    x = dev(synth.activations(synth.x_seed(1), m, d_model))
    args = (pack3(pbg, gate), dev(sg), pack3(pbg, up), dev(su), pack3(pbg, down), dev(sd))
    h0, y0 = pbg.ternary3_ffn_swiglu(*args, x)
    h = torch.empty_like(h0)
    y = torch.full_like(y0, float("nan"))
    for _ in range(3):
        pbg.ternary3_ffn_swiglu(*args, x, h, y)
        assert torch.equal(h, h0) and torch.equal(y, y0)
        y.fill_(float("nan"))
    h_gpu = h0.cpu().numpy()
    y_down = oracle.ternary3_gemm_small(dp, sd, d_ff, h_gpu)
    assert_within(y0.cpu().numpy(), y_down, ternary3_bound(down, sd, h_gpu.astype(np.float64)), "y = down h")


def test_ffn3_errors(pbg):
    """Layout checks of the binding and the C ABI's own argument checks on device tensors."""
    d_model, d_ff = 128, 256
    g = pack3(pbg, np.zeros((d_ff, d_model), dtype=np.int8))
    d = pack3(pbg, np.zeros((d_model, d_ff), dtype=np.int8))
    sg = dev(np.ones(d_ff, dtype=np.float32))
    sd = dev(np.ones(d_model, dtype=np.float32))
    x = dev(np.ones(d_model, dtype=np.float16))
    h, y = pbg.ternary3_ffn_swiglu(g, sg, g, sg, d, sd, x)
    torch.cuda.synchronize()
    assert torch.all(h == 0) and torch.all(y == 0)  # zero codes
    g2 = pbg.pack_ternary(dev(np.zeros((d_ff, d_model), dtype=np.int8)))[0]  # the 2-bit layout is narrower
    with pytest.raises(ValueError):
        pbg.ternary3_ffn_swiglu(g2, sg, g2, sg, d, sd, x)
    lib = pbg.lib()
    stream = torch.cuda.current_stream().cuda_stream
    hbuf = torch.empty(d_ff + 8, dtype=torch.float16, device="cuda:0")
    args = (g.data_ptr(), sg.data_ptr(), g.data_ptr(), sg.data_ptr(), d.data_ptr(), sd.data_ptr())
    assert lib.ternary3_ffn_swiglu(*args, d_model, d_ff, x.data_ptr(), hbuf.data_ptr() + 2, y.data_ptr(), stream) == -3
    assert lib.ternary3_ffn_swiglu(*args, d_model, d_ff, x.data_ptr() + 8, hbuf.data_ptr(), y.data_ptr(), stream) == -3
    for dm, dff in ((100, d_ff), (4104, d_ff), (0, d_ff), (d_model, 0)):
        assert lib.ternary3_ffn_swiglu(*args, dm, dff, x.data_ptr(), hbuf.data_ptr(), y.data_ptr(), stream) == -2


def test_ffn3_max_d_ff(pbg):
    """d_ff = 2^24 with d_model = 8 (the largest gate/up grid; down is one
    16M-column row group): integer probe with codes of magnitude 1 and 2 in all
    three linears, h and y exact."""
    d_model, d_ff = 8, 1 << 24
    say(f"ffn3 max d_ff d_model={d_model} d_ff={d_ff}")
    x = np.array([1, -1, 1, 1, -1, 1, -1, -1], dtype=np.float16)
    sx = np.where(x > 0, 1, -1).astype(np.int8)
    # gate rows: sign(x) times 1 or 2 in every column (negated on rows r = 3 mod 5), scale 8, so
    # g = +-64 or +-128; up rows: one code 1 or 2 times sign(x_j) at column j = r % 8, so u = 1 or 2
    gmag = np.array([1, 2, 1, 2, 2], dtype=np.int8)
    gate = gmag[:, None] * sx[None, :]
    gate[3] = -gate[3]
    g_codes = torch.from_numpy(gate).to("cuda:0").repeat((d_ff + 4) // 5, 1)[:d_ff].contiguous()
    rows = torch.arange(d_ff, device="cuda:0")
    cols = rows % d_model
    umag = 1 + (rows // d_model) % 2
    u_codes = torch.zeros((d_ff, d_model), dtype=torch.int8, device="cuda:0")
    u_codes[rows, cols] = (torch.from_numpy(sx).to("cuda:0")[cols] * umag).to(torch.int8)
    del rows, cols, umag
    gs = torch.full((d_ff,), 8.0, dtype=torch.float32, device="cuda:0")
    us = torch.ones(d_ff, dtype=torch.float32, device="cuda:0")
    down = synth.ternary3_codes(48, d_model, d_ff, synth.balanced(0.9995))
    sd = synth.pow2_scales(49, d_model)
    r = np.arange(d_ff)
    # silu(64 or 128) is 64 or 128 exactly in fp32; silu(-128) * u rounds to -0 in fp16
    h_exp = np.where(r % 5 == 3, 0.0, 64.0 * gmag[r % 5] * (1 + (r // d_model) % 2))
    assert np.all(np.abs(down).astype(np.int64) @ h_exp.astype(np.int64) * 2 < 2 ** 24)  # exact fp32 sums
    y_exp = (down.astype(np.int64) @ h_exp.astype(np.int64)).astype(np.float64) * sd.astype(np.float64)
    h, y = pbg.ternary3_ffn_swiglu(pbg.pack_ternary3(g_codes)[0], gs, pbg.pack_ternary3(u_codes)[0], us,
                                   pack3(pbg, down), dev(sd), dev(x))
    del g_codes, u_codes
    assert np.array_equal(h.cpu().numpy().astype(np.float64), h_exp)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), y_exp)
