"""Benchmark of the packed ternary GEMV path on one MI355X.

Headline (one JSON line on stdout): achieved HBM GB/s of the feed-forward
ternary linears at M = 1 (gate and up 12288 x 4096, down 4096 x 12288; codes
with 71 % zeros for gate/down in layers 1-3 and 62.63 % elsewhere, Neutrino-1
8B model page, "Inside the coded lane"), run the way the library runs a
gated (SwiGLU) feed-forward block: ternary_ffn_swiglu = one launch for gate
and up with the SwiGLU in its epilogue, then the down GEMV on its output. One
step = one layer's block on fresh activations; steps walk a pool of 36
distinct synthetic layers (1.37 GB of packed weights, far above the 256 MB
Infinity Cache), so every step streams its weights from HBM.

Also reported under "extra": the same three linears as three separate GEMV
launches, microseconds per linear, per decoder layer (7 linears, and with the
shared-input fusions) and per full decode step (36 layers + int8 head
151,936 x 4,096), the head alone and with the fused greedy argmax, the
small-M (speculative verify) shapes, including the fused layer and one whole
verify step at m = 8, the streaming ceiling of a plain copy (torch) at the
same byte count, and the per-launch floor of a dependent kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "achieved HBM GB/s (% of peak) for packed-ternary GEMV, M=1; µs per decoder layer"
HBM_PEAK_GBS = 8000.0
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_swiglu_gate_up_m1.json")
KERNEL_SOURCES = ("packed_bit_gemv_amd/csrc/ffn.hip", "packed_bit_gemv_amd/csrc/pbg_device.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ternary_bytes(n: int, k: int, m: int = 1) -> int:
    """Algorithmic bytes of one call: packed words + fp32 scales + fp16 x + fp32 y."""
    return synth.words_bytes(n, k) + 4 * n + 2 * m * k + 4 * m * n


def gate_up_bytes(d_ff: int, d_model: int, m: int = 1) -> int:
    """Algorithmic bytes of the gate|up + SwiGLU launch: both packed matrices,
    both scale vectors, x in once, h (fp16) out."""
    return 2 * synth.words_bytes(d_ff, d_model) + 2 * 4 * d_ff + 2 * m * d_model + 2 * m * d_ff


def ffn_block_bytes(d_model: int, d_ff: int, m: int = 1) -> int:
    """Algorithmic bytes of the fused block as it runs: the gate|up launch
    plus the down GEMV on h (packed down, its scales, h in, y out). At
    d_model 4,096, d_ff 12,288, m = 1: 25,296,896 + 12,640,256 = 37,937,152."""
    return gate_up_bytes(d_ff, d_model, m) + ternary_bytes(d_model, d_ff, m)


def ternary3_bytes(n: int, k: int, m: int = 1) -> int:
    """Algorithmic bytes of one 3-bit call: packed rows + fp32 scales + fp16 x + fp32 y."""
    return synth.words3_bytes(n, k) + 4 * n + 2 * m * k + 4 * m * n


def ffn3_block_bytes(d_model: int, d_ff: int, m: int = 1) -> int:
    """Algorithmic bytes of the 3-bit block as it runs: the gate|up launch (both
    3-bit matrices and scales, x in, h out) plus the down launch on h. At
    d_model 4,096, d_ff 12,288, m = 1: 37,879,808 + 18,931,712 = 56,811,520."""
    gate_up = 2 * synth.words3_bytes(d_ff, d_model) + 2 * 4 * d_ff + 2 * m * d_model + 2 * m * d_ff
    return gate_up + ternary3_bytes(d_model, d_ff, m)


def head_bytes(n: int, k: int, m: int = 1) -> int:
    return n * k + 4 * n + 2 * m * k + 4 * m * n


def kernel_hash() -> str:
    """Hash of the GEMV kernel sources with comments and blank lines removed,
    so that stored counter readings are dropped once the code changes."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


class Model:
    """36 synthetic decoder layers of packed ternary linears plus the int8 head."""

    def __init__(self, pbg, torch, device, layers: int, with_head: bool, projs=synth.PROJECTIONS):
        self.layers = []
        stats_buf = torch.empty(4, dtype=torch.int64, device=device)
        for l in range(layers):
            lay = {}
            for p in projs:
                n, k = synth.SHAPES[p]
                seed = synth.tensor_seed(l, p)
                codes = synth.ternary_codes_device(seed, n, k, synth.code_dist(l, p), device)
                packed, _, _ = pbg.pack_ternary(codes, stats=stats_buf, check=False)
                del codes
                lay[p] = (packed, synth.row_scales_device(seed, n, device), n, k)
            self.layers.append(lay)
        self.head = None
        if with_head:
            n, k = synth.HEAD_SHAPE
            self.head = (synth.head_weights_device(synth.SEED_HEAD, n, k, device),
                         synth.row_scales_device(synth.SEED_HEAD, n, device), n, k)
        torch.cuda.synchronize()


def capture(torch, fn):
    """Captures fn() into a HIP graph (fn launches on the current stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# Untimed replays before every timed figure. After an idle gap (a graph
# capture, host work) the chip's power management slows VALU-heavy kernels
# for roughly 3-30 ms of renewed load: the M = 2 head runs 91 us per launch in
# its first ~30 launches, 110-128 us in the next ~150, and 91-92 us from ~400
# on. Timing starts once the figure's own work has run for this long.
SETTLE_S = 50e-3


def time_graphs(torch, graphs, steps: int, warmup: int, settle_s: float | None = None):
    """Replays graphs[i % len] for settle_s seconds (SETTLE_S by default) and
    then warmup times, untimed, then times exactly `steps` replays; ms per replay."""
    settle_s = SETTLE_S if settle_s is None else settle_s
    t0, i = time.perf_counter(), 0
    while settle_s > 0:
        for _ in range(4):
            graphs[i % len(graphs)].replay()
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= settle_s:
            break
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        graphs[(warmup + i) % len(graphs)].replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_baseline(budget_s: float):
    """The CPU oracle timed on this host on a bounded sample of the workload.

    cores = the CPUs this process may run on (its affinity mask); the oracle's
    BLAS matvec is limited to that many threads, its NumPy unpack runs on one.
    The unpack is also timed alone, so that the matvec's share follows.
    """
    import oracle

    cores = len(os.sched_getaffinity(0))
    rows = 1024
    samples = []
    for p in ("gate", "up", "down"):
        n, k = synth.SHAPES[p]
        codes = synth.ternary_codes(synth.tensor_seed(1, p), rows, k, synth.code_dist(1, p))
        samples.append((oracle.pack(codes)[0], synth.row_scales(synth.tensor_seed(1, p), rows), k,
                        synth.activations(synth.x_seed(0), 1, k)[0], rows))

    def run(seconds, fn):
        done, reps, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for packed, s, k, x, r in samples:
                fn(packed, s, k, x)
                done += ternary_bytes(r, k)
            reps += 1
        return done, reps, time.perf_counter() - t0

    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # without it BLAS keeps its own thread count
        threadpool_limits = None

    def limited(threads, seconds, fn):
        if threadpool_limits is None:
            return run(seconds, fn)
        with threadpool_limits(limits=threads):
            return run(seconds, fn)

    done_bytes, reps, dt = limited(cores, budget_s, oracle.ternary_gemv)
    _, u_reps, u_dt = run(budget_s / 6, lambda packed, s, k, x: oracle.unpack(packed, k))
    b1, _, dt1 = limited(1, budget_s / 3, oracle.ternary_gemv)
    blas_threads = cores
    try:
        from threadpoolctl import threadpool_info

        with threadpool_limits(limits=cores):
            blas_threads = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()
                                      if i.get("user_api") == "blas"])
    except Exception:
        pass
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    pass_s, unpack_s = dt / reps, u_dt / u_reps
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{reps} passes over the first {rows} rows of layer-1 gate, up and down (M=1), "
                   f"{dt:.1f} s; unpack in NumPy (1 thread) + fp64 matvec in BLAS ({blas_threads} threads)"),
        "blas_threads": blas_threads,
        "pass_s": round(pass_s, 5),
        "unpack_s": round(unpack_s, 5),
        "matvec_s": round(pass_s - unpack_s, 5),
        "unpack_share": round(unpack_s / pass_s, 3),
        "value_1_thread": round(b1 / dt1 / 1e9, 4),
        "cpu_model": model,
    }


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # 2,000 untimed steps (~25 ms): with 20 the timed steps still ran while the
    # chip's clocks rose (12.2-12.3 against 11.7 us per step, measured)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    # untimed replays before each extra figure (and the roofline launch); 0
    # only for counter runs, whose bytes and instructions do not depend on clocks
    ap.add_argument("--settle-ms", type=float, default=SETTLE_S * 1e3)
    args = ap.parse_args()
    SETTLE_S = args.settle_ms * 1e-3

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the packed ternary GEMV path has no multi-GPU part here "
              "(every published figure is single-device). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import packed_bit_gemv_amd as pbg

    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    log(f"device: {torch.cuda.get_device_name(device)}")
    t0 = time.time()
    model = Model(pbg, torch, device, args.layers, with_head=not args.no_extra,
                  projs=synth.PROJECTIONS if not args.no_extra else ("gate", "up", "down"))
    log(f"model built in {time.time() - t0:.1f} s")

    # Counter calibration: a plain device-to-device copy of exactly the gate's
    # packed byte count, run a few times outside the timed region. Profiling
    # runs read FETCH_SIZE / WRITE_SIZE of this copy to scale the GEMV's.
    calib_bytes = synth.words_bytes(*synth.SHAPES["gate"])
    calib_src = torch.ones(calib_bytes // 4, dtype=torch.int32, device=device)
    calib_dst = torch.empty_like(calib_src)
    for _ in range(3):
        calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    ffn = ("gate", "up", "down")
    xs = {k: torch.from_numpy(synth.activations(synth.x_seed(0), 8, k)).to(device) for k in (synth.HIDDEN, synth.FFN)}
    ys = {p: torch.empty((8, synth.SHAPES[p][0]), dtype=torch.float32, device=device) for p in synth.PROJECTIONS}
    L = len(model.layers)

    # split-K workspace for the down projection at m >= 2 (the entry point
    # splits only where it measured faster, else runs ternary_gemm_small)
    ws_down = pbg.splitk_workspace(*synth.SHAPES["down"], device)

    def linear(layer, p, m=1):
        packed, s, n, k = model.layers[layer][p]
        if m == 1:
            pbg.ternary_gemv(packed, s, k, xs[k][0], ys[p][0])
        elif p == "down":
            pbg.ternary_gemm_splitk(packed, s, k, xs[k][:m], ws_down, ys[p][:m])
        else:
            pbg.ternary_gemm_small(packed, s, k, xs[k][:m], ys[p][:m])

    def ffn_step(layer):
        for p in ffn:
            linear(layer, p)

    h_ff = torch.empty(synth.FFN, dtype=torch.float16, device=device)
    y_ff = torch.empty(synth.HIDDEN, dtype=torch.float32, device=device)

    def ffn_block(layer):
        lay = model.layers[layer]
        pbg.ternary_ffn_swiglu(lay["gate"][0], lay["gate"][1], lay["up"][0], lay["up"][1], lay["down"][0],
                               lay["down"][1], xs[synth.HIDDEN][0], h_ff, y_ff)

    def gate_up(layer):
        lay = model.layers[layer]
        pbg.ternary_swiglu_gate_up(lay["gate"][0], lay["gate"][1], lay["up"][0], lay["up"][1], synth.HIDDEN,
                                   xs[synth.HIDDEN][0], h_ff)

    # ---- headline: the FFN block at M = 1 ------------------------------------
    # Step i runs the block of layer i % L, so consecutive steps stream
    # different weights from HBM. The W warm-up steps are one replayed HIP
    # graph; the K timed steps are one replay of a graph that holds exactly
    # those K steps, bracketed by events on the replay stream.
    W0, K0 = args.warmup, args.steps
    warm = capture(torch, lambda: [ffn_block(i % L) for i in range(W0)]) if W0 > 0 else None
    timed = capture(torch, lambda: [ffn_block((W0 + i) % L) for i in range(K0)])
    # the fused path's own bytes (h written once as fp16 and read back by down)
    bytes_step = ffn_block_bytes(synth.HIDDEN, synth.FFN)
    three_bytes = sum(ternary_bytes(*synth.SHAPES[p]) for p in ffn)  # as three separate GEMVs
    # Untimed, whatever W is: ~20 ms of the same steps first, so that the
    # chip's clocks have settled when the W warm-up and K timed steps run.
    settle = capture(torch, lambda: [ffn_block(i % L) for i in range(L)])
    settle_replays = max(1, round(20e-3 / (L * 12e-6)))
    for _ in range(settle_replays):
        settle.replay()
    settle_steps = settle_replays * L
    del settle
    if warm is not None:
        warm.replay()
    torch.cuda.synchronize()
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    ev_start.record()
    timed.replay()
    ev_end.record()
    torch.cuda.synchronize()
    ms_step = ev_start.elapsed_time(ev_end) / K0
    value = bytes_step / (ms_step * 1e-3) / 1e9
    log(f"ffn block step {ms_step * 1e3:.3f} us, {value:.1f} GB/s")
    del warm, timed

    # dominant kernel of the step: the gate|up + SwiGLU launch, timed alone
    # (a graph of L consecutive launches over the pool)
    g = capture(torch, lambda: [gate_up(l) for l in range(L)])
    gate_up_us = time_graphs(torch, [g], max(5, args.steps // 40), 1) * 1e3 / L
    gu_bytes = gate_up_bytes(synth.FFN, synth.HIDDEN)
    achieved = gu_bytes / (gate_up_us * 1e-6) / 1e9
    del g

    # the same three linears as three separate M = 1 GEMV launches
    g = capture(torch, lambda: [ffn_step(l) for l in range(L)])
    three_us = time_graphs(torch, [g], 5, 1) * 1e3 / L
    del g

    # per-projection launch time: a graph of the same projection over all layers
    per_proj_us = {}
    for p in ffn:
        g = capture(torch, lambda p=p: [linear(l, p) for l in range(L)])
        per_proj_us[p] = time_graphs(torch, [g], 5, 1) * 1e3 / L

    # streaming-read ceiling (pbg_stream_read: the GEMVs' loads, no decode),
    # timed like the launches above: over the pool's packed gate matrices, and
    # over L buffers of the gate|up launch's packed bytes
    sink = torch.zeros(pbg.binding.STREAM_READ_SINK_WORDS, dtype=torch.int32, device=device)
    g = capture(torch, lambda: [pbg.stream_read(model.layers[l]["gate"][0], sink) for l in range(L)])
    read_gate_us = time_graphs(torch, [g], 5, 1) * 1e3 / L
    gu_words = 2 * synth.words_bytes(*synth.SHAPES["gate"]) // 4
    gu_pool = [torch.empty(gu_words, dtype=torch.int32, device=device) for _ in range(L)]
    g = capture(torch, lambda: [pbg.stream_read(gu_pool[l], sink) for l in range(L)])
    read_gu_us = time_graphs(torch, [g], max(5, args.steps // 40), 1) * 1e3 / L
    del g, gu_pool

    traffic, traffic_note = None, "null: the counter reading on file was taken from other kernel source"
    if os.path.exists(PROFILE_TRAFFIC):
        with open(PROFILE_TRAFFIC) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_launch")
            traffic_note = ("stored, not measured in this run: rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, "
                            "scaled by a plain copy's reading, from profiles/traffic_swiglu_gate_up_m1.json; "
                            f"emitted only while the kernel source hash equals the stored one ({tr['kernel_hash']})")

    extra = {"ffn_three_gemv_m1_us": round(three_us, 3),
             "ffn_three_gemv_m1_GBs": round(three_bytes / (three_us * 1e-6) / 1e9, 1),
             "ffn_three_gemv_m1_bytes": three_bytes,
             "swiglu_gate_up_us_per_launch": round(gate_up_us, 3),
             "us_per_launch": {p: round(v, 3) for p, v in per_proj_us.items()},
             "GBs_per_launch": {p: round(ternary_bytes(*synth.SHAPES[p]) / (v * 1e-6) / 1e9, 1)
                                for p, v in per_proj_us.items()},
             "layers_in_pool": L, "pool_bytes_packed": 3 * synth.words_bytes(synth.FFN, synth.HIDDEN) * L,
             "stream_read_us": {"gate_12.6MB": round(read_gate_us, 3), "gate_up_25.2MB": round(read_gu_us, 3)}}

    if not args.no_extra:
        K, W = max(20, args.steps // 4), 5
        layer_bytes = sum(ternary_bytes(*synth.SHAPES[p]) for p in synth.PROJECTIONS)
        for p in ("q", "k", "v", "o"):
            g = capture(torch, lambda p=p: [linear(l, p) for l in range(L)])
            us = time_graphs(torch, [g], 5, 1) * 1e3 / L
            n, k = synth.SHAPES[p]
            extra["us_per_launch"][p] = round(us, 3)
            extra["GBs_per_launch"][p] = round(ternary_bytes(n, k) / (us * 1e-6) / 1e9, 1)
        # read ceiling of the smaller packed shapes: q/o 4.2 MB, k/v 1.0 MB
        for p, label in (("q", "q_4.2MB"), ("k", "k_1.0MB")):
            g = capture(torch, lambda p=p: [pbg.stream_read(model.layers[l][p][0], sink) for l in range(L)])
            extra["stream_read_us"][label] = round(time_graphs(torch, [g], 5, 1) * 1e3 / L, 3)
            del g

        def layer_step(layer, m=1):
            for p in synth.PROJECTIONS:
                linear(layer, p, m)

        layer_graphs = [capture(torch, lambda l=l: layer_step(l)) for l in range(L)]
        ms = time_graphs(torch, layer_graphs, K, W)
        extra["layer_m1_us"] = round(ms * 1e3, 3)
        extra["layer_m1_GBs"] = round(layer_bytes / (ms * 1e-3) / 1e9, 1)
        del layer_graphs

        hw, hs, hn, hk = model.head
        yh = torch.empty((8, hn), dtype=torch.float32, device=device)

        def head(m=1):
            pbg.int8_head_gemv(hw, hs, xs[hk][:m], yh[:m])

        # 8 launches per graph, so that a graph's own launch (~6 us here) is
        # amortised as in the other per-launch figures; the 622 MB head does
        # not fit the Infinity Cache, so every launch streams it from HBM
        HL = 8
        for m in (1, 2, 4, 7, 8):
            g = capture(torch, lambda m=m: [head(m) for _ in range(HL)])
            ms = time_graphs(torch, [g], 8, 2) / HL
            extra[f"head_m{m}_us"] = round(ms * 1e3, 2)
            extra[f"head_m{m}_GBs"] = round(head_bytes(hn, hk, m) / (ms * 1e-3) / 1e9, 1)

        g = capture(torch, lambda: [pbg.stream_read(hw, sink) for _ in range(HL)])
        extra["stream_read_us"]["head_622MB"] = round(time_graphs(torch, [g], 8, 2) / HL * 1e3, 2)
        del g

        def decode_step():
            for l in range(L):
                layer_step(l)
            head(1)

        g = capture(torch, decode_step)
        ms = time_graphs(torch, [g], 5, 1)
        dec_bytes = layer_bytes * L + head_bytes(hn, hk)
        extra["decode_step_m1_us"] = round(ms * 1e3, 1)
        extra["decode_step_m1_GBs"] = round(dec_bytes / (ms * 1e-3) / 1e9, 1)
        del g

        # the down projection alone at m = 8: the plain small-M GEMM and the K-split one
        for label, fn in (("down_m8_plain_us", lambda l: pbg.ternary_gemm_small(
                              model.layers[l]["down"][0], model.layers[l]["down"][1], synth.FFN, xs[synth.FFN][:8],
                              ys["down"][:8])),
                          ("down_m8_splitk_us", lambda l: linear(l, "down", 8))):
            g = capture(torch, lambda fn=fn: [fn(l) for l in range(L)])
            extra[label] = round(time_graphs(torch, [g], 5, 1) * 1e3 / L, 3)
            del g

        for m in (2, 4, 7, 8):
            graphs = [capture(torch, lambda l=l, m=m: layer_step(l, m)) for l in range(L)]
            ms = time_graphs(torch, graphs, K, W)
            lb = sum(ternary_bytes(*synth.SHAPES[p], m) for p in synth.PROJECTIONS)
            extra[f"layer_m{m}_us"] = round(ms * 1e3, 3)
            extra[f"layer_m{m}_GBs"] = round(lb / (ms * 1e-3) / 1e9, 1)
            del graphs

        # greedy token through the head (logits never written)
        keys = torch.zeros(8 * pbg.binding.ARGMAX_KEYS_PER_ROW, dtype=torch.int64, device=device)
        tok = torch.empty(8, dtype=torch.int32, device=device)
        lgt = torch.empty(8, dtype=torch.float32, device=device)
        for m in (1, 7, 8):
            g = capture(torch, lambda m=m: [pbg.int8_head_argmax(hw, hs, xs[hk][:m], keys, tok[:m], lgt[:m])
                                            for _ in range(HL)])
            ms = time_graphs(torch, [g], 8, 2) / HL
            extra[f"head_argmax_m{m}_us"] = round(ms * 1e3, 2)
            extra[f"head_argmax_m{m}_GBs"] = round(head_bytes(hn, hk, m) / (ms * 1e-3) / 1e9, 1)
            del g

        # pack_ternary (load time, not per token): the gate shape over a pool of 8
        # code tensors (403 MB of int8 codes, above the Infinity Cache)
        n, k = synth.SHAPES["gate"]
        codes_pool = [synth.ternary_codes_device(synth.tensor_seed(l, "gate"), n, k, synth.code_dist(l, "gate"),
                                                 device) for l in range(8)]
        pk = torch.empty((n, pbg.words_per_row(k)), dtype=torch.int32, device=device)
        rs = torch.empty(n, dtype=torch.int32, device=device)
        stt = torch.empty(4, dtype=torch.int64, device=device)
        g = capture(torch, lambda: [pbg.pack_ternary(c, pk, rs, stt, check=False) for c in codes_pool])
        ms = time_graphs(torch, [g], 5, 1) / len(codes_pool)
        pb = n * k + synth.words_bytes(n, k) + 4 * n + 32  # codes in; words, row sums and counts out
        extra["pack_gate_us"] = round(ms * 1e3, 2)
        extra["pack_gate_GBs"] = round(pb / (ms * 1e-3) / 1e9, 1)
        del g, codes_pool, pk, rs, stt

        # the embedding row of each token (int8 row x row scale, 4 KiB read per
        # token); the head tensor stands in for the input embedding, which has
        # the same shape and type
        for m in (1, 8):
            ids = np.random.default_rng(synth.SEED_HEAD + m).integers(0, hn, m).astype(np.int32)
            toks = torch.from_numpy(ids).to(device)
            emb = torch.empty((m, hk), dtype=torch.float32, device=device)
            g = capture(torch, lambda toks=toks, emb=emb: [pbg.int8_embedding_gather(hw, hs, toks, emb)
                                                           for _ in range(36)])
            ms = time_graphs(torch, [g], 5, 1) / 36
            eb = m * (hk + 4 + 4 + 4 * hk)  # row, scale and id in; fp32 row out
            extra[f"embedding_m{m}_us"] = round(ms * 1e3, 3)
            extra[f"embedding_m{m}_GBs"] = round(eb / (ms * 1e-3) / 1e9, 1)
            del g, toks, emb

        # shared-input fusions: q|k|v as one packed matrix (row concatenation of
        # packs with the same K is itself a pack), o, then the FFN block
        fused = []
        for l in range(L):
            lay = model.layers[l]
            fused.append((torch.cat([lay[p][0] for p in ("q", "k", "v")]),
                          torch.cat([lay[p][1] for p in ("q", "k", "v")])))
        y_qkv = torch.empty(fused[0][0].shape[0], dtype=torch.float32, device=device)

        def fused_layer(l):
            qp, qs = fused[l]
            pbg.ternary_gemv(qp, qs, synth.HIDDEN, xs[synth.HIDDEN][0], y_qkv)
            linear(l, "o")
            ffn_block(l)

        graphs = [capture(torch, lambda l=l: fused_layer(l)) for l in range(L)]
        ms = time_graphs(torch, graphs, K, W)
        extra["layer_fused_m1_us"] = round(ms * 1e3, 3)
        extra["layer_fused_m1_GBs"] = round(layer_bytes / (ms * 1e-3) / 1e9, 1)
        g = capture(torch, lambda: [fused_layer(l) for l in range(L)])
        ms = time_graphs(torch, [g], 5, 1) / L
        extra["layer_fused_m1_us_36_per_graph"] = round(ms * 1e3, 3)
        extra["layer_fused_m1_GBs_36_per_graph"] = round(layer_bytes / (ms * 1e-3) / 1e9, 1)

        def decode_fused():
            for l in range(L):
                fused_layer(l)
            head(1)

        g = capture(torch, decode_fused)
        ms = time_graphs(torch, [g], 5, 1)
        extra["decode_step_fused_m1_us"] = round(ms * 1e3, 1)
        extra["decode_step_fused_m1_GBs"] = round(dec_bytes / (ms * 1e-3) / 1e9, 1)
        del graphs, g

        # the fused layer at the speculative-verify shapes: q|k|v and o as small-M
        # GEMMs, the FFN block with m activation rows (gate|up + SwiGLU, then down)
        yqkv_m = torch.empty((8, fused[0][0].shape[0]), dtype=torch.float32, device=device)
        h_m = torch.empty((8, synth.FFN), dtype=torch.float16, device=device)
        y_m = torch.empty((8, synth.HIDDEN), dtype=torch.float32, device=device)

        def fused_layer_m(l, m):
            qp, qs = fused[l]
            pbg.ternary_gemm_small(qp, qs, synth.HIDDEN, xs[synth.HIDDEN][:m], yqkv_m[:m])
            linear(l, "o", m)
            lay = model.layers[l]
            # the block: gate|up + SwiGLU for m rows, then down on h (split over K in two slices added
            # onto y, which the gate|up launch clears)
            pbg.ternary_ffn_swiglu(lay["gate"][0], lay["gate"][1], lay["up"][0], lay["up"][1], lay["down"][0],
                                   lay["down"][1], xs[synth.HIDDEN][:m], h_m[:m], y_m[:m])

        for m in (2, 4, 7, 8):
            graphs = [capture(torch, lambda l=l, m=m: fused_layer_m(l, m)) for l in range(L)]
            ms = time_graphs(torch, graphs, K, W)
            lb = sum(ternary_bytes(*synth.SHAPES[p], m) for p in synth.PROJECTIONS)
            extra[f"layer_fused_m{m}_us"] = round(ms * 1e3, 3)
            extra[f"layer_fused_m{m}_GBs"] = round(lb / (ms * 1e-3) / 1e9, 1)
            g = capture(torch, lambda m=m: [fused_layer_m(l, m) for l in range(L)])
            ms = time_graphs(torch, [g], 5, 1) / L
            extra[f"layer_fused_m{m}_us_36_per_graph"] = round(ms * 1e3, 3)
            extra[f"layer_fused_m{m}_GBs_36_per_graph"] = round(lb / (ms * 1e-3) / 1e9, 1)
            del graphs, g

        # one speculative verify step: 36 fused layers and the greedy token of
        # each of the 8 rows through the head, one graph
        def verify_step():
            for l in range(L):
                fused_layer_m(l, 8)
            pbg.int8_head_argmax(hw, hs, xs[hk][:8], keys, tok, lgt)

        g = capture(torch, verify_step)
        ms = time_graphs(torch, [g], 5, 1)
        vb = L * sum(ternary_bytes(*synth.SHAPES[p], 8) for p in synth.PROJECTIONS) + head_bytes(hn, hk, 8)
        extra["verify_step_fused_m8_us"] = round(ms * 1e3, 1)
        extra["verify_step_fused_m8_GBs"] = round(vb / (ms * 1e-3) / 1e9, 1)
        del g, fused, yqkv_m, h_m, y_m

        # the 3-bit lane (five-level codes, the shipped lane's 72,351,744 bytes
        # of weights per layer): a pool of L layers of the 7 linears, per-linear
        # launches, the read of their packed bytes, and whole layers at M = 1 and 8
        pool3, fused3 = [], []
        st6 = torch.empty(6, dtype=torch.int64, device=device)
        for l in range(L):
            lay, qkv = {}, []
            for p in synth.PROJECTIONS:
                n, k = synth.SHAPES[p]
                seed = synth.tensor_seed(l, p)
                codes = synth.ternary3_codes_device(seed, n, k, synth.code_dist(l, p), device)
                lay[p] = (pbg.pack_ternary3(codes, stats=st6, check=False)[0], synth.row_scales_device(seed, n, device),
                          n, k)
                if p in ("q", "k", "v"):
                    qkv.append(codes)
                del codes
            # q|k|v as one 6,144-row pack (one launch for the three linears of the same x)
            cat = torch.cat(qkv)
            fused3.append((pbg.pack_ternary3(cat, stats=st6, check=False)[0],
                           torch.cat([lay[p][1] for p in ("q", "k", "v")])))
            del qkv, cat
            pool3.append(lay)
        torch.cuda.synchronize()

        def linear3(l, p, m=1):
            packed, s, n, k = pool3[l][p]
            if m == 1:
                pbg.ternary3_gemv(packed, s, k, xs[k][0], ys[p][0])
            else:
                pbg.ternary3_gemm_small(packed, s, k, xs[k][:m], ys[p][:m])

        lane3 = {"us_per_launch": {}, "GBs_per_launch": {}, "stream_read_us": {}}
        for p in synth.PROJECTIONS:
            n, k = synth.SHAPES[p]
            g = capture(torch, lambda p=p: [linear3(l, p) for l in range(L)])
            us = time_graphs(torch, [g], 5, 1) * 1e3 / L
            lane3["us_per_launch"][p] = round(us, 3)
            lane3["GBs_per_launch"][p] = round(ternary3_bytes(n, k) / (us * 1e-6) / 1e9, 1)
            del g
        for p in ("gate", "down", "q", "k"):
            g = capture(torch, lambda p=p: [pbg.stream_read(pool3[l][p][0], sink) for l in range(L)])
            lane3["stream_read_us"][p] = round(time_graphs(torch, [g], 5, 1) * 1e3 / L, 3)
            del g
        layer3_weights = sum(synth.words3_bytes(*synth.SHAPES[p]) for p in synth.PROJECTIONS)
        lane3["layer_weight_bytes"] = layer3_weights
        for m in (1, 8):
            graphs = [capture(torch, lambda l=l, m=m: [linear3(l, p, m) for p in synth.PROJECTIONS])
                      for l in range(L)]
            ms = time_graphs(torch, graphs, K, W)
            lb = sum(ternary3_bytes(*synth.SHAPES[p], m) for p in synth.PROJECTIONS)
            lane3[f"layer_m{m}_us"] = round(ms * 1e3, 3)
            lane3[f"layer_m{m}_GBs"] = round(lb / (ms * 1e-3) / 1e9, 1)
            del graphs
            g = capture(torch, lambda m=m: [linear3(l, p, m) for l in range(L) for p in synth.PROJECTIONS])
            ms = time_graphs(torch, [g], 5, 1) / L
            lane3[f"layer_m{m}_us_36_per_graph"] = round(ms * 1e3, 3)
            lane3[f"layer_m{m}_GBs_36_per_graph"] = round(lb / (ms * 1e-3) / 1e9, 1)
            del g
        # the SwiGLU block with 3-bit linears (gate|up + SwiGLU in one launch, then
        # down on h), and the fused layer: q|k|v pack, o, the block (4 launches)
        h3 = torch.empty((8, synth.FFN), dtype=torch.float16, device=device)
        y3 = torch.empty((8, synth.HIDDEN), dtype=torch.float32, device=device)
        yqkv3 = torch.empty((8, fused3[0][0].shape[0]), dtype=torch.float32, device=device)

        def ffn3_block(l, m=1):
            lay = pool3[l]
            xin = xs[synth.HIDDEN][0] if m == 1 else xs[synth.HIDDEN][:m]
            pbg.ternary3_ffn_swiglu(lay["gate"][0], lay["gate"][1], lay["up"][0], lay["up"][1], lay["down"][0],
                                    lay["down"][1], xin, h3[0] if m == 1 else h3[:m], y3[0] if m == 1 else y3[:m])

        def fused_layer3(l, m=1):
            qp, qs = fused3[l]
            if m == 1:
                pbg.ternary3_gemv(qp, qs, synth.HIDDEN, xs[synth.HIDDEN][0], yqkv3[0])
            else:
                pbg.ternary3_gemm_small(qp, qs, synth.HIDDEN, xs[synth.HIDDEN][:m], yqkv3[:m])
            linear3(l, "o", m)
            ffn3_block(l, m)

        for m in (1, 8):
            g = capture(torch, lambda m=m: [ffn3_block(l, m) for l in range(L)])
            us = time_graphs(torch, [g], 5, 1) * 1e3 / L
            fb = ffn3_block_bytes(synth.HIDDEN, synth.FFN, m)
            lane3[f"ffn_block_m{m}_us"] = round(us, 3)
            lane3[f"ffn_block_m{m}_GBs"] = round(fb / (us * 1e-6) / 1e9, 1)
            del g
            lb = sum(ternary3_bytes(*synth.SHAPES[p], m) for p in synth.PROJECTIONS)
            g = capture(torch, lambda m=m: [fused_layer3(l, m) for l in range(L)])
            ms = time_graphs(torch, [g], 5, 1) / L
            lane3[f"layer_fused_m{m}_us_36_per_graph"] = round(ms * 1e3, 3)
            lane3[f"layer_fused_m{m}_GBs_36_per_graph"] = round(lb / (ms * 1e-3) / 1e9, 1)
            del g
        extra["lane3"] = lane3
        del pool3, fused3, h3, y3, yqkv3

        # streaming-read ceiling at the gate byte count: torch copy over a pool
        nbytes = synth.words_bytes(*synth.SHAPES["gate"])
        pool = [torch.empty(nbytes // 4, dtype=torch.int32, device=device) for _ in range(48)]
        dst = torch.empty(nbytes // 4, dtype=torch.int32, device=device)
        g = capture(torch, lambda: [dst.copy_(pool[i]) for i in range(48)])
        ms = time_graphs(torch, [g], 5, 1) / 48
        extra["copy_12.6MB_us"] = round(ms * 1e3, 3)
        extra["copy_12.6MB_GBs_read_plus_write"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
        del pool, dst, g

        # per-launch floor of a dependent kernel in a graph: 36 launches of a
        # one-element kernel, timed like the per-linear figures
        one = torch.zeros(1, dtype=torch.float32, device=device)
        g = capture(torch, lambda: [one.add_(1.0) for _ in range(36)])
        ms = time_graphs(torch, [g], 20, 2) / 36
        extra["launch_floor_us"] = round(ms * 1e3, 3)
        del g, one

    # each linear at M = 1 against the HBM peak: its fraction, and the time a
    # launch would take at 75 % of the peak (the per-linear goal)
    extra["frac_of_peak_per_launch"] = {p: round(v / HBM_PEAK_GBS, 4) for p, v in extra["GBs_per_launch"].items()}
    extra["us_at_75pct_of_peak"] = {p: round(ternary_bytes(*synth.SHAPES[p]) / (0.75 * HBM_PEAK_GBS * 1e3), 3)
                                    for p in extra["GBs_per_launch"]}

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16*ternary->f32",
        "data": "synthetic",
        "config": {
            "workload": "ffn_gate_up_down_m1",
            "shapes": {p: list(synth.SHAPES[p]) for p in ffn},
            "m": 1,
            "layers_in_pool": L,
            "us_per_step": round(ms_step * 1e3, 3),
            "bytes_per_step": bytes_step,
            "path": "ternary_ffn_swiglu: gate|up + SwiGLU in one launch, then the down GEMV on its fp16 output",
            "untimed": f"{settle_steps} settle steps (~20 ms, for the clocks) then the {args.warmup} warm-up steps",
            "extra_settle_ms": args.settle_ms,
            "plain_three_gemv": {"us_per_step": round(three_us, 3),
                                 "GBs": round(three_bytes / (three_us * 1e-6) / 1e9, 1),
                                 "bytes_per_step": three_bytes},
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_note": traffic_note,
            "kernel": "swiglu_gate_up_kernel",
            "bytes_per_launch": gu_bytes,
            "avg_launch_us": round(gate_up_us, 3),
            "read_ceiling_us": round(read_gu_us, 3),
            "frac_of_read_ceiling": round(read_gu_us / gate_up_us, 4),
            "read_ceiling_note": "pbg_stream_read of the launch's packed bytes (25,165,824 B): the GEMVs' loads "
                                 "alone, one launch each, timed the same way",
            "launch_us_note": f"HIP events around a replayed graph of {L} consecutive launches over the pool, "
                              f"divided by {L} (inter-launch gaps included), after {args.settle_ms:g} ms of "
                              f"untimed replays",
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(args.cpu_budget),
        "extra": extra,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
