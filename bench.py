"""Benchmark of the packed ternary GEMV path on one MI355X.

Headline (one JSON line on stdout): achieved HBM GB/s of the feed-forward
ternary GEMVs at M = 1 (gate and up 12288 x 4096, down 4096 x 12288; codes
with 71 % zeros for gate/down in layers 1-3 and 62.63 % elsewhere, Neutrino-1 8B
model page, "Inside the coded lane"). One step = one decoder layer's three FFN
GEMVs on fresh activations; steps walk a pool of 36 distinct synthetic layers
(1.37 GB of packed weights, far above the 256 MB Infinity Cache), so every
step streams its weights from HBM.

Also reported under "extra": microseconds per linear, per decoder layer (7
linears) and per full decode step (36 layers + int8 head 151,936 x 4,096), the
head alone, and the small-M (speculative verify) shapes, plus the streaming
read ceiling of a plain copy (torch) at the same byte count.
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
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_ternary_gemv_ffn_m1.json")
CHUNK = 12  # steps per replayed graph in the timed region
KERNEL_SOURCES = ("packed_bit_gemv_amd/csrc/ternary.hip", "packed_bit_gemv_amd/csrc/pbg_device.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ternary_bytes(n: int, k: int, m: int = 1) -> int:
    """Algorithmic bytes of one call: packed words + fp32 scales + fp16 x + fp32 y."""
    return synth.words_bytes(n, k) + 4 * n + 2 * m * k + 4 * m * n


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


def time_graphs(torch, graphs, steps: int, warmup: int):
    """Replays graphs[i % len] warmup times, then times exactly `steps` replays; ms per replay."""
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
    """The CPU oracle timed on this host on a bounded sample of the workload."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([1] + [int(i.get("num_threads", 1)) for i in threadpool_info()])
    except Exception:
        threads = 1
    rows = 1024
    samples = []
    for p in ("gate", "up", "down"):
        n, k = synth.SHAPES[p]
        codes = synth.ternary_codes(synth.tensor_seed(1, p), rows, k, synth.code_dist(1, p))
        samples.append((oracle.pack(codes)[0], synth.row_scales(synth.tensor_seed(1, p), rows), k,
                        synth.activations(synth.x_seed(0), 1, k)[0], rows))
    done_bytes = 0
    reps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        for packed, s, k, x, r in samples:
            oracle.ternary_gemv(packed, s, k, x)
            done_bytes += ternary_bytes(r, k)
        reps += 1
    dt = time.perf_counter() - t0
    return {
        "value": round(done_bytes / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{reps} passes over the first {rows} rows of layer-1 gate, up and down (M=1), "
                   f"{dt:.1f} s; unpack in NumPy (1 thread) + fp64 matvec in BLAS ({threads} threads)"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args()

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

    def linear(layer, p, m=1):
        packed, s, n, k = model.layers[layer][p]
        if m == 1:
            pbg.ternary_gemv(packed, s, k, xs[k][0], ys[p][0])
        else:
            pbg.ternary_gemm_small(packed, s, k, xs[k][:m], ys[p][:m])

    def ffn_step(layer):
        for p in ffn:
            linear(layer, p)

    # ---- headline: FFN GEMVs at M = 1 ---------------------------------------
    # Steps are replayed from HIP graphs: step i runs the gate, up and down
    # GEMVs of layer i % L, so consecutive steps stream different weights from
    # HBM. Runs of CHUNK steps that start at a multiple of CHUNK replay one
    # graph of 3 * CHUNK launches; other steps replay a one-step graph, so
    # exactly `steps` steps are timed. Events on the replay stream bracket the
    # timed region.
    chunk = CHUNK if L % CHUNK == 0 else 1
    single = [capture(torch, lambda l=l: ffn_step(l)) for l in range(L)]
    chunked = [capture(torch, lambda c=c: [ffn_step(c * chunk + j) for j in range(chunk)])
               for c in range(L // chunk)]

    def replay_steps(first, count):
        i = first
        while i < first + count:
            if chunk > 1 and i % chunk == 0 and i + chunk <= first + count:
                chunked[(i % L) // chunk].replay()
                i += chunk
            else:
                single[i % L].replay()
                i += 1

    bytes_step = sum(ternary_bytes(*synth.SHAPES[p]) for p in ffn)
    replay_steps(0, args.warmup)
    torch.cuda.synchronize()
    ev_start = torch.cuda.Event(enable_timing=True)
    ev_end = torch.cuda.Event(enable_timing=True)
    ev_start.record()
    replay_steps(args.warmup, args.steps)
    ev_end.record()
    torch.cuda.synchronize()
    ms_step = ev_start.elapsed_time(ev_end) / args.steps
    value = bytes_step / (ms_step * 1e-3) / 1e9
    avg_launch_us = ms_step * 1e3 / len(ffn)
    achieved = bytes_step / len(ffn) / (avg_launch_us * 1e-6) / 1e9
    log(f"ffn step {ms_step * 1e3:.3f} us, {value:.1f} GB/s; {avg_launch_us:.3f} us per launch")
    del single, chunked

    # per-projection launch time: a graph of the same projection over all layers
    per_proj_us = {}
    for p in ffn:
        g = capture(torch, lambda p=p: [linear(l, p) for l in range(L)])
        per_proj_us[p] = time_graphs(torch, [g], 5, 1) * 1e3 / L

    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        with open(PROFILE_TRAFFIC) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_launch")

    extra = {"us_per_launch": {p: round(v, 3) for p, v in per_proj_us.items()},
             "GBs_per_launch": {p: round(ternary_bytes(*synth.SHAPES[p]) / (v * 1e-6) / 1e9, 1)
                                for p, v in per_proj_us.items()},
             "layers_in_pool": L, "pool_bytes_packed": bytes_step * L}

    if not args.no_extra:
        K, W = max(20, args.steps // 4), 5
        layer_bytes = sum(ternary_bytes(*synth.SHAPES[p]) for p in synth.PROJECTIONS)
        for p in ("q", "k", "v", "o"):
            g = capture(torch, lambda p=p: [linear(l, p) for l in range(L)])
            us = time_graphs(torch, [g], 5, 1) * 1e3 / L
            n, k = synth.SHAPES[p]
            extra["us_per_launch"][p] = round(us, 3)
            extra["GBs_per_launch"][p] = round(ternary_bytes(n, k) / (us * 1e-6) / 1e9, 1)

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

        for m in (1, 2, 4, 7, 8):
            g = capture(torch, lambda m=m: head(m))
            ms = time_graphs(torch, [g], 10, 2)
            extra[f"head_m{m}_us"] = round(ms * 1e3, 2)
            extra[f"head_m{m}_GBs"] = round(head_bytes(hn, hk, m) / (ms * 1e-3) / 1e9, 1)

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

        for m in (2, 4, 7, 8):
            graphs = [capture(torch, lambda l=l, m=m: layer_step(l, m)) for l in range(L)]
            ms = time_graphs(torch, graphs, K, W)
            lb = sum(ternary_bytes(*synth.SHAPES[p], m) for p in synth.PROJECTIONS)
            extra[f"layer_m{m}_us"] = round(ms * 1e3, 3)
            extra[f"layer_m{m}_GBs"] = round(lb / (ms * 1e-3) / 1e9, 1)
            del graphs

        # greedy token through the head (logits never written)
        keys = torch.empty(8, dtype=torch.int64, device=device)
        tok = torch.empty(8, dtype=torch.int32, device=device)
        lgt = torch.empty(8, dtype=torch.float32, device=device)
        for m in (1, 7):
            g = capture(torch, lambda m=m: pbg.int8_head_argmax(hw, hs, xs[hk][:m], keys[:m], tok[:m], lgt[:m]))
            ms = time_graphs(torch, [g], 10, 2)
            extra[f"head_argmax_m{m}_us"] = round(ms * 1e3, 2)
            extra[f"head_argmax_m{m}_GBs"] = round(head_bytes(hn, hk, m) / (ms * 1e-3) / 1e9, 1)
            del g

        # shared-input fusion: q|k|v and gate|up as one packed matrix each
        # (row concatenation of packs with the same K is itself a pack)
        fused = []
        for l in range(L):
            lay = model.layers[l]
            qkv = (torch.cat([lay[p][0] for p in ("q", "k", "v")]), torch.cat([lay[p][1] for p in ("q", "k", "v")]))
            gu = (torch.cat([lay[p][0] for p in ("gate", "up")]), torch.cat([lay[p][1] for p in ("gate", "up")]))
            fused.append((qkv, gu))
        y_qkv = torch.empty(fused[0][0][0].shape[0], dtype=torch.float32, device=device)
        y_gu = torch.empty(fused[0][1][0].shape[0], dtype=torch.float32, device=device)

        def fused_ffn(l):
            (gp, gs) = fused[l][1]
            pbg.ternary_gemv(gp, gs, synth.HIDDEN, xs[synth.HIDDEN][0], y_gu)
            linear(l, "down")

        def fused_layer(l):
            (qp, qs) = fused[l][0]
            pbg.ternary_gemv(qp, qs, synth.HIDDEN, xs[synth.HIDDEN][0], y_qkv)
            linear(l, "o")
            fused_ffn(l)

        ffn_bytes = sum(ternary_bytes(*synth.SHAPES[p]) for p in ffn)
        graphs = [capture(torch, lambda l=l: fused_ffn(l)) for l in range(L)]
        ms = time_graphs(torch, graphs, K, W)
        extra["ffn_fused_m1_us"] = round(ms * 1e3, 3)
        extra["ffn_fused_m1_GBs"] = round(ffn_bytes / (ms * 1e-3) / 1e9, 1)
        g = capture(torch, lambda: [fused_ffn(l) for l in range(L)])
        ms = time_graphs(torch, [g], 5, 1) / L
        extra["ffn_fused_m1_us_36_per_graph"] = round(ms * 1e3, 3)
        extra["ffn_fused_m1_GBs_36_per_graph"] = round(ffn_bytes / (ms * 1e-3) / 1e9, 1)
        g = capture(torch, lambda: [fused_layer(l) for l in range(L)])
        ms = time_graphs(torch, [g], 5, 1) / L
        extra["layer_fused_m1_us"] = round(ms * 1e3, 3)
        extra["layer_fused_m1_GBs"] = round(layer_bytes / (ms * 1e-3) / 1e9, 1)
        del graphs, g, fused

        # streaming-read ceiling at the gate byte count: torch copy over a pool
        nbytes = synth.words_bytes(*synth.SHAPES["gate"])
        pool = [torch.empty(nbytes // 4, dtype=torch.int32, device=device) for _ in range(48)]
        dst = torch.empty(nbytes // 4, dtype=torch.int32, device=device)
        g = capture(torch, lambda: [dst.copy_(pool[i]) for i in range(48)])
        ms = time_graphs(torch, [g], 5, 1) / 48
        extra["copy_12.6MB_us"] = round(ms * 1e3, 3)
        extra["copy_12.6MB_GBs_read_plus_write"] = round(2 * nbytes / (ms * 1e-3) / 1e9, 1)
        del pool, dst, g

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel": "ternary_gemv_kernel",
            "avg_launch_us": round(avg_launch_us, 3),
            "launch_us_note": "timed-region time / launches; HIP graphs of 12 steps (36 launches), gaps included",
        },
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(args.cpu_budget),
        "extra": extra,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
