"""The benchmark's host-side contract, without a GPU: the byte accounting
behind every GB/s figure, and the refusal to run on more than one GPU.

The expected byte counts are worked out by hand from the Qwen3-8B shapes on
the Neutrino-1 8B model page (geometry table; per-row scales, "Where the
bytes live"): packed N * K / 4 + fp32 scales + fp16 x + fp32 y, and for the
int8 head N * K + scales + x + y.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


@pytest.mark.parametrize("proj,expected", [("gate", 12_689_408), ("up", 12_689_408), ("down", 12_640_256),
                                           ("q", 4_235_264), ("o", 4_235_264), ("k", 1_064_960),
                                           ("v", 1_064_960)])
def test_linear_bytes_m1(proj, expected):
    assert bench.ternary_bytes(*synth.SHAPES[proj]) == expected


def test_layer_and_small_m_bytes():
    layer = sum(bench.ternary_bytes(*synth.SHAPES[p]) for p in ("q", "k", "v", "o", "gate", "up", "down"))
    assert layer == 48_619_520
    assert bench.ternary_bytes(*synth.SHAPES["gate"], 8) == 13_090_816
    assert bench.ternary_bytes(*synth.SHAPES["down"], 8) == 12_926_976
    assert 36 * layer + bench.head_bytes(151_936, 4096) == 2_373_856_256  # one decode step


def test_head_bytes():
    assert bench.head_bytes(151_936, 4096) == 623_553_536
    assert bench.head_bytes(151_936, 4096, 8) == 627_865_088


def test_gate_up_launch_bytes():
    # both packed matrices, both scale vectors, x once and the fp16 h
    assert bench.gate_up_bytes(synth.FFN, synth.HIDDEN) == 2 * 12_582_912 + 2 * 4 * 12_288 + 2 * 4096 + 2 * 12_288
    assert bench.gate_up_bytes(synth.FFN, synth.HIDDEN) == 25_296_896


def test_ffn_block_bytes():
    # the fused block as it runs: the gate|up launch, then down on the fp16 h
    # (12,582,912 packed + 16,384 scales + 24,576 h in + 16,384 y out)
    assert bench.ffn_block_bytes(synth.HIDDEN, synth.FFN) == 25_296_896 + 12_640_256 == 37_937_152
    # three separate GEMVs would move 81,920 B more: x read twice more, g and u written as fp32
    three = sum(bench.ternary_bytes(*synth.SHAPES[p]) for p in ("gate", "up", "down"))
    assert three - bench.ffn_block_bytes(synth.HIDDEN, synth.FFN) == 81_920
    # m rows: x and h scale with m, the weights do not
    assert bench.ffn_block_bytes(synth.HIDDEN, synth.FFN, 8) == (3 * 12_582_912 + 2 * 4 * 12_288 + 4 * 4096
                                                                 + 8 * (2 * 4096 + 2 * 12_288 + 2 * 12_288
                                                                        + 4 * 4096))


def test_lane3_bytes():
    # the 3-bit rows of the seven linears are the shipped lane's 72,351,744 bytes per layer
    weights = sum(synth.words3_bytes(*synth.SHAPES[p]) for p in synth.PROJECTIONS)
    assert weights == 72_351_744
    assert bench.ternary3_bytes(*synth.SHAPES["gate"]) == 12288 * 1536 + 4 * 12288 + 2 * 4096 + 4 * 12288
    assert bench.ternary3_bytes(*synth.SHAPES["down"], 8) == 4096 * 4608 + 4 * 4096 + 8 * (2 * 12288 + 4 * 4096)
    # the 3-bit block: both 3-bit gate|up matrices and scales, x in, h out; then down on h
    assert bench.ffn3_block_bytes(synth.HIDDEN, synth.FFN) == (2 * 12288 * 1536 + 2 * 4 * 12288 + 2 * 4096
                                                               + 2 * 12288 + 4096 * 4608 + 4 * 4096 + 2 * 12288
                                                               + 4 * 4096) == 56_811_520


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                          text=True, timeout=300, cwd=ROOT)
    assert proc.returncode == 2
    assert "one GPU" in proc.stdout + proc.stderr
    assert proc.stdout.strip() == "" or not proc.stdout.strip().startswith("{")
