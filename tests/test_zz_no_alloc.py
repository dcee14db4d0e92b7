"""int8_head_argmax_noalloc through the C ABI against int8_head_argmax.

The allocation-free entry point keeps the greedy-argmax bins in a device
array the library owns instead of the caller's workspace; it runs the same
kernels, so tokens and logits must equal those of the workspace entry point
bit for bit. Two calls in a row, the second with a smaller input (fewer rows
of the head, a shorter k, fewer activation rows), show that a call leaves the
array ready for the next one.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import synth
from helpers import head_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def pbg(gpu):
    import packed_bit_gemv_amd

    packed_bit_gemv_amd.lib()
    return packed_bit_gemv_amd


def _case(seed: int, n: int, k: int, m: int):
    w = synth.head_weights(seed, n, k)
    s = synth.row_scales(seed + 1, n)
    x = synth.activations(seed + 2, m, k)
    return w, s, x


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


@pytest.mark.parametrize("first,second", [((40000, 4096, 8), (5003, 1024, 3)),
                                          ((9000, 4112, 7), (33, 4096, 1)),
                                          ((2000, 4096, 2), (1000, 1024, 1))])
def test_noalloc_matches_workspace_entry_point(pbg, first, second):
    lib = pbg.lib()
    for n, k, m in (first, second):
        say(f"noalloc argmax n={n} k={k} m={m}")
        w, s, x = _case(700 + n + k + m, n, k, m)
        wd, sd, xd = _dev(w), _dev(s), _dev(x)
        tok = torch.full((m,), -7, dtype=torch.int32, device="cuda:0")
        lg = torch.full((m,), float("nan"), dtype=torch.float32, device="cuda:0")
        stream = torch.cuda.current_stream().cuda_stream
        rc = lib.int8_head_argmax_noalloc(wd.data_ptr(), sd.data_ptr(), n, k, xd.data_ptr(), m, tok.data_ptr(),
                                          lg.data_ptr(), stream)
        assert rc == 0
        keys = torch.zeros(m * pbg.binding.ARGMAX_KEYS_PER_ROW, dtype=torch.int64, device="cuda:0")
        tok_ws, lg_ws = pbg.int8_head_argmax(wd, sd, xd, keys=keys)
        torch.cuda.synchronize()
        assert torch.equal(tok, tok_ws) and torch.equal(lg, lg_ws)
        # and a valid greedy token of the exact logits
        _, y_ref = oracle.int8_head_argmax(w, s, x)
        b = head_bound(w, s, x)
        t = tok.cpu().numpy()
        for i in range(m):
            assert y_ref[i, t[i]] >= np.max(y_ref[i] - b[i]) - b[i, t[i]]


def test_noalloc_rejects_too_many_rows(pbg):
    lib = pbg.lib()
    w = torch.zeros((16, 64), dtype=torch.int8, device="cuda:0")
    s = torch.ones(16, dtype=torch.float32, device="cuda:0")
    x = torch.zeros((9, 64), dtype=torch.float16, device="cuda:0")
    tok = torch.empty(9, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    assert lib.int8_head_argmax_noalloc(w.data_ptr(), s.data_ptr(), 16, 64, x.data_ptr(), 9, tok.data_ptr(), None,
                                        stream) == -2
