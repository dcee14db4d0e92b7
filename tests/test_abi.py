"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments before any HIP call.

The calls below use fake pointer values that always fail validation; they are
never made when a GPU is visible, so no kernel can be launched on them.
"""
from __future__ import annotations

import ctypes

import pytest

from packed_bit_gemv_amd import binding

GOOD = 0x10000  # 64 KiB aligned fake address, never dereferenced
HOST_GPU = None


def _gpu_visible() -> bool:
    global HOST_GPU
    if HOST_GPU is None:
        try:
            import torch

            HOST_GPU = bool(torch.cuda.is_available())
        except Exception:
            HOST_GPU = False
    return HOST_GPU


no_gpu_only = pytest.mark.skipif("_gpu_visible()", reason="fake-pointer calls are only made without a GPU")


def test_exports_every_header_function():
    names = binding.header_functions()
    assert set(names) >= {"pack_ternary", "ternary_gemv", "ternary_gemm_small", "int8_head_gemv",
                          "int8_head_argmax", "int8_embedding_gather",
                          "pbg_abi_version", "pbg_strerror", "pbg_words_per_row"}
    lib = binding.lib()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(binding._SIGNATURES)


def test_helpers():
    lib = binding.lib()
    assert lib.pbg_abi_version() == 2
    for k, w in [(1, 4), (64, 4), (65, 8), (4096, 256), (12288, 768), (0, 0), (-5, 0)]:
        assert lib.pbg_words_per_row(k) == w
    for code in range(-6, 1):
        assert lib.pbg_strerror(code)
    assert lib.pbg_strerror(-99) == b"unknown error code"
    # split-K workspace: one 8-byte accumulator per output, at most 8 activation rows, row blocks
    # of at most 64 rows; 0 for an invalid shape
    assert lib.pbg_splitk_workspace_bytes(4096, 12288) == 8 * 8 * (4096 + 64)
    assert lib.pbg_splitk_workspace_bytes(8, 4096) == 8 * 8 * 72
    assert lib.pbg_splitk_workspace_bytes(0, 4096) == 0 and lib.pbg_splitk_workspace_bytes(8, 0) == 0


@no_gpu_only
def test_null_pointers():
    lib = binding.lib()
    assert lib.ternary_gemv(None, GOOD, 4, 64, GOOD, GOOD, None) == -1
    assert lib.ternary_gemv(GOOD, GOOD, 4, 64, None, GOOD, None) == -1
    assert lib.ternary_gemm_small(GOOD, None, 4, 64, GOOD, 2, GOOD, None) == -1
    assert lib.int8_head_gemv(GOOD, GOOD, 4, 64, GOOD, 1, None, None) == -1
    assert lib.pack_ternary(GOOD, 4, 64, GOOD, GOOD, None, None, None) == -1
    assert lib.int8_head_argmax(GOOD, GOOD, 4, 64, GOOD, 1, None, GOOD, None, None) == -1
    assert lib.int8_head_argmax(GOOD, GOOD, 4, 64, GOOD, 1, GOOD, None, None, None) == -1
    assert lib.int8_embedding_gather(GOOD, GOOD, 4, 64, None, 2, GOOD, None) == -1


@no_gpu_only
@pytest.mark.parametrize("n,k,m", [(0, 64, 1), (4, 0, 1), (-1, 64, 1), (4, 64, 0), (4, 64, 9),
                                   (2 ** 24 + 1, 64, 1), (4, 2 ** 24 + 1, 1)])
def test_bad_shapes(n, k, m):
    lib = binding.lib()
    assert lib.ternary_gemm_small(GOOD, GOOD, n, k, GOOD, m, GOOD, None) == -2
    assert lib.int8_head_gemv(GOOD, GOOD, n, k, GOOD, m, GOOD, None) == -2
    assert lib.int8_head_argmax(GOOD, GOOD, n, k, GOOD, m, GOOD, GOOD, None, None) == -2
    if m == 1:
        assert lib.ternary_gemv(GOOD, GOOD, n, k, GOOD, GOOD, None) == -2
        assert lib.pack_ternary(GOOD, n, k, GOOD, GOOD, GOOD, None, None) == -2


@no_gpu_only
def test_misaligned():
    lib = binding.lib()
    assert lib.ternary_gemv(GOOD + 4, GOOD, 4, 64, GOOD, GOOD, None) == -3
    assert lib.ternary_gemv(GOOD, GOOD + 2, 4, 64, GOOD, GOOD, None) == -3
    assert lib.ternary_gemv(GOOD, GOOD, 4, 64, GOOD + 1, GOOD, None) == -3
    assert lib.ternary_gemv(GOOD, GOOD, 4, 64, GOOD, GOOD + 2, None) == -3
    assert lib.int8_head_gemv(GOOD + 8, GOOD, 4, 64, GOOD, 1, GOOD, None) == -3
    assert lib.ternary_gemm_small(GOOD + 8, GOOD, 4, 64, GOOD, 2, GOOD, None) == -3
    assert lib.pack_ternary(GOOD, 4, 64, GOOD + 4, GOOD, GOOD, None, None) == -3
    assert lib.pack_ternary(GOOD, 4, 64, GOOD, GOOD, GOOD + 4, None, None) == -3
    assert lib.int8_head_argmax(GOOD, GOOD, 4, 64, GOOD, 1, GOOD + 4, GOOD, None, None) == -3
    assert lib.int8_head_argmax(GOOD, GOOD, 4, 64, GOOD, 1, GOOD, GOOD + 2, None, None) == -3
    assert lib.int8_embedding_gather(GOOD + 1, GOOD + 2, 4, 64, GOOD, 2, GOOD, None) == -3
    assert lib.int8_embedding_gather(GOOD, GOOD, 4, 64, GOOD + 2, 2, GOOD, None) == -3


@no_gpu_only
def test_embedding_shapes():
    lib = binding.lib()
    assert lib.int8_embedding_gather(GOOD, GOOD, 4, 64, GOOD, 0, GOOD, None) == -2
    assert lib.int8_embedding_gather(GOOD, GOOD, 0, 64, GOOD, 2, GOOD, None) == -2
    assert lib.int8_embedding_gather(GOOD, GOOD, 4, 4096, GOOD, 2 ** 22, GOOD, None) == -2


def test_binding_rejects_cpu_tensors():
    import torch

    with pytest.raises(ValueError):
        binding.ternary_gemv(torch.zeros((4, 4), dtype=torch.int32), torch.zeros(4), 64,
                             torch.zeros(64, dtype=torch.float16))


def test_strerror_is_static():
    lib = binding.lib()
    a = ctypes.cast(lib.pbg_strerror(-1), ctypes.c_char_p)
    assert a.value == b"a required pointer is NULL"


@no_gpu_only
@pytest.mark.parametrize("prefix", ["ternary", "ternary3"])
def test_ffn_validation(prefix):
    lib = binding.lib()
    ffn, gate_up = getattr(lib, f"{prefix}_ffn_swiglu"), getattr(lib, f"{prefix}_swiglu_gate_up")
    p6 = [GOOD] * 6
    assert ffn(None, *p6[1:], 4096, 12288, GOOD, GOOD, GOOD, None) == -1
    assert ffn(*p6, 4096, 12288, GOOD, GOOD, None, None) == -1
    for dm, dff in ((0, 12288), (4096 + 8, 12288), (100, 12288), (4, 12288), (4096, 0), (4096, 2 ** 24 + 1)):
        assert ffn(*p6, dm, dff, GOOD, GOOD, GOOD, None) == -2
    assert ffn(*p6, 4096, 12288, GOOD + 8, GOOD, GOOD, None) == -3   # x
    assert ffn(*p6, 4096, 12288, GOOD, GOOD + 2, GOOD, None) == -3   # h
    assert ffn(*p6, 4096, 12288, GOOD, GOOD, GOOD + 2, None) == -3   # y
    assert ffn(GOOD + 4, *p6[1:], 4096, 12288, GOOD, GOOD, GOOD, None) == -3
    assert gate_up(GOOD, GOOD, GOOD, GOOD, 4096, 12288, GOOD, None, None) == -1
    assert gate_up(GOOD, GOOD, GOOD, GOOD, 4100, 12288, GOOD, GOOD, None) == -2
    assert gate_up(GOOD, GOOD, GOOD, GOOD, 4096, 12288, GOOD, GOOD + 2, None) == -3


@pytest.mark.parametrize("prefix", ["ternary", "ternary3"])
def test_ffn_small_validation(prefix):
    lib = binding.lib()
    ffn, gate_up = getattr(lib, f"{prefix}_ffn_swiglu_small"), getattr(lib, f"{prefix}_swiglu_gate_up_small")
    p6 = [GOOD] * 6
    assert ffn(None, *p6[1:], 4096, 12288, GOOD, 4, GOOD, GOOD, None) == -1
    assert ffn(*p6, 4096, 12288, GOOD, 4, GOOD, None, None) == -1
    for m in (0, 9, -1):
        assert ffn(*p6, 4096, 12288, GOOD, m, GOOD, GOOD, None) == -2
        assert gate_up(GOOD, GOOD, GOOD, GOOD, 4096, 12288, GOOD, m, GOOD, None) == -2
    for dm, dff in ((0, 12288), (4096 + 8, 12288), (100, 12288), (4096, 0)):
        assert ffn(*p6, dm, dff, GOOD, 4, GOOD, GOOD, None) == -2
    assert ffn(*p6, 4096, 12288, GOOD + 8, 4, GOOD, GOOD, None) == -3   # x
    assert ffn(*p6, 4096, 12288, GOOD, 4, GOOD + 2, GOOD, None) == -3   # h
    assert ffn(*p6, 4096, 12288, GOOD, 4, GOOD, GOOD + 2, None) == -3   # y
    assert gate_up(GOOD, GOOD, GOOD, GOOD, 4096, 12288, GOOD, 4, None, None) == -1
    assert gate_up(GOOD, GOOD, GOOD + 4, GOOD, 4096, 12288, GOOD, 4, GOOD, None) == -3


def test_stream_read_validation():
    lib = binding.lib()
    assert lib.pbg_stream_read(None, 1024, GOOD, None) == -1
    assert lib.pbg_stream_read(GOOD, 1024, None, None) == -1
    for nbytes in (0, 8, 1000, -16, 2 ** 40 + 16):
        assert lib.pbg_stream_read(GOOD, nbytes, GOOD, None) == -2
    assert lib.pbg_stream_read(GOOD + 8, 1024, GOOD, None) == -3
    assert lib.pbg_stream_read(GOOD, 1024, GOOD + 2, None) == -3


@no_gpu_only
def test_splitk_validation():
    lib = binding.lib()
    need = lib.pbg_splitk_workspace_bytes(4096, 12288)
    assert lib.ternary_gemm_splitk(GOOD, GOOD, 4096, 12288, GOOD, 8, GOOD, None, need, None) == -1
    assert lib.ternary_gemm_splitk(None, GOOD, 4096, 12288, GOOD, 8, GOOD, GOOD, need, None) == -1
    for n, k, m in ((0, 12288, 1), (4096, 0, 1), (4096, 12288, 0), (4096, 12288, 9)):
        assert lib.ternary_gemm_splitk(GOOD, GOOD, n, k, GOOD, m, GOOD, GOOD, need, None) == -2
    assert lib.ternary_gemm_splitk(GOOD + 4, GOOD, 4096, 12288, GOOD, 8, GOOD, GOOD, need, None) == -3
    assert lib.ternary_gemm_splitk(GOOD, GOOD, 4096, 12288, GOOD, 8, GOOD, GOOD + 128, need, None) == -3
    assert lib.ternary_gemm_splitk(GOOD, GOOD, 4096, 12288, GOOD, 8, GOOD, GOOD, need - 1, None) == -6


@no_gpu_only
def test_noalloc_argmax_validation():
    lib = binding.lib()
    assert lib.int8_head_argmax_noalloc(None, GOOD, 4, 64, GOOD, 1, GOOD, None, None) == -1
    assert lib.int8_head_argmax_noalloc(GOOD, GOOD, 4, 64, GOOD, 1, None, None, None) == -1
    for n, k, m in ((0, 64, 1), (4, 0, 1), (4, 64, 0), (4, 64, 9)):
        assert lib.int8_head_argmax_noalloc(GOOD, GOOD, n, k, GOOD, m, GOOD, None, None) == -2
    assert lib.int8_head_argmax_noalloc(GOOD + 8, GOOD, 4, 64, GOOD, 1, GOOD, None, None) == -3
    assert lib.int8_head_argmax_noalloc(GOOD, GOOD, 4, 64, GOOD, 1, GOOD + 2, None, None) == -3


@no_gpu_only
def test_ternary3_validation():
    lib = binding.lib()
    assert lib.pbg_words_per_row3(1) == 12 and lib.pbg_words_per_row3(4096) == 384
    assert lib.pbg_words_per_row3(129) == 24 and lib.pbg_words_per_row3(0) == 0
    assert lib.pack_ternary3(None, 4, 64, GOOD, GOOD, GOOD, None, None) == -1
    assert lib.pack_ternary3(GOOD, 0, 64, GOOD, GOOD, GOOD, None, None) == -2
    assert lib.pack_ternary3(GOOD, 4, 64, GOOD + 4, GOOD, GOOD, None, None) == -3
    assert lib.ternary3_gemv(GOOD, None, 4, 64, GOOD, GOOD, None) == -1
    assert lib.ternary3_gemv(GOOD, GOOD, 4, 2 ** 24 + 1, GOOD, GOOD, None) == -2
    assert lib.ternary3_gemv(GOOD + 8, GOOD, 4, 64, GOOD, GOOD, None) == -3
    for m in (0, 9):
        assert lib.ternary3_gemm_small(GOOD, GOOD, 4, 64, GOOD, m, GOOD, None) == -2
    assert lib.ternary3_gemm_small(GOOD, GOOD, 4, 64, GOOD + 1, 2, GOOD, None) == -3
