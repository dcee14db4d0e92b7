"""MI355X (gfx950) packed ternary GEMV: HIP kernels behind a C ABI.

The compute path is libpackedbitgemv.so (built from csrc/ by build.py); this
package only binds it. Packed words are carried in torch.int32 tensors (same
bits as the uint32 words of the C ABI).
"""
from .binding import (  # noqa: F401
    PbgError,
    int8_embedding_gather,
    int8_head_argmax,
    int8_head_argmax_noalloc,
    int8_head_gemv,
    lib,
    pack_ternary,
    pack_ternary3,
    splitk_workspace,
    stream_read,
    ternary_ffn_swiglu,
    ternary_swiglu_gate_up,
    ternary_gemm_small,
    ternary_gemm_splitk,
    ternary_gemv,
    ternary3_ffn_swiglu,
    ternary3_gemm_small,
    ternary3_gemv,
    ternary3_swiglu_gate_up,
    words_per_row,
    words_per_row3,
)

__all__ = [
    "PbgError",
    "int8_embedding_gather",
    "int8_head_argmax",
    "int8_head_argmax_noalloc",
    "int8_head_gemv",
    "lib",
    "pack_ternary",
    "pack_ternary3",
    "splitk_workspace",
    "stream_read",
    "ternary_ffn_swiglu",
    "ternary_swiglu_gate_up",
    "ternary_gemm_small",
    "ternary_gemm_splitk",
    "ternary_gemv",
    "ternary3_ffn_swiglu",
    "ternary3_gemm_small",
    "ternary3_gemv",
    "ternary3_swiglu_gate_up",
    "words_per_row",
    "words_per_row3",
]
