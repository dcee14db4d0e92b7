"""ctypes binding of libpackedbitgemv.so.

Argument marshalling only: every function checks tensor placement, dtype and
shape, passes raw device pointers and the current HIP stream to the C entry
point of the same name, and raises PbgError on a nonzero return code. All
computation happens in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

from .build import LIB_PATH

PBG_ERR_CODE = -4
ARGMAX_KEYS_PER_ROW = 4096  # PBG_ARGMAX_KEYS_PER_ROW
MAX_M = 8  # PBG_MAX_M
STREAM_READ_SINK_WORDS = 8192  # PBG_STREAM_READ_SINK_WORDS

_c_int = ctypes.c_int
_c_i64 = ctypes.c_int64
_vp = ctypes.c_void_p

# (restype, argtypes) of every entry point declared in include/packed_bit_gemv.h.
_SIGNATURES = {
    "pbg_abi_version": (_c_int, []),
    "pbg_strerror": (ctypes.c_char_p, [_c_int]),
    "pbg_words_per_row": (_c_i64, [_c_i64]),
    "pack_ternary": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp]),
    "ternary_gemv": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp]),
    "ternary_gemm_small": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp]),
    "pbg_words_per_row3": (_c_i64, [_c_i64]),
    "pack_ternary3": (_c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp]),
    "ternary3_gemv": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp]),
    "ternary3_gemm_small": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp]),
    "pbg_splitk_workspace_bytes": (_c_i64, [_c_i64, _c_i64]),
    "ternary_gemm_splitk": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp, _c_i64, _vp]),
    "int8_head_gemv": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp]),
    "int8_head_argmax": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp, _vp, _vp]),
    "int8_head_argmax_noalloc": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp, _vp]),
    "int8_embedding_gather": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp]),
    "ternary_swiglu_gate_up": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp]),
    "ternary_ffn_swiglu": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
    "ternary_swiglu_gate_up_small": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp]),
    "ternary_ffn_swiglu_small": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp,
                                          _vp]),
    "ternary3_ffn_swiglu_small": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp,
                                           _vp]),
    "ternary3_swiglu_gate_up": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp]),
    "ternary3_ffn_swiglu": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
    "ternary3_swiglu_gate_up_small": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, _vp]),
    "pbg_stream_read": (_c_int, [_vp, _c_i64, _vp, _vp]),
}


class PbgError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({code})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m packed_bit_gemv_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions declared in include/packed_bit_gemv.h."""
    path = os.path.join(os.path.dirname(os.path.dirname(LIB_PATH)), "include", "packed_bit_gemv.h")
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise PbgError(fn, rc, lib().pbg_strerror(rc).decode())


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def words_per_row(k: int) -> int:
    return int(lib().pbg_words_per_row(int(k)))


def pack_ternary(codes: torch.Tensor, packed: torch.Tensor | None = None, row_sum: torch.Tensor | None = None,
                 stats: torch.Tensor | None = None, check: bool = True):
    """Pack int8 codes [n, k] on the GPU. Returns (packed, row_sum, stats).

    stats holds n_minus, n_zero, n_plus, n_invalid. With check=True the call
    waits for the stream and raises PbgError if any code is outside {-1,0,1}.
    """
    _dev(codes, "codes", torch.int8)
    if codes.dim() != 2:
        raise ValueError("codes must be [n, k]")
    n, k = codes.shape
    dev = codes.device
    if packed is None:
        packed = torch.empty((n, words_per_row(k)), dtype=torch.int32, device=dev)
    if row_sum is None:
        row_sum = torch.empty((n,), dtype=torch.int32, device=dev)
    if stats is None:
        stats = torch.empty((4,), dtype=torch.int64, device=dev)
    _dev(packed, "packed", torch.int32)
    _dev(row_sum, "row_sum", torch.int32)
    _dev(stats, "stats", torch.int64)
    if tuple(packed.shape) != (n, words_per_row(k)) or tuple(row_sum.shape) != (n,) or stats.numel() != 4:
        raise ValueError("output shapes do not match codes")
    host = (ctypes.c_int64 * 4)() if check else None
    rc = lib().pack_ternary(codes.data_ptr(), n, k, packed.data_ptr(), row_sum.data_ptr(), stats.data_ptr(),
                            ctypes.addressof(host) if host is not None else None, _stream(codes))
    _check("pack_ternary", rc)
    return packed, row_sum, stats


def _ternary_args(packed, scale, k, x):
    _dev(packed, "packed", torch.int32)
    _dev(scale, "scale", torch.float32)
    _dev(x, "x", torch.float16)
    n = packed.shape[0]
    if packed.dim() != 2 or packed.shape[1] != words_per_row(k):
        raise ValueError(f"packed must be [n, {words_per_row(k)}] for k={k}")
    if tuple(scale.shape) != (n,):
        raise ValueError("scale must be [n]")
    return n


def ternary_gemv(packed: torch.Tensor, scale: torch.Tensor, k: int, x: torch.Tensor,
                 y: torch.Tensor | None = None) -> torch.Tensor:
    """y[r] = scale[r] * sum_j c[r, j] * x[j]; x is fp16 [k], y fp32 [n]."""
    n = _ternary_args(packed, scale, k, x)
    if tuple(x.shape) != (k,):
        raise ValueError(f"x must be [{k}]")
    if y is None:
        y = torch.empty((n,), dtype=torch.float32, device=packed.device)
    _dev(y, "y", torch.float32)
    if tuple(y.shape) != (n,):
        raise ValueError("y must be [n]")
    rc = lib().ternary_gemv(packed.data_ptr(), scale.data_ptr(), n, k, x.data_ptr(), y.data_ptr(), _stream(packed))
    _check("ternary_gemv", rc)
    return y


def ternary_gemm_small(packed: torch.Tensor, scale: torch.Tensor, k: int, x: torch.Tensor,
                       y: torch.Tensor | None = None) -> torch.Tensor:
    """Y[i, r] = scale[r] * sum_j c[r, j] * X[i, j]; X fp16 [m, k], m <= 8; Y fp32 [m, n]."""
    n = _ternary_args(packed, scale, k, x)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=packed.device)
    _dev(y, "y", torch.float32)
    if tuple(y.shape) != (m, n):
        raise ValueError("y must be [m, n]")
    rc = lib().ternary_gemm_small(packed.data_ptr(), scale.data_ptr(), n, k, x.data_ptr(), m, y.data_ptr(),
                                  _stream(packed))
    _check("ternary_gemm_small", rc)
    return y


def words_per_row3(k: int) -> int:
    return int(lib().pbg_words_per_row3(int(k)))


def pack_ternary3(codes: torch.Tensor, packed: torch.Tensor | None = None, row_sum: torch.Tensor | None = None,
                  stats: torch.Tensor | None = None, check: bool = True):
    """Pack five-level int8 codes [n, k] (-2..+2) on the GPU. Returns (packed, row_sum, stats).

    stats holds the counts of -2, -1, 0, +1, +2 and of invalid codes. With check=True the call
    waits for the stream and raises PbgError if any code is outside -2..+2.
    """
    _dev(codes, "codes", torch.int8)
    if codes.dim() != 2:
        raise ValueError("codes must be [n, k]")
    n, k = codes.shape
    dev = codes.device
    if packed is None:
        packed = torch.empty((n, words_per_row3(k)), dtype=torch.int32, device=dev)
    if row_sum is None:
        row_sum = torch.empty((n,), dtype=torch.int32, device=dev)
    if stats is None:
        stats = torch.empty((6,), dtype=torch.int64, device=dev)
    _dev(packed, "packed", torch.int32)
    _dev(row_sum, "row_sum", torch.int32)
    _dev(stats, "stats", torch.int64)
    if tuple(packed.shape) != (n, words_per_row3(k)) or tuple(row_sum.shape) != (n,) or stats.numel() != 6:
        raise ValueError("output shapes do not match codes")
    host = (ctypes.c_int64 * 6)() if check else None
    rc = lib().pack_ternary3(codes.data_ptr(), n, k, packed.data_ptr(), row_sum.data_ptr(), stats.data_ptr(),
                             ctypes.addressof(host) if host is not None else None, _stream(codes))
    _check("pack_ternary3", rc)
    return packed, row_sum, stats


def _ternary3_args(packed, scale, k, x):
    _dev(packed, "packed", torch.int32)
    _dev(scale, "scale", torch.float32)
    _dev(x, "x", torch.float16)
    n = packed.shape[0]
    if packed.dim() != 2 or packed.shape[1] != words_per_row3(k):
        raise ValueError(f"packed must be [n, {words_per_row3(k)}] for k={k}")
    if tuple(scale.shape) != (n,):
        raise ValueError("scale must be [n]")
    return n


def ternary3_gemv(packed: torch.Tensor, scale: torch.Tensor, k: int, x: torch.Tensor,
                  y: torch.Tensor | None = None) -> torch.Tensor:
    """Five-level y[r] = scale[r] * sum_j c[r, j] * x[j]; x fp16 [k], y fp32 [n]."""
    n = _ternary3_args(packed, scale, k, x)
    if tuple(x.shape) != (k,):
        raise ValueError(f"x must be [{k}]")
    if y is None:
        y = torch.empty((n,), dtype=torch.float32, device=packed.device)
    _dev(y, "y", torch.float32)
    if tuple(y.shape) != (n,):
        raise ValueError("y must be [n]")
    rc = lib().ternary3_gemv(packed.data_ptr(), scale.data_ptr(), n, k, x.data_ptr(), y.data_ptr(), _stream(packed))
    _check("ternary3_gemv", rc)
    return y


def ternary3_gemm_small(packed: torch.Tensor, scale: torch.Tensor, k: int, x: torch.Tensor,
                        y: torch.Tensor | None = None) -> torch.Tensor:
    """Five-level Y[i, r] = scale[r] * sum_j c[r, j] * X[i, j]; X fp16 [m, k], m <= 8; Y fp32 [m, n]."""
    n = _ternary3_args(packed, scale, k, x)
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=packed.device)
    _dev(y, "y", torch.float32)
    if tuple(y.shape) != (m, n):
        raise ValueError("y must be [m, n]")
    rc = lib().ternary3_gemm_small(packed.data_ptr(), scale.data_ptr(), n, k, x.data_ptr(), m, y.data_ptr(),
                                   _stream(packed))
    _check("ternary3_gemm_small", rc)
    return y


def splitk_workspace(n: int, k: int, device) -> torch.Tensor:
    """A zeroed workspace for ternary_gemm_splitk on [n, k] matrices (any m)."""
    nbytes = int(lib().pbg_splitk_workspace_bytes(int(n), int(k)))
    return torch.zeros(((nbytes + 7) // 8,), dtype=torch.int64, device=device)


def ternary_gemm_splitk(packed: torch.Tensor, scale: torch.Tensor, k: int, x: torch.Tensor, workspace: torch.Tensor,
                        y: torch.Tensor | None = None) -> torch.Tensor:
    """ternary_gemv (x [k] -> y [n]) or ternary_gemm_small (x [m, k] -> y [m, n]) with K split
    across workgroups; workspace from splitk_workspace(n, k), reused across calls."""
    n = _ternary_args(packed, scale, k, x)
    if x.dim() == 1 and x.shape[0] == k:
        m, y_shape = 1, (n,)
    elif x.dim() == 2 and x.shape[1] == k:
        m, y_shape = x.shape[0], (x.shape[0], n)
    else:
        raise ValueError(f"x must be [{k}] or [m, {k}]")
    if y is None:
        y = torch.empty(y_shape, dtype=torch.float32, device=packed.device)
    _dev(y, "y", torch.float32)
    if tuple(y.shape) != y_shape:
        raise ValueError(f"y must be {list(y_shape)}")
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous CUDA (HIP) tensor")
    rc = lib().ternary_gemm_splitk(packed.data_ptr(), scale.data_ptr(), n, k, x.data_ptr(), m, y.data_ptr(),
                                   workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream(packed))
    _check("ternary_gemm_splitk", rc)
    return y


def int8_head_gemv(w: torch.Tensor, scale: torch.Tensor, x: torch.Tensor,
                   y: torch.Tensor | None = None) -> torch.Tensor:
    """Y[i, v] = scale[v] * sum_j w[v, j] * X[i, j]; w int8 [n, k], X fp16 [m, k]; Y fp32 [m, n]."""
    _dev(w, "w", torch.int8)
    _dev(scale, "scale", torch.float32)
    _dev(x, "x", torch.float16)
    if w.dim() != 2:
        raise ValueError("w must be [n, k]")
    n, k = w.shape
    if tuple(scale.shape) != (n,):
        raise ValueError("scale must be [n]")
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x must be [m, {k}]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, n), dtype=torch.float32, device=w.device)
    _dev(y, "y", torch.float32)
    if tuple(y.shape) != (m, n):
        raise ValueError("y must be [m, n]")
    rc = lib().int8_head_gemv(w.data_ptr(), scale.data_ptr(), n, k, x.data_ptr(), m, y.data_ptr(), _stream(w))
    _check("int8_head_gemv", rc)
    return y


def int8_head_argmax(w: torch.Tensor, scale: torch.Tensor, x: torch.Tensor, keys: torch.Tensor | None = None,
                     token: torch.Tensor | None = None, logit: torch.Tensor | None = None):
    """Greedy token per activation row: (token int32 [m], logit fp32 [m]).

    keys is an int64 workspace of at least m * ARGMAX_KEYS_PER_ROW entries, zero before its first
    use and left zero by every call (a zeroed one is allocated if not given).
    """
    _dev(w, "w", torch.int8)
    _dev(scale, "scale", torch.float32)
    _dev(x, "x", torch.float16)
    if w.dim() != 2 or x.dim() != 2 or x.shape[1] != w.shape[1] or tuple(scale.shape) != (w.shape[0],):
        raise ValueError("w [n, k], scale [n], x [m, k]")
    n, k = w.shape
    m = x.shape[0]
    dev = w.device
    if keys is None:
        keys = torch.zeros((m * ARGMAX_KEYS_PER_ROW,), dtype=torch.int64, device=dev)
    if token is None:
        token = torch.empty((m,), dtype=torch.int32, device=dev)
    if logit is None:
        logit = torch.empty((m,), dtype=torch.float32, device=dev)
    _dev(keys, "keys", torch.int64)
    _dev(token, "token", torch.int32)
    _dev(logit, "logit", torch.float32)
    if keys.numel() < m * ARGMAX_KEYS_PER_ROW or token.numel() != m or logit.numel() != m:
        raise ValueError("keys holds m * ARGMAX_KEYS_PER_ROW entries, token and logit m")
    rc = lib().int8_head_argmax(w.data_ptr(), scale.data_ptr(), n, k, x.data_ptr(), m, keys.data_ptr(),
                                token.data_ptr(), logit.data_ptr(), _stream(w))
    _check("int8_head_argmax", rc)
    return token, logit


def int8_head_argmax_noalloc(w: torch.Tensor, scale: torch.Tensor, x: torch.Tensor,
                             token: torch.Tensor | None = None, logit: torch.Tensor | None = None):
    """int8_head_argmax with the library's own workspace: (token int32 [m], logit fp32 [m]).

    The C call allocates nothing (pass token and logit to keep this wrapper from allocating
    them). Calls that overlap in time on one GPU race.
    """
    _dev(w, "w", torch.int8)
    _dev(scale, "scale", torch.float32)
    _dev(x, "x", torch.float16)
    if w.dim() != 2 or x.dim() != 2 or x.shape[1] != w.shape[1] or tuple(scale.shape) != (w.shape[0],):
        raise ValueError("w [n, k], scale [n], x [m, k]")
    n, k = w.shape
    m = x.shape[0]
    if token is None:
        token = torch.empty((m,), dtype=torch.int32, device=w.device)
    if logit is None:
        logit = torch.empty((m,), dtype=torch.float32, device=w.device)
    _dev(token, "token", torch.int32)
    _dev(logit, "logit", torch.float32)
    if token.numel() != m or logit.numel() != m:
        raise ValueError("token and logit hold m entries")
    rc = lib().int8_head_argmax_noalloc(w.data_ptr(), scale.data_ptr(), n, k, x.data_ptr(), m, token.data_ptr(),
                                        logit.data_ptr(), _stream(w))
    _check("int8_head_argmax_noalloc", rc)
    return token, logit


def int8_embedding_gather(table: torch.Tensor, scale: torch.Tensor, tokens: torch.Tensor,
                          out: torch.Tensor | None = None) -> torch.Tensor:
    """Rows scale[t] * table[t] (fp32 [m, k]) for int32 token ids; ids outside [0, n) give NaN rows."""
    _dev(table, "table", torch.int8)
    _dev(scale, "scale", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    if table.dim() != 2 or tokens.dim() != 1 or tuple(scale.shape) != (table.shape[0],):
        raise ValueError("table [n, k], scale [n], tokens [m]")
    n, k = table.shape
    m = tokens.shape[0]
    if out is None:
        out = torch.empty((m, k), dtype=torch.float32, device=table.device)
    _dev(out, "out", torch.float32)
    if tuple(out.shape) != (m, k):
        raise ValueError("out must be [m, k]")
    rc = lib().int8_embedding_gather(table.data_ptr(), scale.data_ptr(), n, k, tokens.data_ptr(), m,
                                     out.data_ptr(), _stream(table))
    _check("int8_embedding_gather", rc)
    return out


def _ffn_rows(x: torch.Tensor, d_model: int) -> int:
    """0 for x [d_model] (one row), m for x [m, d_model] with 1 <= m <= 8."""
    if x.dim() == 1 and tuple(x.shape) == (d_model,):
        return 0
    if x.dim() == 2 and x.shape[1] == d_model and 1 <= x.shape[0] <= MAX_M:
        return x.shape[0]
    raise ValueError(f"x must be [{d_model}] or [m, {d_model}] with 1 <= m <= {MAX_M}")


def _swiglu_gate_up(prefix: str, wpr, gate, gate_scale, up, up_scale, d_model, x, h):
    for t, name in ((gate, "gate"), (up, "up")):
        _dev(t, name, torch.int32)
    for t, name in ((gate_scale, "gate_scale"), (up_scale, "up_scale")):
        _dev(t, name, torch.float32)
    _dev(x, "x", torch.float16)
    d_ff = gate.shape[0]
    if gate.dim() != 2 or tuple(up.shape) != tuple(gate.shape) or gate.shape[1] != wpr(d_model):
        raise ValueError(f"gate and up must be [d_ff, {wpr(d_model)}]")
    if tuple(gate_scale.shape) != (d_ff,) or tuple(up_scale.shape) != (d_ff,):
        raise ValueError("scales must be [d_ff]")
    m = _ffn_rows(x, d_model)
    h_shape = (d_ff,) if m == 0 else (m, d_ff)
    if h is None:
        h = torch.empty(h_shape, dtype=torch.float16, device=gate.device)
    _dev(h, "h", torch.float16)
    if tuple(h.shape) != h_shape:
        raise ValueError(f"h must be {list(h_shape)}")
    if m == 0:
        name = f"{prefix}_swiglu_gate_up"
        rc = getattr(lib(), name)(gate.data_ptr(), gate_scale.data_ptr(), up.data_ptr(), up_scale.data_ptr(),
                                  d_model, d_ff, x.data_ptr(), h.data_ptr(), _stream(gate))
    else:
        name = f"{prefix}_swiglu_gate_up_small"
        rc = getattr(lib(), name)(gate.data_ptr(), gate_scale.data_ptr(), up.data_ptr(), up_scale.data_ptr(),
                                  d_model, d_ff, x.data_ptr(), m, h.data_ptr(), _stream(gate))
    _check(name, rc)
    return h


def ternary_swiglu_gate_up(gate: torch.Tensor, gate_scale: torch.Tensor, up: torch.Tensor, up_scale: torch.Tensor,
                           d_model: int, x: torch.Tensor, h: torch.Tensor | None = None) -> torch.Tensor:
    """h = fp16(silu(gate x) * up x) in one launch; gate, up packed [d_ff, words_per_row(d_model)].

    x fp16 [d_model] gives h [d_ff]; x [m, d_model] (m <= 8, one weight read for all rows) gives h [m, d_ff].
    """
    return _swiglu_gate_up("ternary", words_per_row, gate, gate_scale, up, up_scale, d_model, x, h)


def ternary3_swiglu_gate_up(gate: torch.Tensor, gate_scale: torch.Tensor, up: torch.Tensor, up_scale: torch.Tensor,
                            d_model: int, x: torch.Tensor, h: torch.Tensor | None = None) -> torch.Tensor:
    """ternary_swiglu_gate_up with gate and up in the 3-bit layout, packed [d_ff, words_per_row3(d_model)]."""
    return _swiglu_gate_up("ternary3", words_per_row3, gate, gate_scale, up, up_scale, d_model, x, h)


def _ffn_swiglu(prefix: str, wpr, gate, gate_scale, up, up_scale, down, down_scale, x, h, y):
    for t, name in ((gate, "gate"), (up, "up"), (down, "down")):
        _dev(t, name, torch.int32)
    for t, name in ((gate_scale, "gate_scale"), (up_scale, "up_scale"), (down_scale, "down_scale")):
        _dev(t, name, torch.float32)
    _dev(x, "x", torch.float16)
    d_ff, d_model = gate.shape[0], down.shape[0]
    if gate.dim() != 2 or tuple(up.shape) != tuple(gate.shape) or gate.shape[1] != wpr(d_model):
        raise ValueError(f"gate and up must be [d_ff, {wpr(d_model)}]")
    if down.dim() != 2 or down.shape[1] != wpr(d_ff):
        raise ValueError(f"down must be [d_model, {wpr(d_ff)}]")
    if tuple(gate_scale.shape) != (d_ff,) or tuple(up_scale.shape) != (d_ff,) or tuple(down_scale.shape) != (d_model,):
        raise ValueError("scales must be [d_ff], [d_ff], [d_model]")
    m = _ffn_rows(x, d_model)
    h_shape = (d_ff,) if m == 0 else (m, d_ff)
    y_shape = (d_model,) if m == 0 else (m, d_model)
    dev = gate.device
    if h is None:
        h = torch.empty(h_shape, dtype=torch.float16, device=dev)
    if y is None:
        y = torch.empty(y_shape, dtype=torch.float32, device=dev)
    _dev(h, "h", torch.float16)
    _dev(y, "y", torch.float32)
    if tuple(h.shape) != h_shape or tuple(y.shape) != y_shape:
        raise ValueError(f"h must be {list(h_shape)} and y {list(y_shape)}")
    if m == 0:
        name = f"{prefix}_ffn_swiglu"
        rc = getattr(lib(), name)(gate.data_ptr(), gate_scale.data_ptr(), up.data_ptr(), up_scale.data_ptr(),
                                  down.data_ptr(), down_scale.data_ptr(), d_model, d_ff, x.data_ptr(), h.data_ptr(),
                                  y.data_ptr(), _stream(gate))
    else:
        name = f"{prefix}_ffn_swiglu_small"
        rc = getattr(lib(), name)(gate.data_ptr(), gate_scale.data_ptr(), up.data_ptr(), up_scale.data_ptr(),
                                  down.data_ptr(), down_scale.data_ptr(), d_model, d_ff, x.data_ptr(), m,
                                  h.data_ptr(), y.data_ptr(), _stream(gate))
    _check(name, rc)
    return h, y


def ternary_ffn_swiglu(gate: torch.Tensor, gate_scale: torch.Tensor, up: torch.Tensor, up_scale: torch.Tensor,
                       down: torch.Tensor, down_scale: torch.Tensor, x: torch.Tensor,
                       h: torch.Tensor | None = None, y: torch.Tensor | None = None):
    """Gated feed-forward block: h = fp16(silu(gate x) * up x), y = down h.

    gate, up: packed [d_ff, words_per_row(d_model)]; down: packed [d_model, words_per_row(d_ff)];
    x fp16 [d_model] -> (h fp16 [d_ff], y fp32 [d_model]), or x [m, d_model] with m <= 8 ->
    (h [m, d_ff], y [m, d_model]), each weight read once for all m rows.
    """
    return _ffn_swiglu("ternary", words_per_row, gate, gate_scale, up, up_scale, down, down_scale, x, h, y)


def ternary3_ffn_swiglu(gate: torch.Tensor, gate_scale: torch.Tensor, up: torch.Tensor, up_scale: torch.Tensor,
                        down: torch.Tensor, down_scale: torch.Tensor, x: torch.Tensor,
                        h: torch.Tensor | None = None, y: torch.Tensor | None = None):
    """ternary_ffn_swiglu with the three linears in the 3-bit layout (rows of words_per_row3 words)."""
    return _ffn_swiglu("ternary3", words_per_row3, gate, gate_scale, up, up_scale, down, down_scale, x, h, y)


def stream_read(src: torch.Tensor, sink: torch.Tensor | None = None) -> torch.Tensor:
    """Read every byte of src once with the GEMVs' loads and fold them by XOR into sink.

    A measurement helper: its time is the streaming-read ceiling for one launch
    moving src.nbytes. sink is int32 [STREAM_READ_SINK_WORDS] (a new zeroed one
    if None); afterwards the XOR of its words, XOR-ed with its XOR before the
    call, is the XOR of all 32-bit words of src.
    """
    if not isinstance(src, torch.Tensor) or not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous CUDA (HIP) tensor")
    if sink is None:
        sink = torch.zeros((STREAM_READ_SINK_WORDS,), dtype=torch.int32, device=src.device)
    _dev(sink, "sink", torch.int32)
    if tuple(sink.shape) != (STREAM_READ_SINK_WORDS,):
        raise ValueError(f"sink must be [{STREAM_READ_SINK_WORDS}]")
    nbytes = src.numel() * src.element_size()
    rc = lib().pbg_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), _stream(src))
    _check("pbg_stream_read", rc)
    return sink
