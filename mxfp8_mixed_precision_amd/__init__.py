"""Python binding of libtemx.so, the MXFP8 Linear hot path for MI355X (gfx950).

Every function named ``te_*`` marshals torch tensors (device memory) and the
current HIP stream into the C entry point of the same name declared in
``include/temx.h``; all computation happens in the library's HIP kernels.
The helpers without the prefix only allocate outputs with torch and call the
``te_*`` functions.  There is no fallback: importing this package fails if
the library has not been built (``python mxfp8_mixed_precision_amd/build.py``).
"""

from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtemx.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python mxfp8_mixed_precision_amd/build.py`")
_lib = ctypes.CDLL(_LIB_PATH)

# enum values of include/temx.h
TE_OK, TE_ERR_NULL, TE_ERR_SHAPE, TE_ERR_ALIGN, TE_ERR_DTYPE, TE_ERR_WORKSPACE, TE_ERR_HIP, TE_ERR_VALUE, TE_ERR_ARCH = range(9)
TE_BF16, TE_FP32, TE_E4M3, TE_E5M2, TE_E8M0, TE_FP16 = range(6)
TE_EPI_NONE, TE_EPI_BIAS, TE_EPI_BIAS_GELU_AUX, TE_EPI_DGELU, TE_EPI_ACCUMULATE = range(5)
TE_ROWWISE, TE_COLWISE, TE_BOTH = 1, 2, 3
TE_AMAX_MAX, TE_AMAX_MOST_RECENT = 0, 1
AMAX_ALGOS = {"max": TE_AMAX_MAX, "most_recent": TE_AMAX_MOST_RECENT}
TE_BLOCK_SCALES_E8M0, TE_BLOCK_SCALES_FP32 = 0, 1
BLOCK_SCALINGS = {"e8m0": TE_BLOCK_SCALES_E8M0, "fp32": TE_BLOCK_SCALES_FP32}

FORMATS = {"e4m3": TE_E4M3, "e5m2": TE_E5M2}
EPILOGUES = {"none": TE_EPI_NONE, "bias": TE_EPI_BIAS, "bias_gelu_aux": TE_EPI_BIAS_GELU_AUX,
             "dgelu": TE_EPI_DGELU, "accumulate": TE_EPI_ACCUMULATE}
DIRECTIONS = {"row": TE_ROWWISE, "col": TE_COLWISE, "both": TE_BOTH}

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "te_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "te_amax_workspace_size": (_sz, [_i64]),
    "te_amax_reduce": (ctypes.c_int, [_vp, _i64, _vp, _vp, _sz, _vp]),
    "te_fp8_cast_current_scaling": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "te_fp8_cast_current_scaling_noalloc": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp]),
    "te_fp8_cast_delayed_scaling": (ctypes.c_int, [_vp, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_int, _vp, _sz, _vp]),
    "te_fp8_gemm": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _i64, _i64, _i64,
                                   _vp, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _sz, _vp]),
    "te_mxfp8_quantize": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _vp, _vp]),
    "te_mxfp8_quantize_bgrad_workspace_size": (_sz, [_i64, _i64]),
    "te_mxfp8_quantize_bgrad": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, ctypes.c_int,
                                               _vp, _sz, _vp]),
    "te_mxfp8_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "te_mxfp8_gemm": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _i64, _i64, _i64,
                                     _vp, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _sz, _vp]),
    "te_mxfp8_gemm_mxout": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _i64, _i64, _i64,
                                           _vp, _vp, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _sz, _vp]),
    "te_mxfp8_grouped_gemm": (ctypes.c_int, [_i32, _vp, _i64, _vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int,
                                             _i64, _i64, _vp, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp, _sz, _vp]),
    "te_fp8_block_quantize": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp]),
    "te_fp8_block_scales_to_mx": (ctypes.c_int, [_vp, _i64, _i64, ctypes.c_int, _vp, _vp]),
    "te_fp8_block_gemm_workspace_size": (_sz, [_i64, _i64, _i64, ctypes.c_int]),
    "te_fp8_block_gemm": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, ctypes.c_int, _i64, _i64,
                                         _i64, _vp, ctypes.c_int, ctypes.c_int, _vp, _vp, ctypes.c_int, ctypes.c_float,
                                         _vp, _sz, _vp]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class TemxError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {te_status_str(status)}")
        self.status = status


def te_status_str(status: int) -> str:
    return _lib.te_status_str(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != TE_OK:
        raise TemxError(fn, status)


def _ptr(t):
    """Device address of a tensor argument.  Every pointer of the C ABI is a device pointer into a dense
    row-major buffer, so host tensors and non-contiguous views are refused here (the library cannot tell
    them apart from valid arguments)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor (row-major, no strides)")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _fmt(f) -> int:
    return FORMATS[f] if isinstance(f, str) else int(f)


# Argument checks of the wrappers.  The C ABI sees only addresses and sizes, so
# a tensor of the wrong shape or element type would be read or written past
# its end there; every wrapper checks its tensors against the sizes it passes
# before calling the library.
_BYTE_DTYPES = {torch.uint8, torch.int8} | {getattr(torch, n) for n in
                                           ("float8_e4m3fn", "float8_e5m2", "float8_e8m0fnu") if hasattr(torch, n)}
_BF16_DTYPES = {torch.bfloat16, torch.int16} | ({torch.uint16} if hasattr(torch, "uint16") else set())


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _check_tensor(t, name: str, shape, dtypes, kind: str, optional: bool = False) -> None:
    """t must have exactly `shape` and a dtype in `dtypes` (None is accepted only when optional)."""
    if t is None:
        _require(optional, f"{name} is required")
        return
    _require(t.dtype in dtypes, f"{name}: expected {kind}, got {t.dtype}")
    _require(tuple(t.shape) == tuple(int(v) for v in shape),
             f"{name}: expected shape {tuple(int(v) for v in shape)}, got {tuple(t.shape)}")


def _codes(t, name, shape, optional=False):
    _check_tensor(t, name, shape, _BYTE_DTYPES, "1-byte codes (uint8)", optional)


def _bf16(t, name, shape, optional=False):
    _check_tensor(t, name, shape, _BF16_DTYPES, "bf16 (or its int16 bits)", optional)


def _f32(t, name, shape, optional=False):
    _check_tensor(t, name, shape, {torch.float32}, "float32", optional)


def _scalar_f32(t, name):
    _require(t is not None and t.dtype == torch.float32 and t.numel() >= 1, f"{name}: expected a float32 scalar")


_OUT_DTYPES = {torch.bfloat16: TE_BF16, torch.float32: TE_FP32, torch.float16: TE_FP16}


def _gemm_out(d, name, M, N, epi, allow_fp16=False):
    """D of the bf16/fp32-output GEMMs: [M, N] bf16 or float32 (float16 too where allowed); "accumulate"
    needs float32."""
    kinds = (torch.bfloat16, torch.float32) + ((torch.float16,) if allow_fp16 else ())
    _require(d is not None and d.dtype in kinds,
             f"{name}: expected {' or '.join(str(k).replace('torch.', '') for k in kinds)}, "
             f"got {None if d is None else d.dtype}")
    _require(epi != TE_EPI_ACCUMULATE or d.dtype == torch.float32, f"{name}: the accumulate epilogue needs float32")
    _require(tuple(d.shape) == (M, N), f"{name}: expected shape {(M, N)}, got {tuple(d.shape)}")
    return _OUT_DTYPES[d.dtype]


def _epi_tensors(bias, bias_shape, aux, M, N):
    """bias (bf16, bias_shape) with the bias epilogues; aux (bf16 [M, N]) with GELU aux and dgelu."""
    _bf16(bias, "bias", bias_shape, optional=True)
    _bf16(aux, "aux", (M, N), optional=True)


def _epilogue(epilogue) -> int:
    return EPILOGUES[epilogue] if isinstance(epilogue, str) else int(epilogue)


def _ws_bytes(workspace) -> int:
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


# ---------------------------------------------------------------- entry points

def te_amax_workspace_size(n: int) -> int:
    return int(_lib.te_amax_workspace_size(int(n)))


def te_amax_reduce(x, amax_out, workspace, stream=None) -> None:
    _bf16(x, "x", tuple(x.shape))
    _scalar_f32(amax_out, "amax_out")
    _check("te_amax_reduce", _lib.te_amax_reduce(_ptr(x), x.numel(), _ptr(amax_out), _ptr(workspace),
                                                 workspace.numel() * workspace.element_size(), _stream(stream)))


def te_fp8_cast_current_scaling(x, fmt, q_out, amax_out, scale_out, scale_inv_out, workspace, stream=None) -> None:
    _bf16(x, "x", tuple(x.shape))
    _codes(q_out, "q_out", tuple(x.shape))
    for t, n in ((amax_out, "amax_out"), (scale_out, "scale_out"), (scale_inv_out, "scale_inv_out")):
        _scalar_f32(t, n)
    _check("te_fp8_cast_current_scaling", _lib.te_fp8_cast_current_scaling(
        _ptr(x), x.numel(), _fmt(fmt), _ptr(q_out), _ptr(amax_out), _ptr(scale_out), _ptr(scale_inv_out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)))


def te_fp8_cast_current_scaling_noalloc(x, fmt, q_out, amax_out, scale_out, scale_inv_out, stream=None) -> None:
    _bf16(x, "x", tuple(x.shape))
    _codes(q_out, "q_out", tuple(x.shape))
    for t, n in ((amax_out, "amax_out"), (scale_out, "scale_out"), (scale_inv_out, "scale_inv_out")):
        _scalar_f32(t, n)
    _check("te_fp8_cast_current_scaling_noalloc", _lib.te_fp8_cast_current_scaling_noalloc(
        _ptr(x), x.numel(), _fmt(fmt), _ptr(q_out), _ptr(amax_out), _ptr(scale_out), _ptr(scale_inv_out),
        _stream(stream)))


def te_fp8_cast_delayed_scaling(x, fmt, q_out, q_scale_inv_out, scale, amax_history, workspace, algo="max",
                                margin=0, stream=None) -> None:
    a = AMAX_ALGOS[algo] if isinstance(algo, str) else int(algo)
    _bf16(x, "x", tuple(x.shape))
    _codes(q_out, "q_out", tuple(x.shape))
    _scalar_f32(q_scale_inv_out, "q_scale_inv_out")
    _scalar_f32(scale, "scale")
    _require(amax_history is not None and amax_history.dtype == torch.float32 and amax_history.dim() == 1,
             "amax_history: expected a 1-D float32 tensor")
    _check("te_fp8_cast_delayed_scaling", _lib.te_fp8_cast_delayed_scaling(
        _ptr(x), x.numel(), _fmt(fmt), _ptr(q_out), _ptr(q_scale_inv_out), _ptr(scale), _ptr(amax_history),
        amax_history.numel(), a, int(margin), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def te_fp8_gemm(a, a_scale_inv, a_fmt, b, b_scale_inv, b_fmt, d, epilogue="none", bias=None, aux=None,
                workspace=None, stream=None) -> None:
    _require(a.dim() == 2 and b.dim() == 2, "a and b must be 2-D")
    M, K = a.shape
    N = b.shape[0]
    _codes(a, "a", (M, K))
    _codes(b, "b", (N, K))
    _scalar_f32(a_scale_inv, "a_scale_inv")
    _scalar_f32(b_scale_inv, "b_scale_inv")
    epi = _epilogue(epilogue)
    d_dtype = _gemm_out(d, "d", M, N, epi)
    _epi_tensors(bias, (N,), aux, M, N)
    ws_bytes = _ws_bytes(workspace)
    _check("te_fp8_gemm", _lib.te_fp8_gemm(
        _ptr(a), _ptr(a_scale_inv), _fmt(a_fmt), _ptr(b), _ptr(b_scale_inv), _fmt(b_fmt), M, N, K,
        _ptr(d), d_dtype, epi, _ptr(bias), _ptr(aux), _ptr(workspace), ws_bytes, _stream(stream)))


def te_mxfp8_quantize(x, fmt, direction, q_row=None, s_row=None, q_col=None, s_col=None, stream=None) -> None:
    d = DIRECTIONS[direction] if isinstance(direction, str) else int(direction)
    _require(x.dim() == 2, "x must be 2-D")
    rows, cols = x.shape
    _bf16(x, "x", (rows, cols))
    _codes(q_row, "q_row", (rows, cols), optional=True)
    _codes(s_row, "s_row", (rows, cols // 32), optional=True)
    _codes(q_col, "q_col", (cols, rows), optional=True)
    _codes(s_col, "s_col", (cols, rows // 32), optional=True)
    _check("te_mxfp8_quantize", _lib.te_mxfp8_quantize(
        _ptr(x), rows, cols, _fmt(fmt), d, _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col), _stream(stream)))


def te_mxfp8_quantize_bgrad_workspace_size(rows: int, cols: int) -> int:
    return int(_lib.te_mxfp8_quantize_bgrad_workspace_size(int(rows), int(cols)))


def te_mxfp8_quantize_bgrad(x, fmt, q_row, s_row, q_col, s_col, bgrad, workspace, stream=None) -> None:
    _require(x.dim() == 2, "x must be 2-D")
    rows, cols = x.shape
    _bf16(x, "x", (rows, cols))
    empty = rows == 0  # no codes to write: the outputs may be None
    _codes(q_row, "q_row", (rows, cols), optional=empty)
    _codes(s_row, "s_row", (rows, cols // 32), optional=empty)
    _codes(q_col, "q_col", (cols, rows), optional=empty)
    _codes(s_col, "s_col", (cols, rows // 32), optional=empty)
    _check_tensor(bgrad, "bgrad", (cols,), {torch.float32, torch.bfloat16}, "float32 or bfloat16")
    b_dtype = TE_FP32 if bgrad.dtype == torch.float32 else TE_BF16
    ws_bytes = _ws_bytes(workspace)
    _check("te_mxfp8_quantize_bgrad", _lib.te_mxfp8_quantize_bgrad(
        _ptr(x), rows, cols, _fmt(fmt), _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col), _ptr(bgrad), b_dtype,
        _ptr(workspace), ws_bytes, _stream(stream)))


def te_mxfp8_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(_lib.te_mxfp8_gemm_workspace_size(M, N, K))


def _mx_operands(a, a_scale, b, b_scale):
    """Shapes of two MXFP8 operands: a [M, K] + [M, K/32], b [N, K] + [N, K/32] -> (M, N, K)."""
    _require(a.dim() == 2 and b.dim() == 2, "a and b must be 2-D")
    M, K = a.shape
    N = b.shape[0]
    _codes(a, "a", (M, K))
    _codes(a_scale, "a_scale", (M, K // 32))
    _codes(b, "b", (N, K))
    _codes(b_scale, "b_scale", (N, K // 32))
    return M, N, K


def te_mxfp8_gemm(a, a_scale, a_fmt, b, b_scale, b_fmt, d, epilogue="none", bias=None, aux=None,
                  workspace=None, stream=None) -> None:
    M, N, K = _mx_operands(a, a_scale, b, b_scale)
    epi = _epilogue(epilogue)
    d_dtype = _gemm_out(d, "d", M, N, epi)
    _epi_tensors(bias, (N,), aux, M, N)
    ws_bytes = _ws_bytes(workspace)
    _check("te_mxfp8_gemm", _lib.te_mxfp8_gemm(
        _ptr(a), _ptr(a_scale), _fmt(a_fmt), _ptr(b), _ptr(b_scale), _fmt(b_fmt), M, N, K,
        _ptr(d), d_dtype, epi, _ptr(bias), _ptr(aux), _ptr(workspace), ws_bytes, _stream(stream)))


def te_mxfp8_gemm_mxout(a, a_scale, a_fmt, b, b_scale, b_fmt, d, d_scale, d_fmt, epilogue="none", bias=None,
                        aux=None, workspace=None, stream=None) -> None:
    M, N, K = _mx_operands(a, a_scale, b, b_scale)
    epi = _epilogue(epilogue)
    _codes(d, "d", (M, N))
    _codes(d_scale, "d_scale", (M, N // 32))
    _epi_tensors(bias, (N,), aux, M, N)
    ws_bytes = _ws_bytes(workspace)
    _check("te_mxfp8_gemm_mxout", _lib.te_mxfp8_gemm_mxout(
        _ptr(a), _ptr(a_scale), _fmt(a_fmt), _ptr(b), _ptr(b_scale), _fmt(b_fmt), M, N, K,
        _ptr(d), _ptr(d_scale), _fmt(d_fmt), epi, _ptr(bias), _ptr(aux), _ptr(workspace), ws_bytes, _stream(stream)))


def te_mxfp8_grouped_gemm(m_splits, a, a_scale, a_fmt, b, b_scale, b_fmt, n: int, d, epilogue="none",
                          bias=None, aux=None, workspace=None, stream=None) -> None:
    _require(m_splits is not None and m_splits.dtype == torch.int32 and m_splits.dim() == 1,
             "m_splits: expected a 1-D int32 tensor (one row count per group)")
    G = m_splits.numel()
    total_m, _, K = _mx_operands(a, a_scale, b, b_scale)
    _require(b.shape[0] == G * int(n), f"b: expected {G} x {int(n)} = {G * int(n)} rows, got {b.shape[0]}")
    epi = _epilogue(epilogue)
    d_dtype = _gemm_out(d, "d", total_m, int(n), epi)
    _epi_tensors(bias, (G, int(n)), aux, total_m, int(n))
    ws_bytes = _ws_bytes(workspace)
    _check("te_mxfp8_grouped_gemm", _lib.te_mxfp8_grouped_gemm(
        m_splits.numel(), _ptr(m_splits), total_m, _ptr(a), _ptr(a_scale), _fmt(a_fmt), _ptr(b), _ptr(b_scale),
        _fmt(b_fmt), n, K, _ptr(d), d_dtype, epi, _ptr(bias), _ptr(aux), _ptr(workspace), ws_bytes,
        _stream(stream)))


def _block_scaling(mode) -> int:
    return BLOCK_SCALINGS[mode] if isinstance(mode, str) else int(mode)


def _block_scale_shape(rows, cols, block_2d):
    return ((rows + 127) // 128 if block_2d else rows, cols // 128)


def te_fp8_block_quantize(x, fmt, block_2d, q, scale_inv, stream=None) -> None:
    _require(x.dim() == 2, "x must be 2-D")
    rows, cols = x.shape
    _bf16(x, "x", (rows, cols))
    _codes(q, "q", (rows, cols))
    _f32(scale_inv, "scale_inv", _block_scale_shape(rows, cols, block_2d))
    _check("te_fp8_block_quantize", _lib.te_fp8_block_quantize(
        _ptr(x), rows, cols, _fmt(fmt), int(bool(block_2d)), _ptr(q), _ptr(scale_inv), _stream(stream)))


def te_fp8_block_scales_to_mx(scale_inv, rows: int, cols: int, block_2d: bool, mx_scale, stream=None) -> None:
    _f32(scale_inv, "scale_inv", _block_scale_shape(int(rows), int(cols), block_2d))
    _codes(mx_scale, "mx_scale", (int(rows), int(cols) // 32))
    _check("te_fp8_block_scales_to_mx", _lib.te_fp8_block_scales_to_mx(
        _ptr(scale_inv), int(rows), int(cols), int(bool(block_2d)), _ptr(mx_scale), _stream(stream)))


def te_fp8_block_gemm_workspace_size(M: int, N: int, K: int, mode="e8m0") -> int:
    return int(_lib.te_fp8_block_gemm_workspace_size(M, N, K, _block_scaling(mode)))


def te_fp8_block_gemm(a, a_scale_inv, a_fmt, b, b_scale_inv, b_fmt, b_block_2d, d, epilogue="none", bias=None,
                      aux=None, mode="e8m0", workspace=None, stream=None, beta=1.0) -> None:
    _require(a.dim() == 2 and b.dim() == 2, "a and b must be 2-D")
    M, K = a.shape
    N = b.shape[0]
    _codes(a, "a", (M, K))
    _codes(b, "b", (N, K))
    _f32(a_scale_inv, "a_scale_inv", _block_scale_shape(M, K, False))
    _f32(b_scale_inv, "b_scale_inv", _block_scale_shape(N, K, b_block_2d))
    epi = _epilogue(epilogue)
    d_dtype = _gemm_out(d, "d", M, N, epi, allow_fp16=True)
    _epi_tensors(bias, (N,), aux, M, N)
    ws_bytes = _ws_bytes(workspace)
    _check("te_fp8_block_gemm", _lib.te_fp8_block_gemm(
        _ptr(a), _ptr(a_scale_inv), _fmt(a_fmt), _ptr(b), _ptr(b_scale_inv), _fmt(b_fmt), int(bool(b_block_2d)),
        M, N, K, _ptr(d), d_dtype, epi, _ptr(bias), _ptr(aux), _block_scaling(mode), float(beta), _ptr(workspace),
        ws_bytes, _stream(stream)))


# ------------------------------------------------------- allocating helpers

def mxfp8_quantize(x, fmt="e4m3", direction="row", stream=None):
    """bf16 [rows, cols] (torch.bfloat16 or int16/uint16 bits) -> (q_row, s_row, q_col, s_col), None where
    a direction is not requested."""
    rows, cols = x.shape
    d = DIRECTIONS[direction]
    dev = x.device
    q_row = s_row = q_col = s_col = None
    if d & TE_ROWWISE:
        q_row = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
        s_row = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    if d & TE_COLWISE:
        q_col = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
        s_col = torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev)
    te_mxfp8_quantize(x, fmt, d, q_row, s_row, q_col, s_col, stream)
    return q_row, s_row, q_col, s_col


def mxfp8_quantize_bgrad(x, fmt="e5m2", bgrad_dtype=torch.float32, stream=None):
    """bf16 [rows, cols] output gradient -> (q_row, s_row, q_col, s_col, bgrad), one pass; bgrad [cols] is
    the column sum of x (fp32 accumulation), as float32 or bfloat16."""
    rows, cols = x.shape
    dev = x.device
    q_row = torch.empty((rows, cols), dtype=torch.uint8, device=dev)
    s_row = torch.empty((rows, cols // 32), dtype=torch.uint8, device=dev)
    q_col = torch.empty((cols, rows), dtype=torch.uint8, device=dev)
    s_col = torch.empty((cols, rows // 32), dtype=torch.uint8, device=dev)
    bgrad = torch.empty(cols, dtype=bgrad_dtype, device=dev)
    ws = torch.empty(max(te_mxfp8_quantize_bgrad_workspace_size(rows, cols), 16), dtype=torch.uint8, device=dev)
    te_mxfp8_quantize_bgrad(x, fmt, q_row, s_row, q_col, s_col, bgrad, ws, stream)
    return q_row, s_row, q_col, s_col, bgrad


class DelayedScaling:
    """Device state of one tensor under delayed scaling: scale (starts at 1) and the amax history
    (zeros, newest first).  step(x) casts x with the current scale and updates the state."""

    def __init__(self, fmt="e4m3", history_len=16, algo="max", margin=0, device="cuda"):
        self.fmt, self.algo, self.margin = fmt, algo, margin
        self.scale = torch.ones(1, dtype=torch.float32, device=device)
        self.history = torch.zeros(history_len, dtype=torch.float32, device=device)

    def step(self, x, stream=None):
        """-> (q, q_scale_inv): x cast with the scale as it stood, and that scale's inverse."""
        dev = x.device
        q = torch.empty(x.shape, dtype=torch.uint8, device=dev)
        q_inv = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(max(te_amax_workspace_size(x.numel()), 4), dtype=torch.uint8, device=dev)
        te_fp8_cast_delayed_scaling(x, self.fmt, q, q_inv, self.scale, self.history, ws, self.algo, self.margin,
                                    stream)
        return q, q_inv


def fp8_gemm(a, a_scale_inv, a_fmt, b, b_scale_inv, b_fmt, epilogue="none", bias=None, out_dtype=torch.bfloat16,
             stream=None):
    """Per-tensor FP8 GEMM -> (D, aux)."""
    M, N = a.shape[0], b.shape[0]
    d = torch.empty((M, N), dtype=out_dtype, device=a.device)
    aux = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if epilogue == "bias_gelu_aux" else None
    te_fp8_gemm(a, a_scale_inv, a_fmt, b, b_scale_inv, b_fmt, d, epilogue, bias, aux, None, stream)
    return d, aux


def amax(x, stream=None):
    ws = torch.empty(max(te_amax_workspace_size(x.numel()), 4), dtype=torch.uint8, device=x.device)
    out = torch.empty(1, dtype=torch.float32, device=x.device)
    te_amax_reduce(x, out, ws, stream)
    return out


def fp8_cast_current_scaling(x, fmt="e4m3", stream=None):
    """-> (q, amax, scale, scale_inv) with q shaped like x."""
    dev = x.device
    ws = torch.empty(max(te_amax_workspace_size(x.numel()), 4), dtype=torch.uint8, device=dev)
    q = torch.empty(x.shape, dtype=torch.uint8, device=dev)
    a, s, si = (torch.empty(1, dtype=torch.float32, device=dev) for _ in range(3))
    te_fp8_cast_current_scaling(x, fmt, q, a, s, si, ws, stream)
    return q, a, s, si


def gemm_workspace(M: int, N: int, K: int, device="cuda"):
    """The workspace te_mxfp8_gemm / te_mxfp8_gemm_mxout use for an M x N x K GEMM (None if none)."""
    n = te_mxfp8_gemm_workspace_size(M, N, K)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def mxfp8_gemm(a, a_scale, a_fmt, b, b_scale, b_fmt, epilogue="none", bias=None, out_dtype=torch.bfloat16,
               aux=None, out=None, stream=None, workspace="auto"):
    """-> (D, aux) for D = epilogue(A . B^T).  aux is written and returned for "bias_gelu_aux" and is
    the saved pre-activation read by "dgelu"; "accumulate" adds into the given fp32 ``out``.
    workspace: "auto" allocates what the GEMM can use, or a tensor, or None for none."""
    M, N = a.shape[0], b.shape[0]
    d = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=a.device)
    if epilogue == "bias_gelu_aux":
        aux = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if isinstance(workspace, str):
        workspace = gemm_workspace(M, N, a.shape[1], a.device)
    te_mxfp8_gemm(a, a_scale, a_fmt, b, b_scale, b_fmt, d, epilogue, bias, aux, workspace, stream)
    return d, (aux if epilogue == "bias_gelu_aux" else None)


def mxfp8_gemm_mxout(a, a_scale, a_fmt, b, b_scale, b_fmt, epilogue="none", bias=None, out_fmt="e4m3",
                     stream=None):
    """-> (codes, scales, aux): D = epilogue(A . B^T) as a rowwise MXFP8 operand (codes [M, N], E8M0
    scales [M, N/32]); aux as mxfp8_gemm."""
    M, N = a.shape[0], b.shape[0]
    d = torch.empty((M, N), dtype=torch.uint8, device=a.device)
    ds = torch.empty((M, N // 32), dtype=torch.uint8, device=a.device)
    aux = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if epilogue == "bias_gelu_aux" else None
    te_mxfp8_gemm_mxout(a, a_scale, a_fmt, b, b_scale, b_fmt, d, ds, out_fmt, epilogue, bias, aux,
                        gemm_workspace(M, N, a.shape[1], a.device), stream)
    return d, ds, aux


def mxfp8_grouped_gemm(m_splits, a, a_scale, a_fmt, b, b_scale, b_fmt, n, epilogue="none", bias=None,
                       out_dtype=torch.bfloat16, aux=None, out=None, stream=None):
    total_m = a.shape[0]
    d = out if out is not None else torch.empty((total_m, n), dtype=out_dtype, device=a.device)
    if epilogue == "bias_gelu_aux":
        aux = torch.empty((total_m, n), dtype=torch.bfloat16, device=a.device)
    te_mxfp8_grouped_gemm(m_splits, a, a_scale, a_fmt, b, b_scale, b_fmt, n, d, epilogue, bias, aux, None, stream)
    return d, (aux if epilogue == "bias_gelu_aux" else None)


def fp8_block_quantize(x, fmt="e4m3", block_2d=False, stream=None):
    """bf16 [rows, cols] -> (codes uint8 [rows, cols], scale_inv float [rows or ceil(rows/128), cols/128])."""
    rows, cols = x.shape
    q = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    srows = (rows + 127) // 128 if block_2d else rows
    s = torch.empty((srows, cols // 128), dtype=torch.float32, device=x.device)
    te_fp8_block_quantize(x, fmt, block_2d, q, s, stream)
    return q, s


def fp8_block_scales_to_mx(scale_inv, rows: int, cols: int, block_2d: bool, stream=None):
    """FP32 block scale inverses -> E8M0 MXFP8 scales uint8 [rows, cols/32]."""
    out = torch.empty((rows, cols // 32), dtype=torch.uint8, device=scale_inv.device)
    te_fp8_block_scales_to_mx(scale_inv, rows, cols, block_2d, out, stream)
    return out


def fp8_block_gemm(a, a_scale_inv, a_fmt, b, b_scale_inv, b_fmt, b_block_2d=True, epilogue="none", bias=None,
                   out_dtype=torch.bfloat16, aux=None, out=None, mode="e8m0", workspace=None, stream=None, beta=1.0):
    """Blockwise FP8 GEMM -> (D, aux); scale inverses float [M, K/128] for A and [N, K/128] (1-D) or
    [ceil(N/128), K/128] (2-D) for B; mode "e8m0" (scales cast to powers of two) or "fp32"; D bf16, fp16
    or fp32; "accumulate" adds into the fp32 ``out`` scaled by ``beta``."""
    M, K = a.shape
    N = b.shape[0]
    d = out if out is not None else torch.empty((M, N), dtype=out_dtype, device=a.device)
    if epilogue == "bias_gelu_aux":
        aux = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    if workspace is None:
        ws_bytes = te_fp8_block_gemm_workspace_size(M, N, K, mode)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=a.device) if ws_bytes else None
    te_fp8_block_gemm(a, a_scale_inv, a_fmt, b, b_scale_inv, b_fmt, b_block_2d, d, epilogue, bias, aux, mode,
                      workspace, stream, beta)
    return d, (aux if epilogue == "bias_gelu_aux" else None)
