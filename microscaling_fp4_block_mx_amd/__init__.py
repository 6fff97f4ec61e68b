"""MXFP4 block quantization on MI355X (gfx950): Python binding of libmx.so.

This module only marshals arguments: every step of quantize, dequantize,
fake-quant and the error reduction runs in the HIP kernels behind the C ABI
declared in include/mx.h. PyTorch supplies device memory and the current
stream. There is no CPU fallback: if libmx.so is missing or a tensor is not
on a GPU, the call raises.

Two layers:
  * ``mx_quantize``, ``mx_dequantize``, ``mx_fakequant``, ``mx_block_mse``,
    ``mx_status_string``: the C entry points, same names and arguments
    (raw device pointers as ints, stream handle as int), returning the status.
  * ``quantize``, ``dequantize``, ``fakequant``, ``block_mse``: tensor-level
    helpers that allocate outputs with torch and raise on a bad status
    (``ValueError`` for argument errors, as the Axolotl MXFP4 PR page does
    for a block size other than 32; ``RuntimeError`` for HIP errors).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmx.so")

MX_OK, MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_DTYPE, MX_ERR_MODE, MX_ERR_ALIGN, MX_ERR_HIP, \
    MX_ERR_ALIAS, MX_ERR_WORKSPACE = range(9)
MX_F32, MX_BF16 = 0, 1
MX_SCALE_OCP, MX_SCALE_OAS, MX_SCALE_OAS_BITS, MX_SCALE_OAS_NF = 0, 1, 2, 3
BLOCK = 32

_MODES = {"ocp": MX_SCALE_OCP, "oas": MX_SCALE_OAS, "oas_bits": MX_SCALE_OAS_BITS,
          "oas_nf": MX_SCALE_OAS_NF}
MODES = tuple(_MODES)
_DTYPES = {torch.float32: MX_F32, torch.bfloat16: MX_BF16}
EXPORTS = ("mx_quantize", "mx_dequantize", "mx_fakequant", "mx_block_mse",
           "mx_block_mse_workspace_size", "mx_quantize_mxfp8", "mx_dequantize_mxfp8",
           "mx_fakequant_mxfp8", "mx_nvfp4_workspace_size", "mx_quantize_nvfp4",
           "mx_dequantize_nvfp4", "mx_quantize_mbs", "mx_dequantize_mbs", "mx_quantize_multi",
           "mx_fakequant_multi", "mx_fakequant_nvfp4", "mx_fakequant_mbs", "mx_quantize_fused",
           "mx_block_mse_noalloc", "mx_status_string", "mx_last_error_detail")

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmx.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m microscaling_fp4_block_mx_amd.build`")
    lib = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.mx_quantize.argtypes = [p, i32, i64, i64, i32, p, p, p]
    lib.mx_dequantize.argtypes = [p, p, i64, i64, i32, p, p]
    lib.mx_fakequant.argtypes = [p, i32, i64, i64, i32, p, p]
    lib.mx_block_mse.argtypes = [p, i32, p, p, i64, i64, p, p, p, ctypes.c_size_t, p]
    lib.mx_block_mse_workspace_size.argtypes = [i64, i64]
    lib.mx_block_mse_noalloc.argtypes = [p, i32, p, p, i64, i64, p, p, p]
    lib.mx_block_mse_workspace_size.restype = ctypes.c_size_t
    lib.mx_quantize_mxfp8.argtypes = [p, i32, i64, i64, p, p, p]
    lib.mx_dequantize_mxfp8.argtypes = [p, p, i64, i64, i32, p, p]
    lib.mx_fakequant_mxfp8.argtypes = [p, i32, i64, i64, p, p]
    lib.mx_nvfp4_workspace_size.argtypes = [i64, i64]
    lib.mx_nvfp4_workspace_size.restype = ctypes.c_size_t
    lib.mx_quantize_nvfp4.argtypes = [p, i32, i64, i64, p, p, p, p, ctypes.c_size_t, p]
    lib.mx_dequantize_nvfp4.argtypes = [p, p, p, i64, i64, i32, p, p]
    lib.mx_quantize_mbs.argtypes = [p, i32, i64, i64, p, p, p, p]
    lib.mx_dequantize_mbs.argtypes = [p, p, p, i64, i64, i32, p, p]
    lib.mx_quantize_fused.argtypes = [p, i32, i64, i64, i32, p, p, p, p, p, p, ctypes.c_size_t, p]
    lib.mx_fakequant_nvfp4.argtypes = [p, i32, i64, i64, p, p, ctypes.c_size_t, p]
    lib.mx_fakequant_mbs.argtypes = [p, i32, i64, i64, p, p]
    lib.mx_quantize_multi.argtypes = [p, i32, i32, i32, p]
    lib.mx_fakequant_multi.argtypes = [p, i32, i32, i32, p]
    for f in ("mx_quantize", "mx_dequantize", "mx_fakequant", "mx_block_mse",
              "mx_quantize_mxfp8", "mx_dequantize_mxfp8", "mx_fakequant_mxfp8",
              "mx_quantize_nvfp4", "mx_dequantize_nvfp4", "mx_quantize_mbs",
              "mx_dequantize_mbs", "mx_quantize_multi", "mx_fakequant_multi",
              "mx_fakequant_nvfp4", "mx_fakequant_mbs", "mx_quantize_fused",
              "mx_block_mse_noalloc"):
        getattr(lib, f).restype = i32
    lib.mx_status_string.argtypes = [i32]
    lib.mx_status_string.restype = ctypes.c_char_p
    lib.mx_last_error_detail.argtypes = []
    lib.mx_last_error_detail.restype = ctypes.c_char_p
    _lib = lib
    return lib


# ---- C entry points, same names -------------------------------------------

def mx_quantize(x, x_dtype, rows, k, mode, codes, scales, stream) -> int:
    return load_library().mx_quantize(x, x_dtype, rows, k, mode, codes, scales, stream)


def mx_dequantize(codes, scales, rows, k, y_dtype, y, stream) -> int:
    return load_library().mx_dequantize(codes, scales, rows, k, y_dtype, y, stream)


def mx_fakequant(x, dtype, rows, k, mode, y, stream) -> int:
    return load_library().mx_fakequant(x, dtype, rows, k, mode, y, stream)


def mx_block_mse(x, x_dtype, codes, scales, rows, k, block_mse, tensor_sums, workspace,
                 workspace_bytes, stream) -> int:
    return load_library().mx_block_mse(x, x_dtype, codes, scales, rows, k, block_mse,
                                       tensor_sums, workspace, workspace_bytes, stream)


def mx_block_mse_workspace_size(rows, k) -> int:
    return load_library().mx_block_mse_workspace_size(rows, k)


def mx_block_mse_noalloc(x, x_dtype, codes, scales, rows, k, block_mse, tensor_sums,
                         stream) -> int:
    return load_library().mx_block_mse_noalloc(x, x_dtype, codes, scales, rows, k, block_mse,
                                               tensor_sums, stream)


def mx_quantize_mxfp8(x, x_dtype, rows, k, codes, scales, stream) -> int:
    return load_library().mx_quantize_mxfp8(x, x_dtype, rows, k, codes, scales, stream)


def mx_dequantize_mxfp8(codes, scales, rows, k, y_dtype, y, stream) -> int:
    return load_library().mx_dequantize_mxfp8(codes, scales, rows, k, y_dtype, y, stream)


def mx_fakequant_mxfp8(x, dtype, rows, k, y, stream) -> int:
    return load_library().mx_fakequant_mxfp8(x, dtype, rows, k, y, stream)


def mx_nvfp4_workspace_size(rows, k) -> int:
    return load_library().mx_nvfp4_workspace_size(rows, k)


def mx_quantize_nvfp4(x, x_dtype, rows, k, codes, block_scales, tensor_scale, workspace,
                      workspace_bytes, stream) -> int:
    return load_library().mx_quantize_nvfp4(x, x_dtype, rows, k, codes, block_scales,
                                            tensor_scale, workspace, workspace_bytes, stream)


def mx_dequantize_nvfp4(codes, block_scales, tensor_scale, rows, k, y_dtype, y, stream) -> int:
    return load_library().mx_dequantize_nvfp4(codes, block_scales, tensor_scale, rows, k,
                                              y_dtype, y, stream)


def mx_quantize_mbs(x, x_dtype, rows, k, codes, sub_scales, macro_mant, stream) -> int:
    return load_library().mx_quantize_mbs(x, x_dtype, rows, k, codes, sub_scales, macro_mant,
                                          stream)


def mx_dequantize_mbs(codes, sub_scales, macro_mant, rows, k, y_dtype, y, stream) -> int:
    return load_library().mx_dequantize_mbs(codes, sub_scales, macro_mant, rows, k, y_dtype, y,
                                            stream)


def mx_quantize_fused(x, x_dtype, rows, k, mode, codes, scales, y, block_mse, tensor_sums,
                      workspace, workspace_bytes, stream) -> int:
    return load_library().mx_quantize_fused(x, x_dtype, rows, k, mode, codes, scales, y,
                                            block_mse, tensor_sums, workspace, workspace_bytes,
                                            stream)


def mx_fakequant_nvfp4(x, dtype, rows, k, y, workspace, workspace_bytes, stream) -> int:
    return load_library().mx_fakequant_nvfp4(x, dtype, rows, k, y, workspace, workspace_bytes,
                                             stream)


def mx_fakequant_mbs(x, dtype, rows, k, y, stream) -> int:
    return load_library().mx_fakequant_mbs(x, dtype, rows, k, y, stream)


class MxTensor(ctypes.Structure):
    """mx_tensor_t of include/mx.h (pointers as integers)."""
    _fields_ = [("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("rows", ctypes.c_int64), ("k", ctypes.c_int64)]


def mx_quantize_multi(tensors, count, dtype, mode, stream) -> int:
    return load_library().mx_quantize_multi(tensors, count, dtype, mode, stream)


def mx_fakequant_multi(tensors, count, dtype, mode, stream) -> int:
    return load_library().mx_fakequant_multi(tensors, count, dtype, mode, stream)


def mx_status_string(status: int) -> str:
    return load_library().mx_status_string(status).decode()


def mx_last_error_detail() -> str:
    return load_library().mx_last_error_detail().decode()


# ---- tensor helpers --------------------------------------------------------

def _raise(status: int, with_detail: bool = False):
    if status == MX_OK:
        return
    msg = mx_status_string(status)
    if status == MX_ERR_HIP:
        raise RuntimeError(msg + ": " + load_library().mx_last_error_detail().decode())
    if with_detail:
        msg += " (" + load_library().mx_last_error_detail().decode() + ")"
    raise ValueError(msg)


def _check_input(x: torch.Tensor):
    if not isinstance(x, torch.Tensor) or not x.is_cuda:
        raise ValueError("MXFP4 kernels need a GPU tensor")
    if x.dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {x.dtype}")
    if x.dim() == 0:
        raise ValueError("need at least one dimension")
    if not x.is_contiguous():
        raise ValueError("input must be contiguous")
    k = x.shape[-1]
    if k <= 0 or k % BLOCK:
        raise ValueError("MXFP4 needs the last dimension to be a multiple of 32")
    return x.numel() // k if x.numel() else 0, k


def _need(t, name: str, device, dtype=None, numel=None):
    """A tensor the kernels will read or write: on `device`, contiguous, of
    `dtype` and `numel` when given. Anything else is refused here, before a
    pointer reaches the GPU."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return t


def _stream(dev) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _mode(mode: str) -> int:
    try:
        return _MODES[mode]
    except KeyError:
        raise ValueError(f"mode must be one of {MODES}, got {mode!r}") from None


def quantize(x: torch.Tensor, mode: str = "ocp", codes: torch.Tensor | None = None,
             scales: torch.Tensor | None = None):
    """x [..., k] -> (codes uint8 [..., k/2], scales uint8 [..., k/32])."""
    rows, k = _check_input(x)
    lead = tuple(x.shape[:-1])
    if codes is None:
        codes = torch.empty(lead + (k // 2,), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(lead + (k // BLOCK,), dtype=torch.uint8, device=x.device)
    _need(codes, "codes", x.device, torch.uint8, x.numel() // 2)
    _need(scales, "scales", x.device, torch.uint8, x.numel() // BLOCK)
    with torch.cuda.device(x.device):
        _raise(mx_quantize(x.data_ptr(), _DTYPES[x.dtype], rows, k, _mode(mode),
                           codes.data_ptr(), scales.data_ptr(), _stream(x.device)))
    return codes, scales


def dequantize(codes: torch.Tensor, scales: torch.Tensor, dtype=torch.bfloat16,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """codes [..., k/2] + scales [..., k/32] -> y [..., k] in dtype."""
    _need(codes, "codes", getattr(codes, "device", None), torch.uint8)
    _need(scales, "scales", codes.device, torch.uint8)
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {dtype}")
    k = codes.shape[-1] * 2
    rows = codes.numel() // (k // 2) if codes.numel() else 0
    if scales.numel() * BLOCK != codes.numel() * 2:
        raise ValueError("scales do not match codes")
    if out is None:
        out = torch.empty(tuple(codes.shape[:-1]) + (k,), dtype=dtype, device=codes.device)
    _need(out, "out", codes.device, dtype, codes.numel() * 2)
    with torch.cuda.device(codes.device):
        _raise(mx_dequantize(codes.data_ptr(), scales.data_ptr(), rows, k, _DTYPES[dtype],
                             out.data_ptr(), _stream(codes.device)))
    return out


def fakequant(x: torch.Tensor, mode: str = "ocp", out: torch.Tensor | None = None) -> torch.Tensor:
    """dequantize(quantize(x)) in x's dtype; out may be x (in place)."""
    rows, k = _check_input(x)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.device, x.dtype, x.numel())
    with torch.cuda.device(x.device):
        _raise(mx_fakequant(x.data_ptr(), _DTYPES[x.dtype], rows, k, _mode(mode),
                            out.data_ptr(), _stream(x.device)))
    return out


def block_mse(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
              per_block: bool = True):
    """-> (block_mse float32 [..., k/32] or None, sums float64 GPU tensor [2])
    with sums[0] = sum (x - x_hat)^2 and sums[1] = sum x^2. Tensor MSE =
    sums[0] / x.numel(); QSNR = 10 log10(sums[1] / sums[0]) dB."""
    rows, k = _check_input(x)
    _need(codes, "codes", x.device, torch.uint8, x.numel() // 2)
    _need(scales, "scales", x.device, torch.uint8, x.numel() // BLOCK)
    bm = None
    if per_block:
        bm = torch.empty(tuple(x.shape[:-1]) + (k // BLOCK,), dtype=torch.float32,
                         device=x.device)
    sums = torch.empty(2, dtype=torch.float64, device=x.device)
    ws_bytes = mx_block_mse_workspace_size(rows, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _raise(mx_block_mse(x.data_ptr(), _DTYPES[x.dtype], codes.data_ptr(), scales.data_ptr(),
                            rows, k, bm.data_ptr() if bm is not None else None,
                            sums.data_ptr(), ws.data_ptr(), ws_bytes, _stream(x.device)))
    return bm, sums


def quantize_fused(x: torch.Tensor, mode: str = "ocp", want_y: bool = True,
                   want_block_mse: bool = True, want_sums: bool = True):
    """One pass: -> (codes, scales, y or None, block_mse or None, sums or
    None), equal to quantize(), then dequantize() in x's dtype, then
    block_mse() (sums to a relative 1e-6)."""
    rows, k = _check_input(x)
    lead = tuple(x.shape[:-1])
    codes = torch.empty(lead + (k // 2,), dtype=torch.uint8, device=x.device)
    scales = torch.empty(lead + (k // BLOCK,), dtype=torch.uint8, device=x.device)
    y = torch.empty_like(x) if want_y else None
    bm = (torch.empty(lead + (k // BLOCK,), dtype=torch.float32, device=x.device)
          if want_block_mse else None)
    sums = torch.empty(2, dtype=torch.float64, device=x.device) if want_sums else None
    ws_bytes = mx_block_mse_workspace_size(rows, k) if want_sums else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device) if want_sums else None
    ptr = lambda t: t.data_ptr() if t is not None else None  # noqa: E731
    with torch.cuda.device(x.device):
        _raise(mx_quantize_fused(x.data_ptr(), _DTYPES[x.dtype], rows, k, _mode(mode),
                                 codes.data_ptr(), scales.data_ptr(), ptr(y), ptr(bm), ptr(sums),
                                 ptr(ws), ws_bytes, _stream(x.device)))
    return codes, scales, y, bm, sums


# ---- MXFP8 (E4M3) tensor helpers ---------------------------------------------

def quantize_mxfp8(x: torch.Tensor, codes: torch.Tensor | None = None,
                   scales: torch.Tensor | None = None):
    """x [..., k] -> (codes uint8 [..., k] (E4M3 bytes), scales uint8 [..., k/32])."""
    rows, k = _check_input(x)
    if codes is None:
        codes = torch.empty(tuple(x.shape), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(tuple(x.shape[:-1]) + (k // BLOCK,), dtype=torch.uint8,
                             device=x.device)
    _need(codes, "codes", x.device, torch.uint8, x.numel())
    _need(scales, "scales", x.device, torch.uint8, x.numel() // BLOCK)
    with torch.cuda.device(x.device):
        _raise(mx_quantize_mxfp8(x.data_ptr(), _DTYPES[x.dtype], rows, k, codes.data_ptr(),
                                 scales.data_ptr(), _stream(x.device)))
    return codes, scales


def dequantize_mxfp8(codes: torch.Tensor, scales: torch.Tensor, dtype=torch.bfloat16,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """E4M3 codes [..., k] + scales [..., k/32] -> y [..., k] in dtype."""
    _need(codes, "codes", getattr(codes, "device", None), torch.uint8)
    _need(scales, "scales", codes.device, torch.uint8)
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {dtype}")
    k = codes.shape[-1]
    if k <= 0 or k % BLOCK:
        raise ValueError("MXFP8 needs the last dimension to be a multiple of 32")
    rows = codes.numel() // k if codes.numel() else 0
    if scales.numel() * BLOCK != codes.numel():
        raise ValueError("scales do not match codes")
    if out is None:
        out = torch.empty(tuple(codes.shape), dtype=dtype, device=codes.device)
    _need(out, "out", codes.device, dtype, codes.numel())
    with torch.cuda.device(codes.device):
        _raise(mx_dequantize_mxfp8(codes.data_ptr(), scales.data_ptr(), rows, k, _DTYPES[dtype],
                                   out.data_ptr(), _stream(codes.device)))
    return out


def fakequant_mxfp8(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """dequantize_mxfp8(quantize_mxfp8(x)) in x's dtype; out may be x."""
    rows, k = _check_input(x)
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.device, x.dtype, x.numel())
    with torch.cuda.device(x.device):
        _raise(mx_fakequant_mxfp8(x.data_ptr(), _DTYPES[x.dtype], rows, k, out.data_ptr(),
                                  _stream(x.device)))
    return out


# ---- NVFP4 comparator tensor helpers -----------------------------------------

def quantize_nvfp4(x: torch.Tensor):
    """x [..., k] (k % 16 == 0) -> (codes uint8 [..., k/2], block_scales uint8
    [..., k/16] (E4M3 bytes), tensor_scale uint8 GPU tensor [1] (t + 127))."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype not in _DTYPES:
        raise ValueError("need a float32/bfloat16 GPU tensor")
    if x.dim() == 0 or not x.is_contiguous():
        raise ValueError("need a contiguous tensor with at least one dimension")
    k = x.shape[-1]
    if k <= 0 or k % 16:
        raise ValueError("NVFP4 needs the last dimension to be a multiple of 16")
    rows = x.numel() // k if x.numel() else 0
    codes = torch.empty(tuple(x.shape[:-1]) + (k // 2,), dtype=torch.uint8, device=x.device)
    bs = torch.empty(tuple(x.shape[:-1]) + (k // 16,), dtype=torch.uint8, device=x.device)
    ts = torch.full((1,), 127, dtype=torch.uint8, device=x.device)
    wsb = mx_nvfp4_workspace_size(rows, k)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _raise(mx_quantize_nvfp4(x.data_ptr(), _DTYPES[x.dtype], rows, k, codes.data_ptr(),
                                 bs.data_ptr(), ts.data_ptr(), ws.data_ptr(), wsb,
                                 _stream(x.device)))
    return codes, bs, ts


def _check_input_n(x, multiple: int, what: str):
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype not in _DTYPES:
        raise ValueError("need a float32/bfloat16 GPU tensor")
    if x.dim() == 0 or not x.is_contiguous():
        raise ValueError("need a contiguous tensor with at least one dimension")
    k = x.shape[-1]
    if k <= 0 or k % multiple:
        raise ValueError(f"{what} needs the last dimension to be a multiple of {multiple}")
    return x.numel() // k if x.numel() else 0, k


def fakequant_nvfp4(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """dequantize_nvfp4(quantize_nvfp4(x)) in x's dtype, fused; out may be x."""
    rows, k = _check_input_n(x, 16, "NVFP4")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.device, x.dtype, x.numel())
    wsb = mx_nvfp4_workspace_size(rows, k)
    ws = torch.empty(max(wsb, 4), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _raise(mx_fakequant_nvfp4(x.data_ptr(), _DTYPES[x.dtype], rows, k, out.data_ptr(),
                                  ws.data_ptr(), wsb, _stream(x.device)))
    return out


def dequantize_nvfp4(codes: torch.Tensor, block_scales: torch.Tensor, tensor_scale: torch.Tensor,
                     dtype=torch.bfloat16) -> torch.Tensor:
    _need(codes, "codes", getattr(codes, "device", None), torch.uint8)
    _need(block_scales, "block_scales", codes.device, torch.uint8)
    _need(tensor_scale, "tensor_scale", codes.device, torch.uint8, 1)
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {dtype}")
    k = codes.shape[-1] * 2
    rows = codes.numel() // (k // 2) if codes.numel() else 0
    if block_scales.numel() * 16 != codes.numel() * 2:
        raise ValueError("block scales do not match codes")
    y = torch.empty(tuple(codes.shape[:-1]) + (k,), dtype=dtype, device=codes.device)
    with torch.cuda.device(codes.device):
        _raise(mx_dequantize_nvfp4(codes.data_ptr(), block_scales.data_ptr(),
                                   tensor_scale.data_ptr(), rows, k, _DTYPES[dtype], y.data_ptr(),
                                   _stream(codes.device)))
    return y


# ---- MBS-Static tensor helpers ------------------------------------------------

def quantize_mbs(x: torch.Tensor):
    """x [..., k] (k % 128 == 0) -> (codes uint8 [..., k/2], sub_scales uint8
    [..., k/16] (E8M0 bytes), macro_mant uint8 [..., k/128])."""
    if not isinstance(x, torch.Tensor) or not x.is_cuda or x.dtype not in _DTYPES:
        raise ValueError("need a float32/bfloat16 GPU tensor")
    if x.dim() == 0 or not x.is_contiguous():
        raise ValueError("need a contiguous tensor with at least one dimension")
    k = x.shape[-1]
    if k <= 0 or k % 128:
        raise ValueError("MBS-Static needs the last dimension to be a multiple of 128")
    rows = x.numel() // k if x.numel() else 0
    lead = tuple(x.shape[:-1])
    codes = torch.empty(lead + (k // 2,), dtype=torch.uint8, device=x.device)
    ss = torch.empty(lead + (k // 16,), dtype=torch.uint8, device=x.device)
    mm = torch.empty(lead + (k // 128,), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _raise(mx_quantize_mbs(x.data_ptr(), _DTYPES[x.dtype], rows, k, codes.data_ptr(),
                               ss.data_ptr(), mm.data_ptr(), _stream(x.device)))
    return codes, ss, mm


def fakequant_mbs(x: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """dequantize_mbs(quantize_mbs(x)) in x's dtype, fused; out may be x."""
    rows, k = _check_input_n(x, 128, "MBS-Static")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.device, x.dtype, x.numel())
    with torch.cuda.device(x.device):
        _raise(mx_fakequant_mbs(x.data_ptr(), _DTYPES[x.dtype], rows, k, out.data_ptr(),
                                _stream(x.device)))
    return out


def dequantize_mbs(codes: torch.Tensor, sub_scales: torch.Tensor, macro_mant: torch.Tensor,
                   dtype=torch.bfloat16) -> torch.Tensor:
    _need(codes, "codes", getattr(codes, "device", None), torch.uint8)
    _need(sub_scales, "sub_scales", codes.device, torch.uint8)
    _need(macro_mant, "macro_mant", codes.device, torch.uint8)
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {dtype}")
    k = codes.shape[-1] * 2
    rows = codes.numel() // (k // 2) if codes.numel() else 0
    if sub_scales.numel() * 16 != codes.numel() * 2 or macro_mant.numel() * 128 != codes.numel() * 2:
        raise ValueError("sub_scales / macro_mant do not match codes")
    y = torch.empty(tuple(codes.shape[:-1]) + (k,), dtype=dtype, device=codes.device)
    with torch.cuda.device(codes.device):
        _raise(mx_dequantize_mbs(codes.data_ptr(), sub_scales.data_ptr(), macro_mant.data_ptr(),
                                 rows, k, _DTYPES[dtype], y.data_ptr(), _stream(codes.device)))
    return y


# ---- many tensors in one call --------------------------------------------------

def _multi_inputs(xs):
    xs = list(xs)
    if not xs:
        return xs, None, None
    dev, dt = xs[0].device, xs[0].dtype
    for x in xs:
        _check_input(x)
        if x.device != dev or x.dtype != dt:
            raise ValueError("all tensors must share one device and dtype")
    return xs, dev, dt


def quantize_multi(xs, mode: str = "ocp"):
    """[x_i [..., k_i]] -> [(codes_i, scales_i)], as quantize() per tensor,
    with one launch per group of up to 60 tensors of similar size."""
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {MODES}")
    xs, dev, dt = _multi_inputs(xs)
    outs = []
    arr = (MxTensor * max(1, len(xs)))()
    for i, x in enumerate(xs):
        k = x.shape[-1]
        rows = x.numel() // k if x.numel() else 0
        c = torch.empty(tuple(x.shape[:-1]) + (k // 2,), dtype=torch.uint8, device=dev)
        s = torch.empty(tuple(x.shape[:-1]) + (k // BLOCK,), dtype=torch.uint8, device=dev)
        outs.append((c, s))
        arr[i] = MxTensor(x.data_ptr(), None, c.data_ptr(), s.data_ptr(), rows, k)
    if xs:
        with torch.cuda.device(dev):
            _raise(mx_quantize_multi(arr, len(xs), _DTYPES[dt], _MODES[mode], _stream(dev)), True)
    return outs


def fakequant_multi(xs, mode: str = "ocp", out=None):
    """[x_i] -> [y_i], as fakequant() per tensor, with one launch per group
    of up to 60 tensors of similar size; out may be a list of preallocated
    outputs (or the inputs, in place)."""
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {MODES}")
    xs, dev, dt = _multi_inputs(xs)
    ys = list(out) if out is not None else [torch.empty_like(x) for x in xs]
    if len(ys) != len(xs):
        raise ValueError("out must have one tensor per input")
    arr = (MxTensor * max(1, len(xs)))()
    for i, (x, y) in enumerate(zip(xs, ys)):
        if y.dtype != x.dtype or y.numel() != x.numel() or not y.is_contiguous() \
                or y.device != x.device:
            raise ValueError("each out tensor must be a contiguous tensor like its input")
        k = x.shape[-1]
        rows = x.numel() // k if x.numel() else 0
        arr[i] = MxTensor(x.data_ptr(), y.data_ptr(), None, None, rows, k)
    if xs:
        with torch.cuda.device(dev):
            _raise(mx_fakequant_multi(arr, len(xs), _DTYPES[dt], _MODES[mode], _stream(dev)), True)
    return ys
