"""CPU oracle for OCP MXFP4 block quantization (TEST INFRASTRUCTURE).

A plain, slow, scalar C implementation (``mxref.c``) of what the GPU library
computes, plus this ctypes wrapper over host numpy arrays. It is the checker,
not the product: only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import it. It shares no code with the GPU
library and imports nothing from it.

Array conventions (host numpy):
  * fp32 data: ``np.float32`` arrays.
  * bf16 data: ``np.uint16`` arrays holding bfloat16 bit patterns.
  * codes: ``np.uint8 [rows, k/2]``; scales: ``np.uint8 [rows, k/32]``.

Parity is pinned, not assumed: ``tests/test_oracle_*.py`` check this oracle
against closed forms of the E2M1/E8M0 formats, an exact-rational brute force,
hand-derived worked blocks under ``tests/golden/`` and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxref.c")
_LIB = os.path.join(_HERE, "libmxref.so")

F32, BF16 = 0, 1
OCP, OAS, OAS_BITS, OAS_NF = 0, 1, 2, 3
_MODES = {"ocp": OCP, "oas": OAS, "oas_bits": OAS_BITS, "oas_nf": OAS_NF}
MODES = tuple(_MODES)

_lib = None


def build(force: bool = True) -> str:
    """Compile libmxref.so with gcc (strict IEEE: no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        cmd = [
            "gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-ffp-contract=off",
            "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra",
            "-o", _LIB + ".tmp", _SRC, "-lm", "-lpthread",
        ]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.mxref_quantize.argtypes = [p, i32, i64, i64, i32, p, p, i32]
        lib.mxref_dequantize.argtypes = [p, p, i64, i64, i32, p, i32]
        lib.mxref_fakequant.argtypes = [p, i32, i64, i64, i32, p, i32]
        lib.mxref_block_mse.argtypes = [p, i32, p, p, i64, i64, p, p, i32]
        for f in ("mxref_quantize", "mxref_dequantize", "mxref_fakequant",
                  "mxref_block_mse"):
            getattr(lib, f).restype = i32
        lib.mxref_ocp_scale.argtypes = [ctypes.c_double]
        lib.mxref_ocp_scale.restype = i32
        lib.mxref_encode.argtypes = [ctypes.c_double, i32]
        lib.mxref_encode.restype = i32
        lib.mxref_decode.argtypes = [i32, i32]
        lib.mxref_decode.restype = ctypes.c_double
        lib.mxref_oas_sse32.argtypes = [ctypes.POINTER(ctypes.c_double), i32, i32]
        lib.mxref_oas_sse32.restype = ctypes.c_float
        lib.mxref8_quantize.argtypes = [p, i32, i64, i64, p, p, i32]
        lib.mxref8_dequantize.argtypes = [p, p, i64, i64, i32, p, i32]
        lib.mxref8_fakequant.argtypes = [p, i32, i64, i64, p, i32]
        for f in ("mxref8_quantize", "mxref8_dequantize", "mxref8_fakequant"):
            getattr(lib, f).restype = i32
        lib.mxref8_scale.argtypes = [ctypes.c_double]
        lib.mxref8_scale.restype = i32
        lib.mxref8_encode.argtypes = [ctypes.c_double, i32]
        lib.mxref8_encode.restype = i32
        lib.mxref8_decode.argtypes = [i32, i32]
        lib.mxref8_decode.restype = ctypes.c_double
        lib.mxrefnv_quantize.argtypes = [p, i32, i64, i64, p, p, p]
        lib.mxrefnv_quantize.restype = i32
        lib.mxrefnv_dequantize.argtypes = [p, p, i32, i64, i64, i32, p]
        lib.mxrefnv_dequantize.restype = i32
        lib.mxrefnv_tensor_exp.argtypes = [ctypes.c_double]
        lib.mxrefnv_tensor_exp.restype = i32
        lib.mxrefnv_decode.argtypes = [i32, i32, i32]
        lib.mxrefnv_decode.restype = ctypes.c_double
        lib.mxrefmbs_quantize.argtypes = [p, i32, i64, i64, p, p, p]
        lib.mxrefmbs_quantize.restype = i32
        lib.mxrefmbs_dequantize.argtypes = [p, p, p, i64, i64, i32, p]
        lib.mxrefmbs_dequantize.restype = i32
        lib.mxrefmbs_macro_mantissa.argtypes = [ctypes.c_double]
        lib.mxrefmbs_macro_mantissa.restype = i32
        _lib = lib
    return _lib


def _dtype_code(arr: np.ndarray) -> int:
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise ValueError(f"oracle takes float32 or uint16 (bf16 bits), got {arr.dtype}")


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _shape2(x: np.ndarray):
    if x.ndim == 0:
        raise ValueError("need at least 1 dim")
    k = x.shape[-1]
    rows = int(np.prod(x.shape[:-1])) if x.ndim > 1 else 1
    return rows, k


def _check(rc: int):
    if rc == -2:
        raise ValueError("last dim must be a positive multiple of 32")
    if rc != 0:
        raise RuntimeError(f"oracle error {rc}")


def quantize(x: np.ndarray, mode: str = "ocp", threads: int = 1):
    """Return (codes uint8 [..., k/2], scales uint8 [..., k/32])."""
    x = np.ascontiguousarray(x)
    rows, k = _shape2(x)
    codes = np.empty(x.shape[:-1] + (k // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (k // 32,), np.uint8)
    _check(_load().mxref_quantize(_ptr(x), _dtype_code(x), rows, k, _MODES[mode],
                                  _ptr(codes), _ptr(scales), threads))
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, dtype: str = "bf16",
               threads: int = 1) -> np.ndarray:
    """Return y [..., k] as float32 or uint16 (bf16 bits)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    k = codes.shape[-1] * 2
    rows = int(np.prod(codes.shape[:-1])) if codes.ndim > 1 else 1
    if scales.size != rows * (k // 32):
        raise ValueError("scales do not match codes")
    npdt = np.float32 if dtype == "f32" else np.uint16
    y = np.empty(codes.shape[:-1] + (k,), npdt)
    _check(_load().mxref_dequantize(_ptr(codes), _ptr(scales), rows, k,
                                    F32 if dtype == "f32" else BF16, _ptr(y), threads))
    return y


def fakequant(x: np.ndarray, mode: str = "ocp", threads: int = 1) -> np.ndarray:
    """Return dequantize(quantize(x)) in x's dtype."""
    x = np.ascontiguousarray(x)
    rows, k = _shape2(x)
    y = np.empty_like(x)
    _check(_load().mxref_fakequant(_ptr(x), _dtype_code(x), rows, k, _MODES[mode],
                                   _ptr(y), threads))
    return y


def block_mse(x: np.ndarray, codes: np.ndarray, scales: np.ndarray,
              threads: int = 1, with_energy: bool = False):
    """Return (block_mse float32 [..., k/32], tensor_sse float), or with
    with_energy=True (block_mse, tensor_sse, sum of x^2)."""
    x = np.ascontiguousarray(x)
    rows, k = _shape2(x)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    bm = np.empty(x.shape[:-1] + (k // 32,), np.float32)
    sums = np.zeros(2, np.float64)
    _check(_load().mxref_block_mse(_ptr(x), _dtype_code(x), _ptr(codes), _ptr(scales),
                                   rows, k, _ptr(bm), _ptr(sums), threads))
    if with_energy:
        return bm, float(sums[0]), float(sums[1])
    return bm, float(sums[0])


def qsnr_db(x: np.ndarray, codes: np.ndarray, scales: np.ndarray, threads: int = 1) -> float:
    """10 log10(sum x^2 / sum (x - x_hat)^2) of the whole tensor."""
    _, sse, ssq = block_mse(x, codes, scales, threads, with_energy=True)
    return float(10.0 * np.log10(ssq / sse))


# --- single-element helpers (used by the oracle's own pins) -----------------

def ocp_scale(amax: float) -> int:
    return _load().mxref_ocp_scale(float(amax))


def encode(x: float, scale_byte: int) -> int:
    return _load().mxref_encode(float(x), int(scale_byte))


def decode(code: int, scale_byte: int) -> float:
    return _load().mxref_decode(int(code), int(scale_byte))


def oas_sse32(block: np.ndarray, scale_byte: int, unit_byte: int | None = None) -> float:
    """Pinned fp32 squared error of a 32-element block at candidate byte
    scale_byte, measured in units of 2^(unit_byte - 127) (unit_byte: the
    larger of the two candidates; default scale_byte)."""
    b = np.ascontiguousarray(block, dtype=np.float64)
    assert b.shape == (32,)
    h = int(scale_byte) if unit_byte is None else int(unit_byte)
    return float(_load().mxref_oas_sse32(b.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                                         int(scale_byte), h))


# --- MXFP8 (E4M3 elements, one byte each) ----------------------------------

def quantize_mxfp8(x: np.ndarray, threads: int = 1):
    """Return (codes uint8 [..., k], scales uint8 [..., k/32])."""
    x = np.ascontiguousarray(x)
    rows, k = _shape2(x)
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1] + (k // 32,), np.uint8)
    _check(_load().mxref8_quantize(_ptr(x), _dtype_code(x), rows, k, _ptr(codes), _ptr(scales),
                                   threads))
    return codes, scales


def dequantize_mxfp8(codes: np.ndarray, scales: np.ndarray, dtype: str = "bf16",
                     threads: int = 1) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    k = codes.shape[-1]
    rows = int(np.prod(codes.shape[:-1])) if codes.ndim > 1 else 1
    if scales.size != rows * (k // 32):
        raise ValueError("scales do not match codes")
    y = np.empty(codes.shape, np.float32 if dtype == "f32" else np.uint16)
    _check(_load().mxref8_dequantize(_ptr(codes), _ptr(scales), rows, k,
                                     F32 if dtype == "f32" else BF16, _ptr(y), threads))
    return y


def fakequant_mxfp8(x: np.ndarray, threads: int = 1) -> np.ndarray:
    x = np.ascontiguousarray(x)
    rows, k = _shape2(x)
    y = np.empty_like(x)
    _check(_load().mxref8_fakequant(_ptr(x), _dtype_code(x), rows, k, _ptr(y), threads))
    return y


def scale_mxfp8(amax: float) -> int:
    return _load().mxref8_scale(float(amax))


def encode_e4m3(x: float, scale_byte: int) -> int:
    return _load().mxref8_encode(float(x), int(scale_byte))


def decode_e4m3(code: int, scale_byte: int) -> float:
    return _load().mxref8_decode(int(code), int(scale_byte))


# --- NVFP4 comparator (16-element blocks, E4M3 block scales) ---------------

def quantize_nvfp4(x: np.ndarray):
    """Return (codes uint8 [..., k/2], block_scales uint8 [..., k/16] (E4M3),
    tensor_scale int (byte t + 127 of the factor 2^t))."""
    x = np.ascontiguousarray(x)
    rows, k = _shape2(x)
    codes = np.empty(x.shape[:-1] + (k // 2,), np.uint8)
    bs = np.empty(x.shape[:-1] + (k // 16,), np.uint8)
    ts = np.zeros(1, np.uint8)
    rc = _load().mxrefnv_quantize(_ptr(x), _dtype_code(x), rows, k, _ptr(codes), _ptr(bs), _ptr(ts))
    if rc == -2:
        raise ValueError("last dim must be a positive multiple of 16")
    _check(rc)
    return codes, bs, int(ts[0])


def dequantize_nvfp4(codes: np.ndarray, block_scales: np.ndarray, tensor_scale: int,
                     dtype: str = "bf16") -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    bs = np.ascontiguousarray(block_scales, dtype=np.uint8)
    k = codes.shape[-1] * 2
    rows = int(np.prod(codes.shape[:-1])) if codes.ndim > 1 else 1
    y = np.empty(codes.shape[:-1] + (k,), np.float32 if dtype == "f32" else np.uint16)
    _check(_load().mxrefnv_dequantize(_ptr(codes), _ptr(bs), int(tensor_scale), rows, k,
                                      F32 if dtype == "f32" else BF16, _ptr(y)))
    return y


def nvfp4_tensor_exp(amax: float) -> int:
    return _load().mxrefnv_tensor_exp(float(amax))


def nvfp4_decode(code: int, block_scale: int, tensor_scale: int) -> float:
    return _load().mxrefnv_decode(int(code), int(block_scale), int(tensor_scale))


# --- MBS-Static (16-element sub-blocks, 8-bit-mantissa macro factor) --------

def quantize_mbs(x: np.ndarray):
    """Return (codes [..., k/2], sub_scales [..., k/16] (E8M0 bytes),
    macro_mant [..., k/128] (factor 1 + m/256))."""
    x = np.ascontiguousarray(x)
    rows, k = _shape2(x)
    codes = np.empty(x.shape[:-1] + (k // 2,), np.uint8)
    ss = np.empty(x.shape[:-1] + (k // 16,), np.uint8)
    mm = np.empty(x.shape[:-1] + (k // 128,), np.uint8)
    rc = _load().mxrefmbs_quantize(_ptr(x), _dtype_code(x), rows, k, _ptr(codes), _ptr(ss), _ptr(mm))
    if rc == -2:
        raise ValueError("last dim must be a positive multiple of 128")
    _check(rc)
    return codes, ss, mm


def dequantize_mbs(codes, sub_scales, macro_mant, dtype: str = "bf16") -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    k = codes.shape[-1] * 2
    rows = int(np.prod(codes.shape[:-1])) if codes.ndim > 1 else 1
    y = np.empty(codes.shape[:-1] + (k,), np.float32 if dtype == "f32" else np.uint16)
    _check(_load().mxrefmbs_dequantize(_ptr(codes), _ptr(np.ascontiguousarray(sub_scales, np.uint8)),
                                       _ptr(np.ascontiguousarray(macro_mant, np.uint8)), rows, k,
                                       F32 if dtype == "f32" else BF16, _ptr(y)))
    return y


def mbs_macro_mantissa(amax: float) -> int:
    return _load().mxrefmbs_macro_mantissa(float(amax))
