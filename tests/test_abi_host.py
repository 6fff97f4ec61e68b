"""Host-side checks of the C ABI: the library loads, exports every entry point
include/mx.h declares, and rejects bad arguments synchronously. Every call
here fails validation before any HIP call, so no GPU is needed."""
import ctypes
import os
import re

import pytest

import microscaling_fp4_block_mx_amd as mx
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "mx.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.LIB_PATH):
        from microscaling_fp4_block_mx_amd import build
        build.build()
    return mx.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(mx_\w+)\s*\(", text, re.M)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(mx.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(9):
        assert mx.mx_status_string(s).startswith("MX_")
    assert "unknown" in mx.mx_status_string(99)


A = 1 << 20  # fake, 16-byte aligned addresses: validation fails before any use
B = 2 << 30
C = 3 << 30
W = 5 << 30  # fake workspace / tensor_sums region


@pytest.mark.parametrize("rows,k", [(-1, 32), (1, 0), (1, -32), (4, 48), (2, 33),
                                    (1 << 40, 1 << 30)])
def test_bad_shapes(lib, rows, k):
    assert mx.mx_quantize(A, mx.MX_BF16, rows, k, 0, B, C, None) == mx.MX_ERR_SHAPE
    assert mx.mx_dequantize(B, C, rows, k, mx.MX_F32, A, None) == mx.MX_ERR_SHAPE
    assert mx.mx_fakequant(A, mx.MX_F32, rows, k, 0, B, None) == mx.MX_ERR_SHAPE
    assert mx.mx_block_mse(A, mx.MX_F32, B, C, rows, k, A + (64 << 30), None, None, 0,
                           None) == mx.MX_ERR_SHAPE
    assert mx.mx_block_mse_workspace_size(rows, k) == 0


def test_bad_dtype_and_mode(lib):
    assert mx.mx_quantize(A, 2, 1, 32, 0, B, C, None) == mx.MX_ERR_DTYPE
    assert mx.mx_quantize(A, mx.MX_BF16, 1, 32, 4, B, C, None) == mx.MX_ERR_MODE
    assert mx.mx_quantize(A, mx.MX_BF16, 1, 32, -1, B, C, None) == mx.MX_ERR_MODE
    assert mx.mx_dequantize(B, C, 1, 32, 7, A, None) == mx.MX_ERR_DTYPE
    assert mx.mx_fakequant(A, -1, 1, 32, 0, B, None) == mx.MX_ERR_DTYPE
    assert mx.mx_fakequant(A, mx.MX_F32, 1, 32, 9, B, None) == mx.MX_ERR_MODE
    assert mx.mx_block_mse(A, 5, B, C, 1, 32, None, A + 64, W, 64, None) == mx.MX_ERR_DTYPE


def test_null_pointers(lib):
    assert mx.mx_quantize(None, mx.MX_BF16, 1, 32, 0, B, C, None) == mx.MX_ERR_NULL
    assert mx.mx_quantize(A, mx.MX_BF16, 1, 32, 0, None, C, None) == mx.MX_ERR_NULL
    assert mx.mx_quantize(A, mx.MX_BF16, 1, 32, 0, B, None, None) == mx.MX_ERR_NULL
    assert mx.mx_dequantize(None, C, 1, 32, 0, A, None) == mx.MX_ERR_NULL
    assert mx.mx_dequantize(B, C, 1, 32, 0, None, None) == mx.MX_ERR_NULL
    assert mx.mx_fakequant(A, 0, 1, 32, 0, None, None) == mx.MX_ERR_NULL
    # both error outputs NULL
    assert mx.mx_block_mse(A, 0, B, C, 1, 32, None, None, W, 64, None) == mx.MX_ERR_NULL
    assert mx.mx_block_mse(None, 0, B, C, 1, 32, A + 64, None, None, 0, None) == mx.MX_ERR_NULL


def test_empty_is_ok_without_launch(lib):
    assert mx.mx_quantize(None, mx.MX_BF16, 0, 32, 0, None, None, None) == mx.MX_OK
    assert mx.mx_dequantize(None, None, 0, 4096, 0, None, None) == mx.MX_OK
    assert mx.mx_fakequant(None, 1, 0, 64, 1, None, None) == mx.MX_OK
    assert mx.mx_block_mse(None, 1, None, None, 0, 64, A, None, None, 0, None) == mx.MX_OK


def test_alignment(lib):
    assert mx.mx_quantize(A + 2, mx.MX_BF16, 1, 32, 0, B, C, None) == mx.MX_ERR_ALIGN
    assert mx.mx_quantize(A, mx.MX_BF16, 1, 32, 0, B + 4, C, None) == mx.MX_ERR_ALIGN
    assert mx.mx_quantize(A, mx.MX_BF16, 1, 32, 0, B, C + 1, None) == mx.MX_ERR_ALIGN
    assert mx.mx_dequantize(B, C, 1, 32, 0, A + 8, None) == mx.MX_ERR_ALIGN
    assert mx.mx_fakequant(A, 0, 1, 32, 0, B + 8, None) == mx.MX_ERR_ALIGN
    assert mx.mx_block_mse(A, 0, B, C, 1, 32, A + (1 << 25) + 2, None, None, 0, None) == \
        mx.MX_ERR_ALIGN
    assert mx.mx_block_mse(A, 0, B, C, 1, 32, None, A + (1 << 25) + 4, W, 64, None) == \
        mx.MX_ERR_ALIGN


def test_aliasing(lib):
    # codes inside x
    assert mx.mx_quantize(A, mx.MX_F32, 4, 64, 0, A + 64, C, None) == mx.MX_ERR_ALIAS
    # scales inside codes
    assert mx.mx_quantize(A, mx.MX_F32, 4, 64, 0, B, B + 16, None) == mx.MX_ERR_ALIAS
    # dequant output over codes
    assert mx.mx_dequantize(B, C, 4, 64, 0, B - 256, None) == mx.MX_ERR_ALIAS
    # fake-quant: exact in-place is allowed (would launch, so not called
    # here); a shifted overlap is rejected
    assert mx.mx_fakequant(A, 0, 4, 64, 0, A + 16, None) == mx.MX_ERR_ALIAS
    assert mx.mx_block_mse(A, 0, B, C, 4, 64, A, None, None, 0, None) == mx.MX_ERR_ALIAS
    assert mx.mx_block_mse(A, 0, B, C, 4, 64, None, ctypes.c_void_p(B + 64), W, 64, None) == \
        mx.MX_ERR_ALIAS
    # workspace over the input
    assert mx.mx_block_mse(A, 0, B, C, 4, 64, None, W, A + 32, 64, None) == mx.MX_ERR_ALIAS
    # tensor_sums inside the workspace
    assert mx.mx_block_mse(A, 0, B, C, 4, 64, None, W + 8, W, 64, None) == mx.MX_ERR_ALIAS


def _expected_workspace(rows, k):
    """16 bytes per workgroup of the one-pass grid (512 items = 4096 elements
    each, at most 8192^2 of them), plus 16 per group of 8192 partial pairs
    when there is more than one group."""
    items = rows * k // 8
    grid = max(1, min(-(-items // 512), 8192 * 8192))
    groups = -(-grid // 8192) if grid > 8192 else 0
    return 16 * (grid + groups)


def test_workspace(lib):
    need = mx.mx_block_mse_workspace_size(8192, 4096)
    assert need == _expected_workspace(8192, 4096) == 16 * 8192
    for rows, k in ((0, 64), (1, 32), (16, 4096), (917504, 3072), (1 << 26, 4096)):
        assert mx.mx_block_mse_workspace_size(rows, k) == _expected_workspace(rows, k), (rows, k)
    # the 2.8e9-element weight set: 11 MB, 0.4 % of the bf16 input
    assert mx.mx_block_mse_workspace_size(917504, 3072) == 16 * (688128 + 84)
    # missing / small / misaligned workspace when the tensor sum is asked for
    assert mx.mx_block_mse(A, 1, B, C, 8192, 4096, None, W, None, 0, None) == mx.MX_ERR_WORKSPACE
    assert mx.mx_block_mse(A, 1, B, C, 8192, 4096, None, W, W + 64, need - 8, None) == \
        mx.MX_ERR_WORKSPACE
    assert mx.mx_block_mse(A, 1, B, C, 8192, 4096, None, W, W + 68, need, None) == \
        mx.MX_ERR_WORKSPACE


def test_block_mse_noalloc_validation(lib):
    """The entry point without a workspace: the same argument checks as
    mx_block_mse, all before any HIP call (the scratch address is looked up
    only after them)."""
    f = mx.mx_block_mse_noalloc
    for rows, k in ((-1, 32), (1, 0), (4, 48), (1 << 40, 1 << 30)):
        assert f(A, mx.MX_F32, B, C, rows, k, A + (64 << 30), None, None) == mx.MX_ERR_SHAPE
    assert f(A, 5, B, C, 1, 32, None, W, None) == mx.MX_ERR_DTYPE
    assert f(A, 0, B, C, 1, 32, None, None, None) == mx.MX_ERR_NULL      # no output asked
    assert f(None, 0, B, C, 1, 32, A + 64, None, None) == mx.MX_ERR_NULL
    assert f(A, 0, None, C, 1, 32, None, W, None) == mx.MX_ERR_NULL
    assert f(A + 2, 0, B, C, 1, 32, None, W, None) == mx.MX_ERR_ALIGN
    assert f(A, 0, B, C, 1, 32, A + (1 << 25) + 2, None, None) == mx.MX_ERR_ALIGN
    assert f(A, 0, B, C, 1, 32, None, W + 4, None) == mx.MX_ERR_ALIGN
    assert f(A, 0, B, C, 4, 64, A, None, None) == mx.MX_ERR_ALIAS        # block_mse over x
    assert f(A, 0, B, C, 4, 64, None, B + 64, None) == mx.MX_ERR_ALIAS   # sums over codes
    # empty tensor, block MSE only: nothing to write, nothing launched
    assert f(None, 1, None, None, 0, 64, A, None, None) == mx.MX_OK


def test_tensor_helpers_refuse_cpu_tensors(lib):
    import torch
    x = torch.zeros(2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mx.quantize(x)
    with pytest.raises(ValueError):
        mx.fakequant(x)
    u8 = torch.zeros(2, 32, dtype=torch.uint8)
    for f in (lambda: mx.dequantize(u8, u8[:, :2].contiguous()),
              lambda: mx.dequantize_mxfp8(torch.zeros(2, 64, dtype=torch.uint8), u8[:, :2].contiguous()),
              lambda: mx.dequantize_nvfp4(u8, u8[:, :4].contiguous(), u8[0, :1].contiguous()),
              lambda: mx.dequantize_mbs(torch.zeros(2, 64, dtype=torch.uint8), u8[:, :8].contiguous(),
                                        u8[:, :1].contiguous()),
              lambda: mx.quantize_mxfp8(x), lambda: mx.quantize_nvfp4(x),
              lambda: mx.quantize_mbs(torch.zeros(2, 128, dtype=torch.bfloat16)),
              lambda: mx.quantize_multi([x]), lambda: mx.fakequant_multi([x])):
        with pytest.raises(ValueError):
            f()


def test_missing_library_fails_loudly(tmp_path):
    saved = mx._lib
    try:
        mx._lib = None
        with pytest.raises(RuntimeError):
            mx.load_library(str(tmp_path / "nope.so"))
    finally:
        mx._lib = saved


def test_mxfp8_validation(lib):
    assert mx.mx_quantize_mxfp8(A, 3, 1, 32, B, C, None) == mx.MX_ERR_DTYPE
    assert mx.mx_quantize_mxfp8(A, 1, 1, 48, B, C, None) == mx.MX_ERR_SHAPE
    assert mx.mx_quantize_mxfp8(None, 1, 1, 32, B, C, None) == mx.MX_ERR_NULL
    assert mx.mx_quantize_mxfp8(A, 1, 1, 32, B + 8, C, None) == mx.MX_ERR_ALIGN
    assert mx.mx_quantize_mxfp8(A, 1, 0, 32, None, None, None) == mx.MX_OK
    # codes are one byte per element: [rows, k]; a codes buffer starting
    # inside x overlaps
    assert mx.mx_quantize_mxfp8(A, 1, 4, 64, A + 256, C, None) == mx.MX_ERR_ALIAS
    assert mx.mx_quantize_mxfp8(A, 1, 4, 64, B, B + 128, None) == mx.MX_ERR_ALIAS
    assert mx.mx_dequantize_mxfp8(B, C, 1, 32, 9, A, None) == mx.MX_ERR_DTYPE
    assert mx.mx_dequantize_mxfp8(B, C, 4, 64, 0, B + 16, None) == mx.MX_ERR_ALIAS
    assert mx.mx_dequantize_mxfp8(B, C, -1, 64, 0, A, None) == mx.MX_ERR_SHAPE
    assert mx.mx_fakequant_mxfp8(A, 0, 4, 64, A + 16, None) == mx.MX_ERR_ALIAS
    assert mx.mx_fakequant_mxfp8(A, 0, 1, 32, None, None) == mx.MX_ERR_NULL


def test_nvfp4_validation(lib):
    need = mx.mx_nvfp4_workspace_size(8192, 4096)
    assert 4 <= need <= 8192 * 4 and need % 4 == 0
    assert mx.mx_nvfp4_workspace_size(1, 24) == 0
    # one maximum per first-pass workgroup (1024 items each, at most 2048) and
    # the tensor-exponent word
    assert mx.mx_nvfp4_workspace_size(1, 16) == 2 * 4
    assert mx.mx_nvfp4_workspace_size(49153, 4112) == 2049 * 4
    assert mx.mx_quantize_nvfp4(A, 1, 1, 24, B, C, W, W + 64, 64, None) == mx.MX_ERR_SHAPE
    assert mx.mx_quantize_nvfp4(A, 1, 0, 16, None, None, None, None, 0, None) == mx.MX_OK
    assert mx.mx_quantize_nvfp4(A, 1, 1, 16, B, C, None, W + 64, 64, None) == mx.MX_ERR_NULL
    assert mx.mx_quantize_nvfp4(A, 1, 1, 16, B, C, W, None, 0, None) == mx.MX_ERR_WORKSPACE
    assert mx.mx_quantize_nvfp4(A, 1, 1, 16, B, C, W, W + 66, 64, None) == mx.MX_ERR_WORKSPACE
    assert mx.mx_quantize_nvfp4(A, 1, 4, 64, B, C, A + 3, W + 64, 64, None) == mx.MX_ERR_ALIAS
    assert mx.mx_quantize_nvfp4(A, 1, 4, 64, B, B + 64, W, W + 64, 64, None) == mx.MX_ERR_ALIAS
    assert mx.mx_quantize_nvfp4(A, 4, 1, 16, B, C, W, W + 64, 64, None) == mx.MX_ERR_DTYPE
    assert mx.mx_dequantize_nvfp4(B, C, W, 1, 16, 0, None, None) == mx.MX_ERR_NULL
    assert mx.mx_dequantize_nvfp4(B, C, W, 4, 64, 0, B + 32, None) == mx.MX_ERR_ALIAS
    assert mx.mx_dequantize_nvfp4(B, C, W, 1, 16, 0, A + 8, None) == mx.MX_ERR_ALIGN


def test_mbs_validation(lib):
    # k must be a multiple of the 128-element macro block
    assert mx.mx_quantize_mbs(A, 1, 1, 64, B, C, W, None) == mx.MX_ERR_SHAPE
    assert mx.mx_dequantize_mbs(B, C, W, 1, 96, 1, A, None) == mx.MX_ERR_SHAPE
    assert mx.mx_quantize_mbs(A, 1, -1, 128, B, C, W, None) == mx.MX_ERR_SHAPE
    assert mx.mx_quantize_mbs(A, 2, 1, 128, B, C, W, None) == mx.MX_ERR_DTYPE
    assert mx.mx_dequantize_mbs(B, C, W, 1, 128, 7, A, None) == mx.MX_ERR_DTYPE
    assert mx.mx_quantize_mbs(A, 1, 0, 128, None, None, None, None) == mx.MX_OK
    assert mx.mx_dequantize_mbs(None, None, None, 0, 128, 0, None, None) == mx.MX_OK
    assert mx.mx_quantize_mbs(A, 1, 1, 128, B, C, None, None) == mx.MX_ERR_NULL
    assert mx.mx_dequantize_mbs(B, None, W, 1, 128, 0, A, None) == mx.MX_ERR_NULL
    for bad in ((A + 8, B, C, W), (A, B + 4, C, W), (A, B, C + 1, W), (A, B, C, W + 2)):
        assert mx.mx_quantize_mbs(bad[0], 1, 1, 128, *bad[1:], None) == mx.MX_ERR_ALIGN
    assert mx.mx_dequantize_mbs(B, C, W, 1, 128, 0, A + 4, None) == mx.MX_ERR_ALIGN
    # codes [rows, k/2], sub-scales [rows, k/16], macro bytes [rows, k/128]
    assert mx.mx_quantize_mbs(A, 1, 4, 256, A + 1024, C, W, None) == mx.MX_ERR_ALIAS
    assert mx.mx_quantize_mbs(A, 1, 4, 256, B, B + 496, W, None) == mx.MX_ERR_ALIAS
    assert mx.mx_quantize_mbs(A, 1, 4, 256, B, C, C + 48, None) == mx.MX_ERR_ALIAS
    assert mx.mx_quantize_mbs(A, 1, 4, 256, B, C, B + 16, None) == mx.MX_ERR_ALIAS
    assert mx.mx_dequantize_mbs(B, C, W, 4, 256, 0, B + 256, None) == mx.MX_ERR_ALIAS
    assert mx.mx_dequantize_mbs(B, C, W, 4, 256, 1, W - 16, None) == mx.MX_ERR_ALIAS


def test_multi_validation(lib):
    T = mx.MxTensor
    arr = (T * 4)()
    arr[0] = T(A, None, B, C, 4, 64)
    arr[1] = T(A + 4096, None, B + 1024, C + 1024, 4, 48)  # k not a multiple of 32
    assert mx.mx_quantize_multi(arr, 2, 1, 0, None) == mx.MX_ERR_SHAPE
    assert mx.mx_last_error_detail() == "tensor 1: shape"
    assert mx.mx_quantize_multi(arr, 0, 1, 0, None) == mx.MX_OK
    assert mx.mx_quantize_multi(arr, -1, 1, 0, None) == mx.MX_ERR_SHAPE
    assert mx.mx_quantize_multi(None, 1, 1, 0, None) == mx.MX_ERR_NULL
    assert mx.mx_quantize_multi(arr, 1, 5, 0, None) == mx.MX_ERR_DTYPE
    assert mx.mx_quantize_multi(arr, 1, 1, 4, None) == mx.MX_ERR_MODE
    assert mx.mx_fakequant_multi(arr, 1, 1, 0, None) == mx.MX_ERR_NULL  # y missing
    arr[1] = T(A + 4096, None, B + 1024, C + 1028, 4, 64)
    assert mx.mx_quantize_multi(arr, 2, 1, 0, None) == mx.MX_ERR_ALIGN
    assert mx.mx_last_error_detail() == "tensor 1: alignment"
    # tensor 1's codes overlap tensor 0's codes
    arr[1] = T(A + 4096, None, B + 64, C + 1024, 4, 64)
    assert mx.mx_quantize_multi(arr, 2, 1, 0, None) == mx.MX_ERR_ALIAS
    # tensor 1's scales overlap tensor 0's input
    arr[1] = T(A + 4096, None, B + 1024, A + 16, 4, 64)
    assert mx.mx_quantize_multi(arr, 2, 1, 0, None) == mx.MX_ERR_ALIAS
    # in-place fake-quant of tensor 0 while tensor 1 reads inside it
    arr[0] = T(A, A, None, None, 4, 64)
    arr[1] = T(A + 256, B, None, None, 4, 64)
    assert mx.mx_fakequant_multi(arr, 2, 0, 0, None) == mx.MX_ERR_ALIAS
    # y partially overlapping its own x
    arr[0] = T(A, A + 16, None, None, 4, 64)
    assert mx.mx_fakequant_multi(arr, 1, 0, 0, None) == mx.MX_ERR_ALIAS
    # empty tensors only: nothing to launch
    arr[0] = T(None, None, None, None, 0, 64)
    arr[1] = T(None, None, None, None, 0, 32)
    assert mx.mx_quantize_multi(arr, 2, 1, 0, None) == mx.MX_OK
    assert mx.mx_fakequant_multi(arr, 2, 1, 3, None) == mx.MX_OK


def test_multi_helpers_refuse_bad_lists(lib):
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        mx.quantize_multi([torch.zeros(4, 32)])  # CPU tensor
    with pytest.raises(ValueError):
        mx.fakequant_multi([], mode="nope")
    assert mx.quantize_multi([]) == [] and mx.fakequant_multi([]) == []


def _plan(lib, nitems, tile, per_launch=60):
    f = lib.mxi_multi_plan
    f.argtypes = [ctypes.POINTER(ctypes.c_int64), ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                  ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int),
                  ctypes.POINTER(ctypes.c_int64)]
    f.restype = ctypes.c_int
    n = len(nitems)
    items = (ctypes.c_int64 * max(1, n))(*nitems)
    order, first = (ctypes.c_int * (n + 1))(), (ctypes.c_int * (n + 1))()
    gx = (ctypes.c_int64 * (n + 1))()
    launches = f(items, n, tile, per_launch, order, first, gx)
    if launches < 0:
        return None
    return ([list(order[first[l]:first[l + 1]]) for l in range(launches)],
            [gx[l] for l in range(launches)])


def _check_plan(nitems, tile, per_launch, plan):
    launches, gxs = plan
    tiles = [-(-v // tile) for v in nitems]
    seen = [i for group in launches for i in group]
    # every non-empty tensor exactly once, empty ones never
    assert sorted(seen) == [i for i, v in enumerate(nitems) if v > 0]
    # largest first overall, ties in the caller's order (a stable sort)
    assert seen == sorted(seen, key=lambda i: (-nitems[i], i))
    for group, gx in zip(launches, gxs):
        assert 1 <= len(group) <= per_launch
        assert gx == tiles[group[0]]  # the grid covers the launch's largest tensor
        # at most 1/8 of the launch's workgroups idle
        assert all(8 * tiles[i] >= 7 * gx for i in group)
    # a launch ends only at the cap or where the next tensor is too small for it
    for group, gx, nxt in zip(launches, gxs, launches[1:]):
        assert len(group) == per_launch or 8 * tiles[nxt[0]] < 7 * gx


def test_multi_launch_plan(lib):
    """The host plan of mx_quantize_multi / mx_fakequant_multi: launches of
    similar-sized tensors (2-D grids, no per-workgroup lookup), on random
    lists with empty, equal and widely different sizes, past 60 tensors."""
    import numpy as np
    rng = np.random.default_rng(5)
    llama = [o * i // 8 for _ in range(28) for o, i in
             ((3072, 3072), (1024, 3072), (1024, 3072), (3072, 3072), (8192, 3072), (8192, 3072),
              (3072, 8192))]
    plan = _plan(lib, llama, 256)
    _check_plan(llama, 256, 60, plan)
    assert [len(g) for g in plan[0]] == [60, 24, 56, 56]  # 84 large, 56 q/o, 56 k/v
    cases = [[], [0, 0], [4], [5] * 130, list(rng.integers(0, 10 ** 6, 200)),
             list(rng.choice([0, 12, 13, 14, 15, 16, 4096, 4095, 3585, 3584], 150)),
             list(rng.integers(0, 3, 70))]
    for nitems in cases:
        for tile, per in ((256, 60), (512, 60), (1024, 7), (128, 1)):
            plan = _plan(lib, [int(v) for v in nitems], tile, per)
            _check_plan([int(v) for v in nitems], tile, per, plan)
    # a tensor with more tiles than one grid dimension takes: refused whole
    assert _plan(lib, [2 ** 31 * 256 + 256, 10], 256) is None
