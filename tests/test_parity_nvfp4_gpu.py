"""GPU parity of the NVFP4 comparator kernels against the CPU oracle:
codes, E4M3 block scales, the tensor factor byte and decoded values
bit-exact. Inputs from workloads/, expected values from oracle/ only."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import microscaling_fp4_block_mx_amd as mx
from test_parity_gpu import assert_same_bits, host_view, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()
    oracle.build(force=not os.path.exists(os.path.join(os.path.dirname(oracle.__file__),
                                                       "libmxref.so")))
    yield
    torch.cuda.synchronize()


def check_nv(x: torch.Tensor, label: str):
    xh = host_view(x)
    say(f"{label} nvfp4 {tuple(x.shape)} {x.dtype}")
    c, b, t = mx.quantize_nvfp4(x.cuda())
    wc, wb, wt = oracle.quantize_nvfp4(xh)
    assert int(t.item()) == wt, f"{label} tensor factor byte {int(t.item())} != {wt}"
    assert_same_bits(b, wb, f"{label} nvfp4 block scales")
    assert_same_bits(c, wc, f"{label} nvfp4 codes")
    for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        assert_same_bits(mx.dequantize_nvfp4(c, b, t, dt), oracle.dequantize_nvfp4(wc, wb, wt, name),
                         f"{label} nvfp4 dequant {name}")
    # fused fake-quant: the oracle's quantize then dequantize, in x's dtype
    name = "bf16" if x.dtype == torch.bfloat16 else "f32"
    assert_same_bits(mx.fakequant_nvfp4(x.cuda()), oracle.dequantize_nvfp4(wc, wb, wt, name),
                     f"{label} nvfp4 fake-quant")


def test_nvfp4_golden_blocks():
    x = np.zeros((1, 32), np.float32)
    x[0, :6] = [6, 3, 1.5, 0.5, -2, 4]
    x[0, 16] = 5
    check_nv(torch.from_numpy(x), "golden-1")
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 7
    x[0, 16] = 3.1875
    check_nv(torch.from_numpy(x), "golden-2")


@pytest.mark.parametrize("rows,k,scale", [(1, 16, 1.0), (3, 48, 1e-3), (257, 160, 30.0),
                                          (1000, 4096, 0.02), (4099, 64, 1e5), (7, 16 * 257, 1e-30)])
def test_nvfp4_ragged_and_scales(rows, k, scale):
    rng = np.random.default_rng(rows * 13 + k)
    x = rng.standard_t(3, (rows, k)) * np.exp(rng.normal(0, 2, (rows, k // 16))).repeat(16, 1) * scale
    x.reshape(-1, 16)[rng.random(rows * k // 16) < 0.03] = 0
    xt = torch.from_numpy(x.astype(np.float32))
    check_nv(xt, f"ragged-f32 {rows}x{k}")
    check_nv(xt.to(torch.bfloat16), f"ragged-bf16 {rows}x{k}")


def test_nvfp4_special_tensors():
    x = np.zeros((4, 64), np.float32)
    check_nv(torch.from_numpy(x), "all-zero")
    sz = np.zeros((3, 32), np.float32)
    sz[0, [0, 2, 5]] = -0.0          # signed zeros in an all-zero block
    sz[1, :] = -0.0
    sz[2, :] = np.linspace(-1, 1, 32)
    sz[2, [3, 17]] = -0.0            # and beside nonzero values
    check_nv(torch.from_numpy(sz), "signed zeros")
    check_nv(torch.from_numpy(sz).to(torch.bfloat16), "signed zeros")
    x[1, 5] = np.nan
    x[2, 40] = -np.inf
    x[3, :] = np.linspace(-3, 3, 64)
    check_nv(torch.from_numpy(x), "nonfinite blocks")
    big = np.full((2, 32), np.finfo(np.float32).max, np.float32)
    big[1] *= -0.37
    check_nv(torch.from_numpy(big), "near fp32 max")
    tiny = (np.random.default_rng(75).standard_normal((8, 64)) * 1e-42).astype(np.float32)
    check_nv(torch.from_numpy(tiny), "subnormal tensor")


def test_nvfp4_activations_full():
    check_nv(workloads.bf16_student_t_outlier_channels(2), "student-t 8192x4096")


def test_nvfp4_versus_mxfp4_qsnr():
    """The pages' comparison, on N(0, 0.02) weights and on the activations:
    NVFP4's E4M3 block-16 scale gives a higher QSNR than MXFP4 (OCP)."""
    for name, x in (("weights", workloads.bf16_normal(76, (4096, 4096))),
                    ("activations", workloads.bf16_student_t_outlier_channels(2))):
        xd = x.cuda()
        xf = xd.float()
        c, b, t = mx.quantize_nvfp4(xd)
        ynv = mx.dequantize_nvfp4(c, b, t, torch.float32)
        ymx = mx.fakequant(xd).float()
        e = float((xf.double() ** 2).sum())
        q_nv = 10 * np.log10(e / float(((xf - ynv).double() ** 2).sum()))
        q_mx = 10 * np.log10(e / float(((xf - ymx).double() ** 2).sum()))
        say(f"QSNR {name}: nvfp4 {q_nv:.3f} dB, mxfp4-ocp {q_mx:.3f} dB")
        assert q_nv > q_mx


def test_nvfp4_fakequant_in_place():
    x = workloads.bf16_student_t_outlier_channels(31, shape=(512, 4096)).cuda()
    want = mx.fakequant_nvfp4(x)
    y = x.clone()
    got = mx.fakequant_nvfp4(y, out=y)
    assert got.data_ptr() == y.data_ptr()
    assert torch.equal(want.view(torch.int16), got.view(torch.int16))


def test_nvfp4_large_tiling():
    """The multi-GB path (past 2.0e8 elements the tensor exponent is reduced
    once and the block pass runs one tile per workgroup: quantize two items
    per 128 threads, fake-quant one per 256), on a bf16 tensor whose last
    tile is partial in both tilings (49153 x 4112: 514 items per row), whole
    against the oracle; fake-quant also in place."""
    x = workloads.bf16_laplace_sparse_outliers(9, shape=(49153, 4112))
    assert x.numel() // 8 >= 3 << 23 and (x.numel() // 8) % 256 != 0
    check_nv(x, "large-tiling")
    xd = x.cuda()
    want = mx.fakequant_nvfp4(xd)
    got = mx.fakequant_nvfp4(xd, out=xd)
    assert got.data_ptr() == xd.data_ptr()
    assert torch.equal(want.view(torch.int16), got.view(torch.int16)), "large in-place fake-quant"
