"""GPU parity of the MBS-Static kernels against the CPU oracle: codes,
sub-block E8M0 bytes, macro mantissa bytes and decoded values bit-exact.
Inputs from workloads/, expected values from oracle/ only."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads
import microscaling_fp4_block_mx_amd as mx
from conftest import golden_rows
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


def check_mbs(x: torch.Tensor, label: str):
    xh = host_view(x)
    say(f"{label} mbs {tuple(x.shape)} {x.dtype}")
    c, s, m = mx.quantize_mbs(x.cuda())
    wc, ws, wm = oracle.quantize_mbs(xh)
    assert_same_bits(m, wm, f"{label} mbs macro mantissas")
    assert_same_bits(s, ws, f"{label} mbs sub-block scales")
    assert_same_bits(c, wc, f"{label} mbs codes")
    for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        assert_same_bits(mx.dequantize_mbs(c, s, m, dt), oracle.dequantize_mbs(wc, ws, wm, name),
                         f"{label} mbs dequant {name}")
    # fused fake-quant: the oracle's quantize then dequantize, in x's dtype
    name = "bf16" if x.dtype == torch.bfloat16 else "f32"
    assert_same_bits(mx.fakequant_mbs(x.cuda()), oracle.dequantize_mbs(wc, ws, wm, name),
                     f"{label} mbs fake-quant")


def test_mbs_golden_macro_block():
    # the hand-worked macro block of tests/golden/mbs_static_blocks.txt
    x = np.zeros((1, 128), np.float32)
    x[0, 0], x[0, 20], x[0, 40] = 7.5, 1.0, -0.3
    check_mbs(torch.from_numpy(x), "golden")
    head, dec = golden_rows("mbs_static_blocks.txt")[0].split("|")
    f = [int(v) for v in head.split()]
    c, s, m = mx.quantize_mbs(torch.from_numpy(x).cuda())
    assert int(m[0, 0]) == f[0] and s[0].cpu().tolist() == f[1:]
    y = mx.dequantize_mbs(c, s, m, torch.float32).cpu().numpy()
    assert y[0, [0, 20, 40]].tolist() == [float(v) for v in dec.split()]


@pytest.mark.parametrize("rows,k,scale", [(1, 128, 1.0), (3, 384, 1e-3), (257, 1152, 30.0),
                                          (1000, 4096, 0.02), (4099, 128, 1e5),
                                          (7, 128 * 33, 1e-30), (5, 256, 1e30)])
def test_mbs_ragged_and_scales(rows, k, scale):
    rng = np.random.default_rng(rows * 17 + k)
    x = rng.standard_t(3, (rows, k)) * np.exp(rng.normal(0, 2, (rows, k // 16))).repeat(16, 1) * scale
    x.reshape(-1, 16)[rng.random(rows * k // 16) < 0.03] = 0
    xt = torch.from_numpy(x.astype(np.float32))
    check_mbs(xt, f"ragged-f32 {rows}x{k}")
    check_mbs(xt.to(torch.bfloat16), f"ragged-bf16 {rows}x{k}")


def test_mbs_exhaustive_bf16_magnitudes():
    """Every finite bf16 magnitude (both signs) below 8 * 2^(s-127) beside an
    anchor 4 * 2^(s-127), for scale bytes across the range; the blocks are
    regrouped into 128-element macro blocks, so the macro factors vary."""
    b = workloads.exhaustive_bf16_blocks((0, 1, 2, 60, 125, 126, 127, 128, 200, 252))
    flat = b.reshape(-1)
    pad = (-flat.size) % 128
    flat = np.concatenate([flat, np.zeros(pad, np.uint16)]).reshape(-1, 128)
    xb = workloads.from_bf16_bits(flat)
    check_mbs(xb, "exhaustive-bf16")
    check_mbs(xb.float(), "exhaustive-as-f32")


def test_mbs_special_values():
    x = np.zeros((6, 128), np.float32)
    check_mbs(torch.from_numpy(x[:1]), "all-zero")
    x[1, 5] = np.nan
    x[1, 70] = 3.0
    x[2, 3] = -np.inf
    x[2, 9] = 5.0
    x[2].view(np.uint32)[20] = 0xFFC00000  # -NaN in another sub-block
    x[2, 33] = -0.0
    x[3] = np.linspace(-3, 3, 128)
    x[4, :16] = np.finfo(np.float32).max
    x[4, 16:32] = -np.finfo(np.float32).max * 0.37
    x[5].view(np.uint32)[0] = 3           # a_M / 6 underflows: factor 1
    x[5].view(np.uint32)[1] = 0x80000001
    check_mbs(torch.from_numpy(x), "special f32")
    check_mbs(torch.from_numpy(x).to(torch.bfloat16), "special bf16")
    tiny = (np.random.default_rng(77).standard_normal((8, 256)) * 1e-42).astype(np.float32)
    check_mbs(torch.from_numpy(tiny), "subnormal tensor")
    # macro maxima that round the 8-bit mantissa up to a carry (capped at 255)
    top = np.zeros((4, 128), np.float32)
    top[:, 0] = 6 * (1 + np.array([255.25, 255.5, 255.75, 127.5]) / 256)
    top[:, 1:] = np.random.default_rng(78).uniform(-1, 1, (4, 127))
    check_mbs(torch.from_numpy(top), "mantissa carry")


def test_mbs_activations_full():
    check_mbs(workloads.bf16_student_t_outlier_channels(2), "student-t 8192x4096")


def test_mbs_versus_mxfp4_qsnr():
    """MBS-Static's 16-element sub-blocks and macro factor recover accuracy
    that a block-32 power-of-two scale loses ("Unveiling the Potential of
    Quantization with MXFP4", MBS section): higher QSNR than MXFP4 (OCP). On
    the outlier-channel activations it lands within 1 dB of NVFP4, the gap
    the page's contributions section reports for its enhanced MXFP4."""
    for name, x in (("weights", workloads.bf16_normal(76, (4096, 4096))),
                    ("activations", workloads.bf16_student_t_outlier_channels(2))):
        xd = x.cuda()
        xf = xd.float()
        c, s, m = mx.quantize_mbs(xd)
        ymbs = mx.dequantize_mbs(c, s, m, torch.float32)
        ymx = mx.fakequant(xd).float()
        cn, bn, tn = mx.quantize_nvfp4(xd)
        ynv = mx.dequantize_nvfp4(cn, bn, tn, torch.float32)
        e = float((xf.double() ** 2).sum())
        q = {k: 10 * np.log10(e / float(((xf - y).double() ** 2).sum()))
             for k, y in (("mbs", ymbs), ("mx", ymx), ("nv", ynv))}
        say(f"QSNR {name}: mbs-static {q['mbs']:.3f} dB, mxfp4-ocp {q['mx']:.3f} dB, "
            f"nvfp4 {q['nv']:.3f} dB")
        assert q["mbs"] > q["mx"]
        if name == "activations":
            assert q["nv"] - q["mbs"] < 1.0


def test_mbs_fakequant_in_place():
    x = workloads.bf16_student_t_outlier_channels(32, shape=(512, 4096)).cuda()
    want = mx.fakequant_mbs(x)
    y = x.clone()
    got = mx.fakequant_mbs(y, out=y)
    assert got.data_ptr() == y.data_ptr()
    assert torch.equal(want.view(torch.int16), got.view(torch.int16))
