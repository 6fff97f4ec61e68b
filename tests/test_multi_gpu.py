"""GPU parity of the many-tensors-in-one-call entry points: every tensor's
codes, scales and fake-quant output equal the oracle's (and the single-
tensor calls'), across ragged shapes, empty tensors, more tensors than one
launch takes, every scale mode and both dtypes; plus the 196 Llama-3.2-3B-
shaped weights as separate tensors. Expected values from oracle/ only."""
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


def ragged_list(seed: int, n: int, dtype):
    rng = np.random.default_rng(seed)
    xs = []
    for i in range(n):
        rows = int(rng.choice([0, 1, 2, 3, 7, 64, 257, 1000]))
        k = 32 * int(rng.choice([1, 2, 3, 5, 33, 96, 128]))
        x = rng.standard_t(3, (rows, k)) * np.exp(rng.normal(0, 2, (rows, k // 32))).repeat(32, 1)
        xs.append(torch.from_numpy(x.astype(np.float32)).to(dtype))
    return xs


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("mode", mx.MODES)
def test_multi_ragged_vs_oracle(dtype, mode):
    xs = ragged_list(11 + mx.MODES.index(mode), 120, dtype)  # > 60 tensors of many sizes
    xd = [x.cuda() for x in xs]
    say(f"multi {mode} {dtype}: {len(xs)} tensors")
    qs = mx.quantize_multi(xd, mode)
    fs = mx.fakequant_multi(xd, mode)
    name = "bf16" if dtype == torch.bfloat16 else "f32"
    for i, (x, (c, s), f) in enumerate(zip(xs, qs, fs)):
        xh = host_view(x)
        wc, ws = oracle.quantize(xh, mode)
        assert_same_bits(c, wc, f"tensor {i} codes {mode}")
        assert_same_bits(s, ws, f"tensor {i} scales {mode}")
        assert_same_bits(f, oracle.fakequant(xh, mode), f"tensor {i} fake-quant {mode}")


def test_multi_in_place_and_leading_dims():
    xs = [workloads.bf16_student_t_outlier_channels(20 + i, shape=(2, 3, 64 * (i + 1))).cuda()
          for i in range(5)]
    want = [mx.fakequant(x) for x in xs]
    got = mx.fakequant_multi(xs, out=xs)  # in place
    for w, g, x in zip(want, got, xs):
        assert g.data_ptr() == x.data_ptr()
        assert torch.equal(w.view(torch.int16), g.view(torch.int16))


@pytest.mark.parametrize("mode", ["ocp", "oas", "oas_nf"])
def test_multi_large_tiling_unequal_sizes(mode):
    """A call past the large-tensor size (the tiling of multi-GB weight
    sets) whose tensors differ in size by less than 1/8, so they share a
    launch and the smaller ones leave tiles of the 2-D grid idle; plus small
    and empty tensors in their own launches. Bit-equal to one call per
    tensor, in both directions of the size order."""
    # 2.2e8 elements in all (past 2^24 * 12 = 2.0e8); the seven large ones
    # are within 7/8 of the largest
    shapes = [(8192, 4096), (7680, 4096), (8000, 4096), (7424, 4096), (7200, 4096),
              (0, 4096), (3, 96), (8192, 4096), (7900, 4096), (1, 32)]
    xs = [workloads.bf16_student_t_outlier_channels(40 + i, shape=sh).cuda() if sh[0] else
          torch.empty(sh, dtype=torch.bfloat16, device="cuda") for i, sh in enumerate(shapes)]
    for order in (xs, xs[::-1]):
        say(f"multi large {mode}: {[tuple(x.shape) for x in order]}")
        qs = mx.quantize_multi(order, mode)
        fs = mx.fakequant_multi(order, mode)
        for i, (x, (c, s), f) in enumerate(zip(order, qs, fs)):
            c1, s1 = mx.quantize(x, mode)
            assert torch.equal(c, c1) and torch.equal(s, s1), f"tensor {i} {tuple(x.shape)}"
            assert torch.equal(f.view(torch.int16), mx.fakequant(x, mode).view(torch.int16)), \
                f"tensor {i} {tuple(x.shape)} fake-quant"


def test_multi_llama32_3b_separate_weights():
    """The 196 weights as separate tensors, one call: bit-equal to one
    quantize call per matrix (4 launches instead of 196)."""
    say("generating llama weights on device")
    ms = [workloads.llama32_3b_matrix(layer, which, "cuda")
          for layer in range(workloads.LLAMA32_3B_LAYERS)
          for which in range(len(workloads.LLAMA32_3B_LINEARS))]
    qs = mx.quantize_multi(ms)
    for i, (m, (c, s)) in enumerate(zip(ms, qs)):
        c1, s1 = mx.quantize(m)
        assert torch.equal(c, c1) and torch.equal(s, s1), f"matrix {i}"
    # and the oracle on sampled rows of a few of them
    rng = np.random.default_rng(77)
    for i in (0, 1, 4, 6, 195):
        rows = np.sort(rng.choice(ms[i].shape[0], 64, replace=False))
        idx = torch.from_numpy(rows).cuda()
        wc, ws = oracle.quantize(host_view(ms[i].index_select(0, idx)), "ocp")
        assert_same_bits(qs[i][0].index_select(0, idx), wc, f"matrix {i} codes (sampled rows)")
        assert_same_bits(qs[i][1].index_select(0, idx), ws, f"matrix {i} scales (sampled rows)")


def test_other_formats_past_2_31_elements():
    """MXFP8, NVFP4 and MBS-Static on one bf16 tensor of 2^31 + 2^20
    elements (64-bit indexing in every kernel), checked on sampled rows
    including the last ones."""
    rows, k = (1 << 31) // 4096 + 256, 4096
    say(f"big tensor [{rows}, {k}]")
    g = torch.Generator(device="cuda")
    g.manual_seed(91)
    x = torch.empty((rows, k), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, rows, 65536):
        r1 = min(rows, r0 + 65536)
        x[r0:r1] = (torch.randn((r1 - r0, k), generator=g, device="cuda") * 3).to(torch.bfloat16)
    # sampled rows: the first and last ones, random ones, and the row holding
    # the tensor's largest |x| (so the NVFP4 tensor factor of the sample is
    # the whole tensor's)
    top = int(torch.argmax(x.view(-1).abs()).item()) // k
    pick = np.unique(np.concatenate([np.arange(4), np.random.default_rng(92).choice(rows, 60, replace=False),
                                     np.arange(rows - 4, rows), [top]]))
    idx = torch.from_numpy(pick).cuda()
    xs = host_view(x.index_select(0, idx))
    say("mxfp8")
    c, s = mx.quantize_mxfp8(x)
    wc, ws = oracle.quantize_mxfp8(xs)
    assert_same_bits(c.index_select(0, idx), wc, "mxfp8 codes (sampled rows)")
    assert_same_bits(s.index_select(0, idx), ws, "mxfp8 scales (sampled rows)")
    del c, s
    say("mbs-static")
    c, s, m = mx.quantize_mbs(x)
    wc, ws, wm = oracle.quantize_mbs(xs)
    assert_same_bits(c.index_select(0, idx), wc, "mbs codes (sampled rows)")
    assert_same_bits(s.index_select(0, idx), ws, "mbs sub-scales (sampled rows)")
    assert_same_bits(m.index_select(0, idx), wm, "mbs macro bytes (sampled rows)")
    y = mx.dequantize_mbs(c, s, m, torch.bfloat16)
    assert_same_bits(y.index_select(0, idx), oracle.dequantize_mbs(wc, ws, wm, "bf16"),
                     "mbs dequant (sampled rows)")
    del c, s, m, y
    say("nvfp4")
    c, b, t = mx.quantize_nvfp4(x)
    wc, wb, wt = oracle.quantize_nvfp4(xs)
    assert int(t.item()) == wt, "nvfp4 tensor factor byte"
    assert_same_bits(c.index_select(0, idx), wc, "nvfp4 codes (sampled rows)")
    assert_same_bits(b.index_select(0, idx), wb, "nvfp4 block scales (sampled rows)")
    y = mx.dequantize_nvfp4(c, b, t, torch.bfloat16)
    assert_same_bits(y.index_select(0, idx), oracle.dequantize_nvfp4(wc, wb, wt, "bf16"),
                     "nvfp4 dequant (sampled rows)")
