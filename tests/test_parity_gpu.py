"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Bar: codes, scales, dequantized and fake-quantized values are bit-exact;
block MSE and tensor SSE agree to relative 1e-6 (the two sides sum in a
different order, both in fp64). Inputs come from the seeded generators in
workloads/; expected values come only from oracle/.
"""
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
import microscaling_fp4_block_mx_amd as mx

pytestmark = pytest.mark.gpu

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
MODES = ("ocp", "oas", "oas_bits", "oas_nf")


def say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()
    oracle.build(force=not os.path.exists(os.path.join(os.path.dirname(oracle.__file__),
                                                       "libmxref.so")))
    yield
    torch.cuda.synchronize()


def host_view(t: torch.Tensor) -> np.ndarray:
    """CPU numpy view for the oracle: float32 as is, bf16 as uint16 bits."""
    if t.dtype == torch.bfloat16:
        return workloads.to_bf16_bits(t)
    return t.detach().cpu().numpy()


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_same_bits(got: torch.Tensor, want: np.ndarray, what: str):
    g = bits(host_view(got))
    w = bits(want)
    assert g.shape == w.shape, what
    bad = np.flatnonzero(g.reshape(-1) != w.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} mismatches, first at flat {bad[:5]}: " \
        f"got {g.reshape(-1)[bad[:5]]} want {w.reshape(-1)[bad[:5]]}"


def check_all_ops(x: torch.Tensor, label: str, modes=MODES, mse=True):
    """Quantize/dequantize/fakequant(/block_mse) of a CPU tensor x on the GPU,
    each compared with the oracle."""
    xh = host_view(x)
    xd = x.cuda()
    for mode in modes:
        say(f"{label} quantize {mode} {tuple(x.shape)} {x.dtype}")
        c, s = mx.quantize(xd, mode)
        wc, ws = oracle.quantize(xh, mode, threads=THREADS)
        assert_same_bits(s, ws, f"{label} scales {mode}")
        assert_same_bits(c, wc, f"{label} codes {mode}")
        for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
            y = mx.dequantize(c, s, dt)
            assert_same_bits(y, oracle.dequantize(wc, ws, name, threads=THREADS),
                             f"{label} dequant {name} {mode}")
        y = mx.fakequant(xd, mode)
        assert_same_bits(y, oracle.fakequant(xh, mode, threads=THREADS),
                         f"{label} fakequant {mode}")
        if mse:
            bm, sums = mx.block_mse(xd, c, s)
            wbm, wsse, wssq = oracle.block_mse(xh, wc, ws, threads=THREADS, with_energy=True)
            g = bm.cpu().numpy()
            np.testing.assert_array_equal(np.isnan(g), np.isnan(wbm))
            ok = ~np.isnan(wbm)
            np.testing.assert_allclose(g[ok], wbm[ok], rtol=1e-6, atol=0)
            got, got_sq = sums.tolist()
            for a, b in ((got, wsse), (got_sq, wssq)):
                if np.isnan(b):
                    assert np.isnan(a)
                elif np.isinf(b):
                    assert a == b
                else:
                    assert abs(a - b) <= 1e-6 * abs(b), (a, b)


# ---- exhaustive and special inputs ----------------------------------------

def test_exhaustive_bf16_every_scale():
    """Every bf16 magnitude below 8*2^(s-127), both signs, at every scale
    byte s = 0..252 (17M elements)."""
    blocks = workloads.exhaustive_bf16_blocks(range(0, 253))
    x = workloads.from_bf16_bits(blocks)
    check_all_ops(x, "exhaustive-bf16", mse=False)


def test_exhaustive_bf16_fp32_widened():
    """Same values widened to fp32 (exact), through the fp32 kernels."""
    blocks = workloads.exhaustive_bf16_blocks(range(0, 253, 3))
    x = workloads.from_bf16_bits(blocks).float()
    check_all_ops(x, "exhaustive-f32", mse=False)


def test_special_blocks():
    x = torch.from_numpy(workloads.special_blocks_f32())
    check_all_ops(x, "special-f32")
    check_all_ops(x.to(torch.bfloat16), "special-bf16")


def test_fp32_subnormal_and_wide_range():
    rng = np.random.default_rng(21)
    rows = 512
    # magnitudes up to 4 * 2^125 (normal values times 2^e stay finite in fp32,
    # so the tensor sums below are finite and compared)
    e = rng.integers(-149, 126, (rows, 1))
    x = np.clip(rng.standard_normal((rows, 64)), -3.9, 3.9) * np.ldexp(1.0, e)
    x = x.astype(np.float32)
    assert np.isfinite(x).all() and np.isfinite((x.astype(np.float64) ** 2).sum())
    x[:64] = np.ldexp(rng.integers(-8, 9, (64, 64)).astype(np.float64), -149).astype(np.float32)
    check_all_ops(torch.from_numpy(x), "wide-f32")


def test_oas_tie_prone_blocks():
    """Blocks where the overflow-aware choices go both ways (and tie), so
    both the evaluated and the bounded-out branch of the kernel run."""
    x = workloads.oas_tie_prone_blocks(26, 200_000)
    _, s0 = oracle.quantize(x, "ocp", threads=THREADS)
    for mode in ("oas", "oas_nf"):
        _, ws = oracle.quantize(x, mode, threads=THREADS)
        assert (ws != s0).sum() > 1000  # the other candidate wins in many blocks
    modes = ("oas", "oas_bits", "oas_nf")
    check_all_ops(torch.from_numpy(x), "oas-tie-prone-f32", modes=modes)
    check_all_ops(torch.from_numpy(x).to(torch.bfloat16), "oas-tie-prone-bf16", modes=modes)


def test_overflow_aware_at_the_ends_of_the_byte_range():
    """Tie-prone blocks moved so that their OCP byte (and, for half of them,
    their no-overflow byte) is 1, 2, 251 or 252: the smallest and largest
    bytes that have a smaller candidate, where the blocks' small elements are
    fp32 subnormals or the top ones near fp32's largest values. Both
    outcomes of each choice occur; the hand-worked blocks (4 with sixteen or
    seventeen 0.75; 3.25 with five 0.75) ride along at each byte."""
    x = workloads.oas_tie_prone_blocks(28, 4000).astype(np.float64)
    amax = np.abs(x).max(1, keepdims=True)
    x = x / 2.0 ** np.floor(np.log2(amax))          # block maximum in [1, 2)
    rng = np.random.default_rng(29)
    s = rng.choice([1, 2, 251, 252], (x.shape[0], 1))
    # normalized maximum in [4, 8) for the OCP byte s (half the blocks), or
    # in (3, 6] for the no-overflow byte s
    nf = rng.random((x.shape[0], 1)) < 0.5
    x = x * np.where(nf, 3.0, 4.0)
    x = (x * 2.0 ** (s - 127)).astype(np.float32)
    worked = []
    for b in (1, 2, 251, 252):
        for n in (16, 17):
            w = np.zeros(32)
            w[0], w[1:1 + n] = 4.0, 0.75
            worked.append(w * 2.0 ** (b - 127))
        w = np.zeros(32)
        w[3], w[10:15] = 3.25, 0.75
        worked.append(w * 2.0 ** (b - 127))
    x = np.concatenate([x, np.array(worked, np.float32)])
    assert np.isfinite(x).all()
    _, s0 = oracle.quantize(x, "ocp", threads=THREADS)
    assert set(np.unique(s0)) >= {1, 2, 251, 252}
    for mode in ("oas", "oas_nf"):
        _, ws = oracle.quantize(x, mode, threads=THREADS)
        assert (ws.astype(int) < s0.astype(int)).any() and (ws == s0).any(), mode
    check_all_ops(torch.from_numpy(x), "byte-range-ends-f32")
    check_all_ops(torch.from_numpy(x).to(torch.bfloat16), "byte-range-ends-bf16")


def test_page_modes_near_scale_ceiling():
    """Block maxima near the largest finite values: the page modes cap the
    scale byte at 252 and never decode to Inf."""
    f = np.float32
    top = [np.finfo(np.float32).max, f(7.9) * f(2.0 ** 125), f(6.5) * f(2.0 ** 125),
           f(7.01) * f(2.0 ** 125), f(5.0) * f(2.0 ** 125), f(7.5) * f(2.0 ** -127),
           f(6.5) * f(2.0 ** -127)]
    rng = np.random.default_rng(27)
    x = (rng.standard_normal((len(top), 64)) * 0.1).astype(np.float32)
    for i, t in enumerate(top):
        x[i] *= t
        x[i, 3] = t
    check_all_ops(torch.from_numpy(x), "near-ceiling-f32")
    y = mx.fakequant(torch.from_numpy(x).cuda(), "oas_bits")
    assert torch.isfinite(y).all()


def test_dequantize_every_scale_byte():
    """Random codes at every scale byte 0..255 (253/254 overflow, 255 NaN)."""
    rng = np.random.default_rng(22)
    codes = rng.integers(0, 256, (256, 64), dtype=np.uint8)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 4, 1)
    cd, sd = torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda()
    for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        y = mx.dequantize(cd, sd, dt)
        assert_same_bits(y, oracle.dequantize(codes, scales, name), f"dequant-all-s {name}")
    # block error against user-made scales, including Inf / NaN reconstructions
    x = torch.from_numpy(rng.standard_normal((256, 128)).astype(np.float32))
    bm, _ = mx.block_mse(x.cuda(), cd, sd)
    wbm, _ = oracle.block_mse(x.numpy(), codes, scales)
    g = bm.cpu().numpy()
    np.testing.assert_array_equal(np.isnan(g), np.isnan(wbm))
    np.testing.assert_array_equal(np.isinf(g), np.isinf(wbm))
    ok = np.isfinite(wbm)
    np.testing.assert_allclose(g[ok], wbm[ok], rtol=1e-6)


@pytest.mark.parametrize("rows,k", [(1, 32), (3, 96), (5, 4096), (257, 160), (1000, 8192),
                                    (33, 1056), (4099, 64), (7, 32 * 257)])
def test_ragged_shapes(rows, k):
    """Sizes that leave partial tiles and ragged tails, mixed block scales,
    zero blocks and outliers."""
    rng = np.random.default_rng(rows * 100003 + k)
    x = rng.laplace(0, 1, (rows, k)) * np.exp(rng.normal(0, 3, (rows, k // 32))).repeat(32, 1)
    x[rng.random((rows, k)) < 0.002] *= 300
    x = x.astype(np.float32)
    x.reshape(-1, 32)[rng.random(rows * k // 32) < 0.05] = 0
    xt = torch.from_numpy(x)
    check_all_ops(xt, f"ragged-f32 {rows}x{k}")
    check_all_ops(xt.to(torch.bfloat16), f"ragged-bf16 {rows}x{k}")


def test_leading_dims_and_empty():
    x = workloads.bf16_normal(23, (3, 5, 2, 96), std=1.0)
    check_all_ops(x, "4d")
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    c, s = mx.quantize(e)
    assert c.shape == (0, 32) and s.shape == (0, 2)
    assert mx.fakequant(e).shape == (0, 64)
    _, sums = mx.block_mse(e, c, s)
    assert sums.tolist() == [0.0, 0.0]


def test_bad_arguments_raise_on_gpu():
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mx.quantize(x[:, :48].contiguous())
    with pytest.raises(ValueError):
        mx.quantize(x.t())
    y = torch.zeros(4 * 64 + 8, dtype=torch.bfloat16, device="cuda")[1:257].view(4, 64)
    with pytest.raises(ValueError):  # 2-byte offset: not 16-byte aligned
        mx.quantize(y)
    with pytest.raises(ValueError):
        mx.quantize(x, mode="nope")


def test_helpers_refuse_host_or_mismatched_tensors_before_launch():
    """A CPU, wrong-dtype, wrong-size or strided tensor handed to any helper
    is refused on the host, so no host pointer ever reaches a kernel."""
    x = torch.zeros(4, 128, dtype=torch.bfloat16, device="cuda")
    c, s = mx.quantize(x)
    cpu_c, cpu_s = c.cpu(), s.cpu()
    cases = [
        lambda: mx.quantize(x, codes=cpu_c),
        lambda: mx.quantize(x, scales=torch.empty(4, 4, dtype=torch.int32, device="cuda")),
        lambda: mx.quantize(x, codes=torch.empty(4, 63, dtype=torch.uint8, device="cuda")),
        lambda: mx.dequantize(c, cpu_s),
        lambda: mx.dequantize(c, s, out=torch.empty(4, 128, dtype=torch.bfloat16)),
        lambda: mx.dequantize(c, s, torch.float32, out=torch.empty(4, 128, dtype=torch.bfloat16,
                                                                   device="cuda")),
        lambda: mx.fakequant(x, out=torch.empty(4, 128, dtype=torch.bfloat16)),
        lambda: mx.fakequant(x, out=torch.empty(128, 4, dtype=torch.bfloat16, device="cuda").t()),
        lambda: mx.block_mse(x, cpu_c, s),
        lambda: mx.block_mse(x, c, s[:, :2].contiguous()),
        lambda: mx.quantize_mxfp8(x, codes=torch.empty(4, 64, dtype=torch.uint8, device="cuda")),
        lambda: mx.dequantize_mxfp8(torch.zeros(4, 128, dtype=torch.uint8, device="cuda"), cpu_s),
        lambda: mx.fakequant_mxfp8(x, out=torch.empty(4, 128, dtype=torch.bfloat16)),
        lambda: mx.dequantize_nvfp4(c, torch.zeros(4, 8, dtype=torch.uint8, device="cuda"),
                                    torch.zeros(1, dtype=torch.uint8)),
        lambda: mx.dequantize_nvfp4(c, torch.zeros(4, 8, dtype=torch.uint8),
                                    torch.zeros(1, dtype=torch.uint8, device="cuda")),
        lambda: mx.dequantize_mbs(c, torch.zeros(4, 8, dtype=torch.uint8, device="cuda"),
                                  torch.zeros(4, 1, dtype=torch.uint8)),
        lambda: mx.fakequant_multi([x], out=[torch.empty(4, 128, dtype=torch.bfloat16)]),
        lambda: mx.quantize_multi([x, x.float()]),
    ]
    for i, f in enumerate(cases):
        with pytest.raises(ValueError):
            f()
    torch.cuda.synchronize()


def test_fakequant_in_place():
    x = workloads.bf16_student_t_outlier_channels(seed=24, shape=(256, 4096)).cuda()
    want = mx.fakequant(x)
    mx.fakequant(x, out=x)
    assert torch.equal(x.view(torch.int16), want.view(torch.int16))


# ---- the workloads at full size -------------------------------------------

def test_fp32_1024x4096_normal_full():
    x = workloads.fp32_normal(1)
    check_all_ops(x, "fp32 1024x4096 N(0,1)")


def test_bf16_8192x4096_student_t_fakequant_full():
    x = workloads.bf16_student_t_outlier_channels(2)
    xh = host_view(x)
    xd = x.cuda()
    for mode in MODES:
        say(f"student-t fakequant {mode}")
        assert_same_bits(mx.fakequant(xd, mode), oracle.fakequant(xh, mode, threads=THREADS),
                         f"student-t fakequant {mode}")
    say("student-t quantize/dequant/mse")
    check_all_ops(x, "student-t", modes=("ocp",))
    # the error-driven modes' codes and scales over the whole tensor (OAS_NF
    # runs the two-lanes-per-block layout at this size)
    for mode in ("oas", "oas_nf"):
        say(f"student-t quantize {mode}")
        c, s = mx.quantize(xd, mode)
        wc, ws = oracle.quantize(xh, mode, threads=THREADS)
        assert_same_bits(s, ws, f"student-t scales {mode}")
        assert_same_bits(c, wc, f"student-t codes {mode}")


def test_large_tensor_tiling_every_mode():
    """One bf16 tensor just at the multi-GB tiling (2^24 * 12 items = 2.0e8
    elements: two items per 128 threads for quantize in every mode, one per
    64 threads for fake-quant, two per 64 for dequantize): every mode's codes, scales and
    fake-quant output, and the dequantized tensor, whole against the oracle;
    likewise MXFP8 and MBS-Static quantize, dequantize and fake-quant."""
    x = workloads.bf16_laplace_sparse_outliers(8, shape=(49152, 4096))
    assert x.numel() // 8 == 3 << 23
    xh = host_view(x)
    xd = x.cuda()
    for mode in MODES:
        say(f"large tiling {mode} {tuple(x.shape)}")
        c, s = mx.quantize(xd, mode)
        wc, ws = oracle.quantize(xh, mode, threads=THREADS)
        assert_same_bits(s, ws, f"large scales {mode}")
        assert_same_bits(c, wc, f"large codes {mode}")
        if mode == "ocp":
            assert_same_bits(mx.dequantize(c, s, torch.bfloat16),
                             oracle.dequantize(wc, ws, "bf16", threads=THREADS), "large dequant")
        del c, s
        assert_same_bits(mx.fakequant(xd, mode), oracle.fakequant(xh, mode, threads=THREADS),
                         f"large fakequant {mode}")
    # MXFP8 at its multi-GB tiling (quantize and fake-quant one item per 64
    # threads, dequantize two per 128)
    say("large tiling mxfp8")
    c, s = mx.quantize_mxfp8(xd)
    wc, ws = oracle.quantize_mxfp8(xh, threads=THREADS)
    assert_same_bits(s, ws, "large mxfp8 scales")
    assert_same_bits(c, wc, "large mxfp8 codes")
    assert_same_bits(mx.dequantize_mxfp8(c, s, torch.bfloat16),
                     oracle.dequantize_mxfp8(wc, ws, "bf16", threads=THREADS), "large mxfp8 dequant")
    del c, s
    assert_same_bits(mx.fakequant_mxfp8(xd), oracle.fakequant_mxfp8(xh, threads=THREADS),
                     "large mxfp8 fakequant")
    # and MBS-Static (quantize two items per 128 threads, fake-quant one per
    # 256; dequantize two per 64)
    say("large tiling mbs-static")
    c, s, m = mx.quantize_mbs(xd)
    wc, ws, wm = oracle.quantize_mbs(xh)
    assert_same_bits(m, wm, "large mbs macro bytes")
    assert_same_bits(s, ws, "large mbs sub-scales")
    assert_same_bits(c, wc, "large mbs codes")
    assert_same_bits(mx.dequantize_mbs(c, s, m, torch.bfloat16),
                     oracle.dequantize_mbs(wc, ws, wm, "bf16"), "large mbs dequant")
    del c, s, m
    assert_same_bits(mx.fakequant_mbs(xd), oracle.dequantize_mbs(wc, ws, wm, "bf16"),
                     "large mbs fakequant")


@pytest.mark.parametrize("rows", [16384, 16385])
def test_oas_nf_layout_threshold(rows):
    # bf16 OAS_NF quantize changes lane layout above 2^23 items (2^26
    # elements): 16384 x 4096 is the largest tensor of the two-lanes-per-block
    # layout, 16385 x 4096 the smallest of the four-lanes one
    rng = np.random.default_rng(31 + rows)
    body = rng.standard_t(3.0, size=(rows, 4096)).astype(np.float32)
    body[:, rng.choice(4096, 20, replace=False)] *= np.float32(50.0)
    x = torch.from_numpy(body).to(torch.bfloat16)
    xh = host_view(x)
    say(f"oas_nf layout threshold {rows}x4096")
    c, s = mx.quantize(x.cuda(), "oas_nf")
    wc, ws = oracle.quantize(xh, "oas_nf", threads=THREADS)
    assert_same_bits(s, ws, f"threshold scales {rows}")
    assert_same_bits(c, wc, f"threshold codes {rows}")


def test_bf16_16384x8192_laplace_all_modes_full():
    x = workloads.bf16_laplace_sparse_outliers(5)
    xh = host_view(x)
    xd = x.cuda()
    mse, qsnr = {}, {}
    for mode in MODES:
        say(f"laplace quantize {mode}")
        c, s = mx.quantize(xd, mode)
        wc, ws = oracle.quantize(xh, mode, threads=THREADS)
        assert_same_bits(s, ws, f"laplace scales {mode}")
        assert_same_bits(c, wc, f"laplace codes {mode}")
        _, sums = mx.block_mse(xd, c, s, per_block=False)
        _, wsse, wssq = oracle.block_mse(xh, wc, ws, threads=THREADS, with_energy=True)
        sse, ssq = sums.tolist()
        assert abs(sse - wsse) <= 1e-6 * wsse and abs(ssq - wssq) <= 1e-6 * wssq
        mse[mode] = sse / x.numel()
        qsnr[mode] = 10 * np.log10(ssq / sse)
    say("laplace tensor MSE " + " ".join(f"{m}={mse[m]:.6g}" for m in MODES))
    say("laplace QSNR dB " + " ".join(f"{m}={qsnr[m]:.4f}" for m in MODES))
    assert mse["oas"] <= mse["ocp"] * (1 + 1e-9)


def _sample_rows(n_rows, n, seed):
    rng = np.random.default_rng(seed)
    pick = np.concatenate([np.arange(min(64, n_rows)), np.arange(max(0, n_rows - 64), n_rows),
                           rng.choice(n_rows, min(n, n_rows), replace=False)])
    return np.unique(pick)


def _check_sampled_rows(x2d: torch.Tensor, c2d: torch.Tensor, s2d: torch.Tensor,
                        label: str, seed: int):
    rows = _sample_rows(x2d.shape[0], 2048, seed)
    idx = torch.from_numpy(rows).to(x2d.device)
    xs = host_view(x2d.index_select(0, idx))
    wc, ws = oracle.quantize(xs, "ocp", threads=THREADS)
    assert_same_bits(c2d.index_select(0, idx), wc, f"{label} codes (sampled rows)")
    assert_same_bits(s2d.index_select(0, idx), ws, f"{label} scales (sampled rows)")
    y = mx.dequantize(c2d, s2d, torch.bfloat16)
    assert_same_bits(y.index_select(0, idx), oracle.dequantize(wc, ws, "bf16"),
                     f"{label} dequant (sampled rows)")
    # whole tensor: dequantize(quantize(x)) is the fused fake-quant, bit for bit
    fq = mx.fakequant(x2d)
    assert torch.equal(fq.view(torch.int16), y.view(torch.int16)), f"{label} fq != dq(q)"
    # and fake-quant is idempotent
    assert torch.equal(mx.fakequant(fq).view(torch.int16), fq.view(torch.int16))


def test_llama32_3b_linears_grouped_full():
    """196 weights [out, in] of a Llama-3.2-3B-shaped stack, grouped by
    in_features into two launches (2.82e9 elements; > 2^31 exercises 64-bit
    indexing)."""
    say("generating llama weights on device")
    a, b = workloads.llama32_3b_grouped("cuda")
    assert a.shape == (688128, 3072) and b.shape == (86016, 8192)
    for t, label, seed in ((a, "llama K=3072", 31), (b, "llama K=8192", 32)):
        say(f"{label} quantize")
        c, s = mx.quantize(t)
        _check_sampled_rows(t, c, s, label, seed)
        del c, s
    # a per-matrix launch gives the same bytes as the grouped launch
    m = workloads.llama32_3b_matrix(5, 4, "cuda")
    cg, sg = mx.quantize(a)
    off = sum(out for layer in range(5) for (n, out, inf) in workloads.LLAMA32_3B_LINEARS
              if inf == 3072) + sum(out for (n, out, inf) in workloads.LLAMA32_3B_LINEARS[:4])
    cm, sm = mx.quantize(m)
    assert torch.equal(cg[off:off + m.shape[0]], cm) and torch.equal(sg[off:off + m.shape[0]], sm)


def test_moe_experts_full():
    say("generating MoE experts on device")
    w13, w2 = workloads.moe_weights("cuda")
    for t, label, seed in ((w13, "moe w13", 41), (w2, "moe w2", 42)):
        say(f"{label} quantize {tuple(t.shape)}")
        c, s = mx.quantize(t)
        assert c.shape == t.shape[:-1] + (t.shape[-1] // 2,)
        assert s.shape == t.shape[:-1] + (t.shape[-1] // 32,)
        k = t.shape[-1]
        _check_sampled_rows(t.view(-1, k), c.view(-1, k // 2), s.view(-1, k // 32), label, seed)
        del c, s


def test_deterministic():
    x = workloads.bf16_laplace_sparse_outliers(6, shape=(4096, 8192)).cuda()
    for mode in MODES:
        c1, s1 = mx.quantize(x, mode)
        c2, s2 = mx.quantize(x, mode)
        assert torch.equal(c1, c2) and torch.equal(s1, s2)
        b1, t1 = mx.block_mse(x, c1, s1)
        b2, t2 = mx.block_mse(x, c1, s1)
        assert torch.equal(b1.view(torch.int32), b2.view(torch.int32))
        assert torch.equal(t1.view(torch.int64), t2.view(torch.int64))


def test_deterministic_other_formats():
    x = workloads.bf16_laplace_sparse_outliers(7, shape=(2048, 8192)).cuda()
    runs = []
    for _ in range(2):
        runs.append([t.clone() for t in (*mx.quantize_mxfp8(x), *mx.quantize_nvfp4(x),
                                         *mx.quantize_mbs(x), mx.fakequant_nvfp4(x),
                                         mx.fakequant_mbs(x), mx.fakequant_mxfp8(x))])
    for a, b in zip(*runs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_concurrent_streams():
    """Two streams at once, each with its own buffers and workspace: results
    equal the same calls made one after another (the library keeps no
    shared state between calls)."""
    xa = workloads.bf16_student_t_outlier_channels(41, shape=(4096, 4096)).cuda()
    xb = workloads.bf16_laplace_sparse_outliers(42, shape=(2048, 8192)).cuda()
    want = []
    for x in (xa, xb):
        c, s = mx.quantize(x, "oas")
        bm, sums = mx.block_mse(x, c, s)
        want.append((c, s, bm, sums, mx.fakequant_nvfp4(x), mx.fakequant(x, "oas_nf")))
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    got = [None, None]
    for _ in range(3):
        for i, (x, st) in enumerate(((xa, sa), (xb, sb))):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                c, s = mx.quantize(x, "oas")
                bm, sums = mx.block_mse(x, c, s)
                got[i] = (c, s, bm, sums, mx.fakequant_nvfp4(x), mx.fakequant(x, "oas_nf"))
        torch.cuda.synchronize()
        for w, g in zip(want, got):
            for a, b in zip(w, g):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_side_stream():
    """Work is enqueued on torch's current stream."""
    x = workloads.bf16_normal(25, (2048, 4096), std=1.0).cuda()
    want = mx.fakequant(x)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = mx.fakequant(x)
    s.synchronize()
    assert torch.equal(y.view(torch.int16), want.view(torch.int16))
