"""The two multi-GB weight workloads, every element against the oracle.

Llama-3.2-3B-shaped linears (Axolotl MXFP4 PR page, QAT example on
Llama-3.2-3B): the 196 matrices laid end to end in one buffer and quantized
by one launch per operation, the launch configuration the benchmark times.
MoE experts (vLLM MXFP8/MXFP4 page, "MXFP4: 4-bit MoE": packed w13
[E, 2I, H] and w2 [E, H, I] quantized along the last dimension): one launch
per tensor. Codes, scales and dequantized values are compared with the oracle
bit for bit over the whole tensors (2,818,572,288 + 2,415,919,104 elements),
streamed through host memory in chunks; block MSE and tensor sums to a
relative 1e-6; fake-quant against dequantize(quantize) on the device; each
matrix's or expert's own launch, and the 196 matrices as separate tensors
through the multi-tensor calls, against their slices of the big launch.
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
CHUNK_ELEMS = 3072 * 65536  # 201,326,592 elements (384 MiB of bf16) per host round trip


def say(msg):
    print(f"[whole] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _setup():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mx.load_library()
    oracle.build(force=not os.path.exists(os.path.join(os.path.dirname(oracle.__file__),
                                                       "libmxref.so")))
    yield
    torch.cuda.empty_cache()


def _same(got: torch.Tensor, want: np.ndarray, what: str):
    g = got.cpu().numpy()
    if g.dtype != want.dtype:
        g = g.view(want.dtype)
    assert g.shape == want.shape, (what, g.shape, want.shape)
    if not np.array_equal(g, want):
        bad = np.flatnonzero(g.reshape(-1) != want.reshape(-1))
        raise AssertionError(f"{what}: {bad.size} mismatches, first at {bad[:5]}")


def check_whole(x: torch.Tensor, label: str, outs: dict):
    """x [R, K] bf16 on the device; outs maps a mode to (codes, scales) and,
    for "ocp", also y (bf16 dequantize) and (block_mse, tensor_sums). Every
    chunk of rows goes to the host once and through the oracle in each mode."""
    R, K = x.shape
    rows_per = max(1, CHUNK_ELEMS // K)
    sse = ssq = 0.0
    for r0 in range(0, R, rows_per):
        r1 = min(R, r0 + rows_per)
        xs = workloads.to_bf16_bits(x[r0:r1])
        for mode, o in outs.items():
            wc, ws = oracle.quantize(xs, mode, threads=THREADS)
            _same(o["codes"][r0:r1], wc, f"{label} codes {mode} rows {r0}:{r1}")
            _same(o["scales"][r0:r1], ws, f"{label} scales {mode} rows {r0}:{r1}")
            if "y" in o:
                wy = oracle.dequantize(wc, ws, "bf16", threads=THREADS)
                _same(o["y"][r0:r1].view(torch.int16), wy.view(np.int16),
                      f"{label} dequant {mode} rows {r0}:{r1}")
                del wy
            if "bm" in o:
                wbm, wsse, wssq = oracle.block_mse(xs, wc, ws, threads=THREADS, with_energy=True)
                np.testing.assert_allclose(o["bm"][r0:r1].cpu().numpy(), wbm, rtol=1e-6, atol=0)
                sse += wsse
                ssq += wssq
        say(f"{label}: rows {r1} / {R} match")
    if "ocp" in outs and "sums" in outs["ocp"]:
        got_sse, got_ssq = outs["ocp"]["sums"].tolist()
        assert abs(got_sse - sse) <= 1e-6 * sse and abs(got_ssq - ssq) <= 1e-6 * ssq, \
            (got_sse, sse, got_ssq, ssq)


def test_llama32_3b_linears_whole():
    say("generating the Llama-3.2-3B arena (196 matrices, 2.82e9 elements)")
    arena, layout = workloads.llama32_3b_arena("cuda")
    x = arena.view(-1, 3072)
    say("quantize OCP / dequantize / block MSE / quantize OAS: one launch each")
    c, s = mx.quantize(x, "ocp")
    y = mx.dequantize(c, s, torch.bfloat16)
    bm, sums = mx.block_mse(x, c, s)
    c2, s2 = mx.quantize(x, "oas")
    # fake-quant is dequantize(quantize) bit for bit, in both modes
    for mode, (cm, sm) in (("ocp", (c, s)), ("oas", (c2, s2))):
        fq = mx.fakequant(x, mode)
        yy = y if mode == "ocp" else mx.dequantize(cm, sm, torch.bfloat16)
        assert torch.equal(fq.view(torch.int16), yy.view(torch.int16)), f"llama fakequant {mode}"
        del fq, yy
    torch.cuda.empty_cache()
    # each matrix quantized on its own equals its slice of the one launch
    say("196 per-matrix launches against the arena launch")
    cf, sf = c.view(-1), s.view(-1)
    for off, out_f, in_f in layout:
        m = arena[off:off + out_f * in_f].view(out_f, in_f)
        cm, sm = mx.quantize(m, "ocp")
        assert torch.equal(cm.view(-1), cf[off // 2:(off + out_f * in_f) // 2]), off
        assert torch.equal(sm.view(-1), sf[off // 32:(off + out_f * in_f) // 32]), off
    del cm, sm
    # the 196 matrices as separate tensors through the multi-tensor calls
    # (chunks of 48 matrices, ~7e8 elements each: the large-tensor tiling)
    say("196 matrices through quantize_multi (OCP, OAS) and fakequant_multi (OCP)")
    mats = [arena[off:off + out_f * in_f].view(out_f, in_f) for off, out_f, in_f in layout]
    cf2, sf2 = c2.view(-1), s2.view(-1)
    for mode, (cw, sw) in (("ocp", (cf, sf)), ("oas", (cf2, sf2))):
        outs = mx.quantize_multi(mats, mode)
        for (off, out_f, in_f), (cm, sm) in zip(layout, outs):
            n = out_f * in_f
            assert torch.equal(cm.view(-1), cw[off // 2:(off + n) // 2]), (mode, off)
            assert torch.equal(sm.view(-1), sw[off // 32:(off + n) // 32]), (mode, off)
        del outs
    yf = y.view(-1)
    fqs = mx.fakequant_multi(mats)
    for (off, out_f, in_f), fm in zip(layout, fqs):
        assert torch.equal(fm.view(-1).view(torch.int16),
                           yf[off:off + out_f * in_f].view(torch.int16)), ("fakequant_multi", off)
    del fqs, mats
    torch.cuda.empty_cache()
    check_whole(x, "llama", {"ocp": {"codes": c, "scales": s, "y": y, "bm": bm, "sums": sums},
                             "oas": {"codes": c2, "scales": s2}})


def test_moe_experts_whole():
    say("generating MoE experts (w13 [128, 3072, 4096], w2 [128, 4096, 1536])")
    w13, w2 = workloads.moe_weights("cuda")
    for t, label in ((w13, "moe w13"), (w2, "moe w2")):
        E, N, K = t.shape
        x = t.view(-1, K)
        say(f"{label}: quantize / dequantize, one launch each")
        c, s = mx.quantize(x, "ocp")
        y = mx.dequantize(c, s, torch.bfloat16)
        c3, s3 = c.view(E, N, K // 2), s.view(E, N, K // 32)
        for e in range(E):  # one launch per expert gives the same bytes
            ce, se = mx.quantize(t[e], "ocp")
            assert torch.equal(ce, c3[e]) and torch.equal(se, s3[e]), (label, e)
        del ce, se
        check_whole(x, label, {"ocp": {"codes": c, "scales": s, "y": y}})
        del c, s, y
        torch.cuda.empty_cache()
