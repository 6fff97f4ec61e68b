"""The C ABI from a plain C99 program (tests/c_client/c_client.c): no Python
binding, no torch, a HIP stream of the client's own. The client calls every
entry point, including refused arguments, and writes its input and outputs
to a file; here every output is checked against the oracle on the same
input, bit for bit (block MSE to a relative 1e-6)."""
import importlib.util
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from conftest import ROOT

pytestmark = pytest.mark.gpu

ROWS, K = 37, 4224
CLIENT_DIR = os.path.join(ROOT, "tests", "c_client")


def _client() -> str:
    exe = os.path.join(CLIENT_DIR, "c_client")
    if not os.path.exists(exe):
        spec = importlib.util.spec_from_file_location(
            "build_client", os.path.join(CLIENT_DIR, "build_client.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        exe = mod.build()
    return exe


def _records(path: str) -> dict:
    recs = {}
    with open(path, "rb") as f:
        while True:
            tag = f.read(32)
            if not tag:
                return recs
            n = int(np.frombuffer(f.read(8), np.int64)[0])
            recs[tag.rstrip(b"\0").decode()] = f.read(n)


def _u8(b, shape):
    return np.frombuffer(b, np.uint8).reshape(shape)


def _same(got: bytes, want: np.ndarray, what: str):
    g = np.frombuffer(got, want.dtype).reshape(want.shape)
    bad = np.flatnonzero(g.view(np.uint8).reshape(-1) != want.view(np.uint8).reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at byte {bad[0]}"


def _close_mse(got_block: bytes, got_sums: bytes, want_block, want_sse, want_ssq, what: str):
    gb = np.frombuffer(got_block, np.float32).reshape(want_block.shape)
    assert np.allclose(gb, want_block, rtol=1e-6, atol=0, equal_nan=True), what
    for g, w in zip(np.frombuffer(got_sums, np.float64), (want_sse, want_ssq)):
        assert (np.isnan(g) and np.isnan(w)) or g == w or abs(g - w) <= 1e-6 * abs(w), \
            f"{what}: tensor sums {g} vs {w}"


@pytest.fixture(scope="module")
def recs(tmp_path_factory):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = _client()
    out = str(tmp_path_factory.mktemp("c_client") / "out.bin")
    print(f"running {exe}", flush=True)
    r = subprocess.run([exe, out], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failed call(s)" in r.stdout
    return _records(out)


def test_c_client_mxfp4(recs):
    x16 = np.frombuffer(recs["x16"], np.uint16).reshape(ROWS, K)
    x32 = np.frombuffer(recs["x32"], np.float32).reshape(ROWS, K)
    wc, ws = oracle.quantize(x16, "ocp")
    _same(recs["q_ocp_bf16.codes"], wc, "codes (OCP, bf16)")
    _same(recs["q_ocp_bf16.scales"], ws, "scales (OCP, bf16)")
    _same(recs["dq_ocp.bf16"], oracle.dequantize(wc, ws, "bf16"), "dequantize -> bf16")
    _same(recs["dq_ocp.f32"], oracle.dequantize(wc, ws, "f32"), "dequantize -> f32")
    bm, sse, ssq = oracle.block_mse(x16, wc, ws, with_energy=True)
    _close_mse(recs["mse_ocp_bf16.block"], recs["mse_ocp_bf16.sums"], bm, sse, ssq, "block MSE")
    for name, x, mode in (("q_oas_nf_bf16", x16, "oas_nf"), ("q_oas_f32", x32, "oas"),
                          ("multi_oas_bf16", x16, "oas")):
        c, s = oracle.quantize(x, mode)
        _same(recs[name + ".codes"], c, name + " codes")
        _same(recs[name + ".scales"], s, name + " scales")
    _same(recs["fq_oas_bits_bf16"], oracle.fakequant(x16, "oas_bits"), "in-place fake-quant")
    c, s = oracle.quantize(x32, "ocp")
    _same(recs["fused_f32.codes"], c, "one-pass codes")
    _same(recs["fused_f32.scales"], s, "one-pass scales")
    _same(recs["fused_f32.y"], oracle.fakequant(x32, "ocp"), "one-pass y")
    bm, sse, ssq = oracle.block_mse(x32, c, s, with_energy=True)
    _close_mse(recs["fused_f32.block"], recs["fused_f32.sums"], bm, sse, ssq, "one-pass error")


def test_c_client_other_formats(recs):
    x16 = np.frombuffer(recs["x16"], np.uint16).reshape(ROWS, K)
    x32 = np.frombuffer(recs["x32"], np.float32).reshape(ROWS, K)
    c8, s8 = oracle.quantize_mxfp8(x16)
    _same(recs["q8_bf16.codes"], c8, "MXFP8 codes")
    _same(recs["q8_bf16.scales"], s8, "MXFP8 scales")
    cn, bn, tn = oracle.quantize_nvfp4(x32)
    _same(recs["qnv_f32.codes"], cn, "NVFP4 codes")
    _same(recs["qnv_f32.block_scales"], bn, "NVFP4 block scales")
    assert recs["qnv_f32.tensor_scale"][0] == tn, "NVFP4 tensor scale"
    cm, sm, mm = oracle.quantize_mbs(x16)
    _same(recs["qmbs_bf16.codes"], cm, "MBS codes")
    _same(recs["qmbs_bf16.sub_scales"], sm, "MBS sub-block scales")
    _same(recs["qmbs_bf16.macro"], mm, "MBS macro bytes")
    _same(recs["fqmbs_f32"], oracle.dequantize_mbs(*oracle.quantize_mbs(x32), "f32"),
          "MBS fake-quant")
