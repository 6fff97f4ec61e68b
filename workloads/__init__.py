"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and
the benchmark.

This module holds no quantization arithmetic: it only draws random numbers,
casts them to bf16/fp32 and lays out test tensors. The tensors it returns are
the ground truth both sides consume; generation details never affect parity.

Workloads (shapes and value distributions follow the pages' workloads):
  * fp32 [1024, 4096] standard normal (seed 1).
  * bf16 activations [8192, 4096]: Student-t(nu=3) body, 20 of the 4096
    hidden channels (0.5 %, rounded) multiplied by 50 as outlier channels
    (seed 2). Outlier-channel activations follow "Unveiling the Potential of
    Quantization with MXFP4" (MBS section) and the BATQuant page (problem
    section).
  * Llama-3.2-3B-shaped linear weights, bf16 N(0, 0.02) [out, in], 28 layers
    x {q, k, v, o, gate, up, down} (seed 3). The QAT example of the Axolotl
    MXFP4 PR page quantizes this model; N(0, 0.02) is the weight example of
    the MXFP4 wiki page (example 2).
  * MoE experts, bf16 N(0, 0.02): w13 [128, 3072, 4096], w2 [128, 4096, 1536]
    (seed 4); the packed-expert layout of the vLLM MXFP8/MXFP4 page ("MXFP4:
    4-bit MoE" section).
  * bf16 activations [16384, 8192]: Laplace(0, 1) body, 0.1 % of elements at
    random positions replaced by +-U(20, 200) (seed 5).
Host-side generation uses numpy.random.default_rng(seed); the bf16 cast is
torch's round-to-nearest-even CPU cast. The two multi-GB weight sets are drawn
on the device with a seeded torch generator (one stream per matrix/expert) so
that a test does not need ~10 GB of host RAM.
"""
from __future__ import annotations

import numpy as np
import torch

# ---- shapes ----------------------------------------------------------------

FP32_NORMAL_SHAPE = (1024, 4096)
STUDENT_T_SHAPE = (8192, 4096)
LAPLACE_SHAPE = (16384, 8192)
STUDENT_T_OUTLIER_CHANNELS = 20
STUDENT_T_OUTLIER_GAIN = 50.0
LAPLACE_OUTLIER_COUNT = 134218  # round(0.001 * 16384 * 8192)

LLAMA32_3B_LAYERS = 28
# (name, out_features, in_features); quantization runs along in_features
LLAMA32_3B_LINEARS = (
    ("q", 3072, 3072), ("k", 1024, 3072), ("v", 1024, 3072), ("o", 3072, 3072),
    ("gate", 8192, 3072), ("up", 8192, 3072), ("down", 3072, 8192),
)
MOE_EXPERTS = 128
MOE_W13_SHAPE = (MOE_EXPERTS, 2 * 1536, 4096)
MOE_W2_SHAPE = (MOE_EXPERTS, 4096, 1536)


def to_bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor (any device) -> host uint16 bit patterns."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(a: np.ndarray) -> torch.Tensor:
    """host uint16 bf16 bit patterns -> CPU bf16 tensor (shares memory)."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


# ---- host-generated workloads ---------------------------------------------

def fp32_normal(seed: int = 1, shape=FP32_NORMAL_SHAPE) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32))


def bf16_student_t_outlier_channels(seed: int = 2, shape=STUDENT_T_SHAPE,
                                    n_channels: int = STUDENT_T_OUTLIER_CHANNELS,
                                    gain: float = STUDENT_T_OUTLIER_GAIN) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    body = rng.standard_t(3.0, size=shape).astype(np.float32)
    chans = rng.choice(shape[-1], n_channels, replace=False)
    body[..., chans] *= np.float32(gain)
    return _bf16(body)


def bf16_laplace_sparse_outliers(seed: int = 5, shape=LAPLACE_SHAPE,
                                 n_outliers: int | None = None) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    if n_outliers is None:
        n_outliers = int(round(0.001 * n))
    body = rng.laplace(0.0, 1.0, size=n).astype(np.float32)
    pos = rng.choice(n, n_outliers, replace=False)
    sign = rng.choice(np.array([-1.0, 1.0], np.float32), n_outliers)
    mag = rng.uniform(20.0, 200.0, n_outliers).astype(np.float32)
    body[pos] = sign * mag
    return _bf16(body.reshape(shape))


def bf16_normal(seed: int, shape, std: float = 0.02) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    return _bf16(rng.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ---- device-generated weight sets (multi-GB) ------------------------------

def _device_normal_bf16(seed: int, shape, std: float, device) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32)
            .mul_(std).to(torch.bfloat16))


def llama32_3b_matrix(layer: int, which: int, device, seed: int = 3) -> torch.Tensor:
    """One [out, in] bf16 weight of the Llama-3.2-3B-shaped stack."""
    _, out_f, in_f = LLAMA32_3B_LINEARS[which]
    return _device_normal_bf16(seed * 1_000_003 + layer * 7 + which, (out_f, in_f), 0.02, device)


def llama32_3b_grouped(device, seed: int = 3):
    """The 196 matrices as two row-stacked tensors grouped by in_features:
    K=3072 (q,k,v,o,gate,up x 28 layers: 688,128 rows) and K=8192 (down x 28:
    86,016 rows)."""
    k3072, k8192 = [], []
    for layer in range(LLAMA32_3B_LAYERS):
        for which in range(len(LLAMA32_3B_LINEARS)):
            m = llama32_3b_matrix(layer, which, device, seed)
            (k8192 if LLAMA32_3B_LINEARS[which][2] == 8192 else k3072).append(m)
    a = torch.cat(k3072, 0)
    del k3072
    b = torch.cat(k8192, 0)
    return a, b


def llama32_3b_arena(device, seed: int = 3):
    """The 196 matrices laid end to end in one contiguous bf16 buffer, layer
    by layer in the order q, k, v, o, gate, up, down (the same values as
    llama32_3b_matrix), and the (offset, out_features, in_features) of each.
    Every matrix starts at a multiple of 3072 * 1024 elements and holds a
    whole number of 32-element blocks per row, so the flat buffer is a run
    of MX blocks in which no block straddles two matrices: quantizing it as
    [n / 3072, 3072] gives every matrix's codes and scales at its offset."""
    total = LLAMA32_3B_LAYERS * sum(o * i for _, o, i in LLAMA32_3B_LINEARS)
    arena = torch.empty(total, dtype=torch.bfloat16, device=device)
    layout = []
    off = 0
    for layer in range(LLAMA32_3B_LAYERS):
        for which, (_, out_f, in_f) in enumerate(LLAMA32_3B_LINEARS):
            m = llama32_3b_matrix(layer, which, device, seed)
            arena[off:off + m.numel()].copy_(m.view(-1))
            layout.append((off, out_f, in_f))
            off += m.numel()
            del m
    assert off == total
    return arena, layout


def moe_weights(device, seed: int = 4):
    """(w13 [128, 3072, 4096], w2 [128, 4096, 1536]) bf16, one stream per expert."""
    w13 = torch.empty(MOE_W13_SHAPE, dtype=torch.bfloat16, device=device)
    w2 = torch.empty(MOE_W2_SHAPE, dtype=torch.bfloat16, device=device)
    for e in range(MOE_EXPERTS):
        w13[e] = _device_normal_bf16(seed * 1_000_003 + 2 * e, MOE_W13_SHAPE[1:], 0.02, device)
        w2[e] = _device_normal_bf16(seed * 1_000_003 + 2 * e + 1, MOE_W2_SHAPE[1:], 0.02, device)
    return w13, w2


# ---- structured test tensors ----------------------------------------------

def exhaustive_bf16_blocks(scale_bytes) -> np.ndarray:
    """bf16 bit patterns, shape [n_blocks, 32], that put every bf16 magnitude
    below 8 * 2^(s-127) (both signs) through a block whose largest element is
    the anchor 4 * 2^(s-127), for each requested scale byte s. Element 0 of
    every block is the anchor; 31 test values follow (the tail is padded with
    zeros)."""
    out = []
    all_mag = np.arange(0, 0x7F80, dtype=np.uint32)  # every finite |bf16|
    for s in scale_bytes:
        # anchor 4*2^(s-127) has biased exponent s+2 (s <= 252)
        anchor = np.uint32((s + 2) << 7)
        limit = np.uint32((s + 3) << 7)  # 8*2^(s-127)
        mags = all_mag[all_mag < limit]
        vals = np.concatenate([mags, mags | 0x8000]).astype(np.uint16)
        n = -(-vals.size // 31)
        pad = np.zeros(n * 31, np.uint16)
        pad[:vals.size] = vals
        blk = np.empty((n, 32), np.uint16)
        blk[:, 0] = anchor
        blk[:, 1:] = pad.reshape(n, 31)
        out.append(blk)
    return np.concatenate(out, 0)


def special_blocks_f32() -> np.ndarray:
    """fp32 blocks [n, 32] exercising zeros, -0, NaN/Inf, subnormals, the E8M0
    range ends and exact ties."""
    f = np.float32
    blocks = []
    z = np.zeros(32, f)
    blocks.append(z.copy())
    blocks.append(-z)  # all -0
    b = z.copy(); b[3] = np.nan; b[4] = 1.0; blocks.append(b)
    b = z.copy(); b[0] = np.inf; b[1] = -2.0; blocks.append(b)
    b = z.copy(); b[5] = -np.inf; blocks.append(b)
    b = z.copy(); b[0] = np.ldexp(f(1), -128); blocks.append(b)        # subnormal alone
    b = z.copy(); b[0] = np.ldexp(f(1), -149); b[1] = -np.ldexp(f(3), -149); blocks.append(b)
    b = z.copy(); b[0] = np.float32(3.4028235e38); b[1] = 1e30; blocks.append(b)  # s = 252
    b = z.copy(); b[:8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0]; blocks.append(b)
    b = z.copy(); b[:8] = [-0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -7.9]; blocks.append(b)
    b = np.full(32, 0.75, f); b[0] = 4.0; b[17:] = 0.0; blocks.append(b)   # OAS tie block
    b = np.full(32, 0.75, f); b[0] = 4.0; b[18:] = 0.0; blocks.append(b)   # OAS picks s0-1
    b = z.copy(); b[0] = np.ldexp(f(1.5), -126); b[1] = np.ldexp(f(1), -127); blocks.append(b)
    b = np.linspace(-7.5, 7.5, 32).astype(f); blocks.append(b)
    return np.stack(blocks)


def oas_tie_prone_blocks(seed: int, n_blocks: int) -> np.ndarray:
    """fp32 blocks [n_blocks, 32] built so that the overflow-aware choice goes
    both ways: many values that sit on rounding ties at scale 2^(s-127) but on
    the grid at half that scale, mixed with eighths, a top element near 4 and
    a random power-of-two block scale."""
    rng = np.random.default_rng(seed)
    tie_prone = np.array([0.25, 0.75, 0.75, 0.5, 1.0, 1.25, 0.0])
    x = (rng.integers(-8, 9, (n_blocks, 32)) / 8.0)
    n_tie = rng.integers(8, 33, n_blocks)
    mask = np.arange(32)[None, :] < n_tie[:, None]
    tie = rng.choice(tie_prone, (n_blocks, 32)) * rng.choice([-1.0, 1.0], (n_blocks, 32))
    x = np.where(mask, tie, x)
    top = rng.choice([4.0, 4.0, 4.125, -4.0, 5.0, 7.5], n_blocks)
    x[np.arange(n_blocks), rng.integers(0, 32, n_blocks)] = top
    x *= 2.0 ** rng.integers(-100, 100, (n_blocks, 1))
    return x.astype(np.float32)
