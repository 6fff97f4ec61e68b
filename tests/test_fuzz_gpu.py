"""Seeded random tensors with special values mixed in, through every format
and entry point, against the oracle (same bar as the other parity tests:
bit for bit, block MSE and tensor sums to a relative 1e-6).

Each tensor draws its shape (rows 1-6, k a multiple of 128 up to 512), a
magnitude per 32-element block from across the fp32 exponent range, blocks
of exact grid points and ties (values m * 2^e with m on and between the E2M1
grid), and single NaN, +-Inf, +-0, fp32 subnormals and fp32 extremes placed
at random. The bf16 copy of each tensor runs too."""
import numpy as np
import pytest
import torch

from test_fused_gpu import check_fused
from test_parity_gpu import MODES, check_all_ops
from test_parity_mbs_gpu import check_mbs
from test_parity_mxfp8_gpu import check8
from test_parity_nvfp4_gpu import check_nv

pytestmark = pytest.mark.gpu

SPECIALS = np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.4e-45, -1.4e-45, 1.0e-40,
                     1.1754944e-38, 3.4028235e38, -3.4028235e38], np.float32)
GRID_AND_TIES = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6, 7])


def random_tensor(rng: np.random.Generator) -> torch.Tensor:
    rows, k = int(rng.integers(1, 7)), 128 * int(rng.integers(1, 5))
    nb = rows * k // 32
    e = np.clip(np.rint(rng.normal(0, 45, nb)), -148, 124).astype(np.int64)
    heavy = rng.standard_t(3, (nb, 32))
    grid = rng.choice(GRID_AND_TIES, (nb, 32)) * rng.choice([-1.0, 1.0], (nb, 32))
    v = np.where((rng.random(nb) < 0.3)[:, None], grid, heavy) * np.ldexp(1.0, e)[:, None]
    with np.errstate(over="ignore"):
        x = v.astype(np.float32)
    hit = rng.random(x.shape) < 0.004
    x[hit] = rng.choice(SPECIALS, int(hit.sum()))
    return torch.from_numpy(x.reshape(rows, k))


@pytest.mark.parametrize("seed", range(24))
def test_fuzz_every_entry_point(seed):
    rng = np.random.default_rng(7000 + seed)
    for case in range(10):
        x = random_tensor(rng)
        for xt in (x, x.to(torch.bfloat16)):
            label = f"fuzz seed {seed} case {case} {tuple(xt.shape)} {xt.dtype}"
            check_all_ops(xt, label)
            check_fused(xt, MODES[case % len(MODES)], label)
            check8(xt, label)
            check_nv(xt, label)
            check_mbs(xt, label)
