"""Helpers of the GPU parity tests: moving the seeded input bits to the
device, reading results back, and the comparison rules.

Tolerances (fixed by the target of this work and written here once):
  * permute: bit-exact;
  * bf16 outputs: max |O_gpu - O_oracle| <= 2e-2, LSE max abs error <= 1e-3;
  * fp32 inputs: ||O_gpu - O_oracle||_inf / ||O_oracle||_inf <= 1e-5, the
    same for the LSE;
  * rows the oracle gives (0, -inf) must come back exactly (0, -inf).
"""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

BF16_O_ATOL = 2e-2
BF16_LSE_ATOL = 1e-3
FP32_REL = 1e-5


def say(*a):
    """Progress line, flushed, so a hang or fault names its case."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.cuda().view(torch.bfloat16)


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return dev_bf16(x)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_pair(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray,
               dtype: str, what: str = "") -> dict:
    """Compare (O, LSE) with the oracle under the stated tolerance; returns
    the error figures.  Shapes must agree; LSE -inf rows must match exactly."""
    assert o_gpu.shape == o_ref.shape, (o_gpu.shape, o_ref.shape)
    assert lse_gpu.shape == lse_ref.shape, (lse_gpu.shape, lse_ref.shape)
    assert not np.isnan(o_gpu).any(), what + ": NaN in O"
    assert not np.isnan(lse_gpu).any(), what + ": NaN in LSE"
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse_gpu), empty), what + ": -inf rows differ"
    assert np.isfinite(lse_gpu[~empty]).all(), what + ": non-finite LSE"
    if empty.any():
        assert (o_gpu[empty] == 0).all(), what + ": rows without keys must give O = 0"
    fin = ~empty
    o_err = float(np.max(np.abs(o_gpu - o_ref))) if o_gpu.size else 0.0
    l_err = float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))) if fin.any() else 0.0
    if dtype == "bf16":
        assert o_err <= BF16_O_ATOL, "%s: O max abs err %.3e > %.1e" % (what, o_err, BF16_O_ATOL)
        assert l_err <= BF16_LSE_ATOL, "%s: LSE max abs err %.3e > %.1e" % (what, l_err, BF16_LSE_ATOL)
    else:
        o_scale = float(np.max(np.abs(o_ref))) if o_ref.size else 0.0
        l_scale = float(np.max(np.abs(lse_ref[fin]))) if fin.any() else 0.0
        o_rel = o_err / o_scale if o_scale > 0 else o_err
        l_rel = l_err / l_scale if l_scale > 0 else l_err
        assert o_rel <= FP32_REL, "%s: O rel err %.3e > %.0e" % (what, o_rel, FP32_REL)
        assert l_rel <= FP32_REL, "%s: LSE rel err %.3e > %.0e" % (what, l_rel, FP32_REL)
    return {"o_err": o_err, "lse_err": l_err}


def sample_rows(n: int, count: int, seed: int, tile: int = 128) -> np.ndarray:
    """Rows to check at full size: the first and last rows, rows on both
    sides of every few tile boundaries, and random rows."""
    rng = np.random.default_rng(seed)
    picks = {0, n - 1, min(n - 1, 1)}
    for t in range(tile, n, tile * max(1, (n // tile) // 8)):
        picks.update({t - 1, t})
    picks.update(rng.integers(0, n, size=max(0, count - len(picks))).tolist())
    return np.array(sorted(p for p in picks if 0 <= p < n), dtype=np.int64)


def finite_or_neginf(x: float) -> str:
    return "-inf" if x == -math.inf else "%.6g" % x
