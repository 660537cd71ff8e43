"""Helpers shared by the GPU parity tests: device copies, oracle inputs, tolerances.

Tolerances (applied element by element against the fp64 oracle):
  * bf16 outputs, and fp32 intermediates computed from bf16 inputs (whose
    P*V product rounds probabilities to bf16): max-abs 1e-2, mean-abs 1e-3;
  * fp32 outputs of the fp32 path, and the merge fed identical fp32 partials:
    max-abs 1e-5;
  * LSE: max-abs 1e-4 everywhere.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle

BF16_MAX, BF16_MEAN = 1e-2, 1e-3
F32_MAX = 1e-5
LSE_MAX = 1e-4


def say(msg: str) -> None:
    """Name the case on stdout before GPU work starts (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a CPU/GPU tensor (bf16 decoded bit by bit)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy())
    return t.to(torch.float64).numpy()


def check_o(got: torch.Tensor, want: np.ndarray, kind: str, what: str = "O") -> None:
    g = to_f64(got)
    assert g.shape == want.shape, (g.shape, want.shape)
    assert not np.any(np.isnan(g)), f"{what}: NaN in GPU output"
    err = np.abs(g - want)
    if kind == "bf16":
        assert err.max() <= BF16_MAX, f"{what}: max-abs {err.max():.3e} > {BF16_MAX}"
        assert err.mean() <= BF16_MEAN, f"{what}: mean-abs {err.mean():.3e} > {BF16_MEAN}"
    else:
        assert err.max() <= F32_MAX, f"{what}: max-abs {err.max():.3e} > {F32_MAX}"


def check_o_scaled(got: torch.Tensor, want: np.ndarray, what: str = "O",
                   mean_rel: float = 2.0 ** -7) -> None:
    """bf16-rounded outputs that need not be small (few visible keys, peaky
    softmax): bf16 rounds a value of size |x| by up to 2^-8 |x| on its own, so
    the bars scale with the reference: max-abs <= 1e-2 * max(1, max|ref|),
    mean-abs <= max(1e-3, mean_rel * mean|ref|)."""
    g = to_f64(got)
    assert g.shape == want.shape and not np.any(np.isnan(g)), what
    err = np.abs(g - want)
    big = max(1.0, float(np.abs(want).max()))
    mean_bar = max(BF16_MEAN, mean_rel * float(np.abs(want).mean()))
    assert err.max() <= BF16_MAX * big, f"{what}: max-abs {err.max():.3e} > {BF16_MAX} * {big:.2f}"
    assert err.mean() <= mean_bar, f"{what}: mean-abs {err.mean():.3e} > {mean_bar:.3e}"


def check_lse(got: torch.Tensor, want: np.ndarray, what: str = "LSE") -> None:
    g = to_f64(got)
    assert g.shape == want.shape, (g.shape, want.shape)
    fin = np.isfinite(want)
    assert np.array_equal(np.isneginf(g), np.isneginf(want)), f"{what}: -inf rows differ"
    assert not np.any(np.isnan(g)) and not np.any(np.isposinf(g)), f"{what}: NaN/+inf"
    if fin.any():
        err = np.abs(g[fin] - want[fin]).max()
        assert err <= LSE_MAX, f"{what}: max-abs {err:.3e} > {LSE_MAX}"


def kind_of(in_dtype: torch.dtype) -> str:
    return "bf16" if in_dtype == torch.bfloat16 else "f32"
