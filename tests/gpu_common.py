"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch

# Tolerances of the HIP path against the fp64 oracle.
BF16_MAX_ABS, BF16_MEAN_ABS = 2e-2, 2e-3
F32_MAX_ABS = 1e-4
LSE_ABS = {"bf16": 1e-3, "f32": 1e-5}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_out_close(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "output"):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(want)), "oracle produced non-finite values"
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values in the GPU result"
    if dtype == "bf16":
        assert err.max() <= BF16_MAX_ABS, f"{what}: max-abs {err.max():.3e}"
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean-abs {err.mean():.3e}"
    else:
        assert err.max() <= F32_MAX_ABS, f"{what}: max-abs {err.max():.3e}"


def assert_lse_close(got: np.ndarray, want: np.ndarray, dtype: str):
    err = np.abs(got - want)
    assert np.all(np.isfinite(got))
    assert err.max() <= LSE_ABS[dtype], f"lse max-abs {err.max():.3e}"


def device() -> torch.device:
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch.device("cuda:0")


class LazyF64:
    """Read-only [b, h, ...] view of a CPU tensor that converts each slice to float64
    on access, so the oracle can sample a large bf16 input without a full copy."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        return self.t[idx].float().numpy().astype(np.float64)


def assert_rows_match_oracle(got_o: np.ndarray, got_l: np.ndarray, want_o: np.ndarray, want_l: np.ndarray,
                             dtype: str, what: str = "decode"):
    """Decode results [B, H, D] / [B, H] against the oracle's, NaN rows included: a row
    the oracle leaves NaN (an invalid length, a bad page) must be NaN in output and
    logsumexp, every other row within the tolerance."""
    nan_rows = np.isnan(want_o).any(axis=-1) | np.isnan(want_l)
    assert np.isnan(want_o[nan_rows]).all() and np.isnan(want_l[nan_rows]).all()
    assert np.isnan(got_o[nan_rows]).all(), f"{what}: rows the oracle leaves NaN are not NaN"
    assert np.isnan(got_l[nan_rows]).all(), f"{what}: logsumexp of NaN rows is not NaN"
    if (~nan_rows).any():
        assert_out_close(got_o[~nan_rows], want_o[~nan_rows], dtype, what)
        assert_lse_close(got_l[~nan_rows], want_l[~nan_rows], dtype)
