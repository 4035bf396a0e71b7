"""Helpers for GPU-vs-oracle parity tests (comparison and row sampling only)."""

import numpy as np
import torch

# Tolerances stated for this path: bf16 outputs vs the fp64 oracle,
# fp8-e4m3 forward vs the oracle on the dequantised inputs.
BF16_MAX_ABS, BF16_MEAN_ABS = 1e-2, 1e-3
FP8_MAX_ABS = 6e-2
LSE_MAX_ABS = 1e-3


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mask = ~np.isnan(ref)
    d = np.abs(got[mask] - ref[mask])
    return float(d.max()) if d.size else 0.0, float(d.mean()) if d.size else 0.0


def assert_close(got, ref, max_abs=BF16_MAX_ABS, mean_abs=BF16_MEAN_ABS, what="O"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    mask = ~np.isnan(ref)
    assert np.isfinite(got[mask]).all(), f"{what}: non-finite values where the oracle is finite"
    mx, mn = errors(got, ref)
    assert mx <= max_abs, f"{what}: max abs error {mx:.3e} > {max_abs:.1e}"
    if mean_abs is not None:
        assert mn <= mean_abs, f"{what}: mean abs error {mn:.3e} > {mean_abs:.1e}"
    return mx, mn


def assert_lse_close(got, ref, tol=LSE_MAX_ABS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    finite = np.isfinite(ref)
    assert (both_inf | finite | np.isnan(ref)).all()
    assert (np.isneginf(got) == np.isneginf(ref))[~np.isnan(ref)].all(), "LSE: -inf rows differ"
    d = np.abs(got[finite] - ref[finite])
    mx = float(d.max()) if d.size else 0.0
    assert mx <= tol, f"LSE: max abs error {mx:.3e} > {tol:.1e}"
    return mx


def sample_rows(n, count, seed):
    """Sorted sample of query rows that always includes the first and last."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    rows.update({0, n - 1})
    return np.array(sorted(rows))
