"""Shared test helpers: tolerances and comparisons (no method arithmetic)."""

import numpy as np
import torch

# Output tolerances: bf16 max-abs 2e-2 and relative Frobenius 1e-2; fp32 1e-4
# for both.  lse (natural log): 5e-3 for bf16 inputs, 2e-5 for fp32.
TOL = {
    torch.bfloat16: dict(max_abs=2e-2, rel_fro=1e-2, lse=5e-3),
    torch.float32: dict(max_abs=1e-4, rel_fro=1e-4, lse=2e-5),
}


def np32(t):
    """Tensor -> float32 numpy on the host (bf16 values are exact in fp32)."""
    return t.detach().to("cpu", torch.float32).numpy()


def compare(got, ref, dtype, what=""):
    """Assert got (GPU) matches ref (oracle, fp64) within the tolerances."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    tol = TOL[dtype]
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / denom) if denom > 0 else 0.0
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert max_abs <= tol["max_abs"], f"{what}: max-abs {max_abs:.3e} > {tol['max_abs']}"
    assert rel <= tol["rel_fro"], f"{what}: rel-Frobenius {rel:.3e} > {tol['rel_fro']}"
    return max_abs, rel


def compare_lse(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):             # -inf - -inf where both are empty rows
        err = np.where(both_inf, 0.0, np.abs(got - ref))
    m = float(err.max()) if err.size else 0.0
    assert m <= TOL[dtype]["lse"], f"{what}: lse max-abs {m:.3e} > {TOL[dtype]['lse']}"
    return m
