"""Shared helpers for the parity tests (no arithmetic of the method here)."""
import numpy as np

# The band the pages use for GPU kernels against a C-side oracle (moeflux
# expert_forward.rs, module doc, Tolerance regime).
BAND_MAX_ABS_REL = 1e-3
BAND_COSINE = 0.9999

# A tighter bound under the band, for regressions the band would let through
# (an intermediate rounded to fp16, a dropped low part of the split
# activations, a scale applied in the wrong precision).  Every schedule's
# measured error across the GPU suite is at most 2.0e-6 of max|out|
# (activations at any power-of-two scale from 2^-24 to 2^18 included) with
# 1 - cosine at most 2e-12; the bound sits ten times above that, fifty times
# below the band.
REGRESSION_MAX_ABS_REL = 2e-5
REGRESSION_ONE_MINUS_COS = 1e-9


def band(got, want, what=""):
    """Assert the fp32 parity band and the regression bound under it; return
    (max_abs_diff / max|want|, cosine)."""
    got = np.asarray(got, np.float64).reshape(-1)
    want = np.asarray(want, np.float64).reshape(-1)
    assert got.shape == want.shape, what
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx = np.abs(want).max()
    diff = np.abs(got - want).max()
    rel = diff / mx if mx > 0 else diff
    nrm = np.linalg.norm(got) * np.linalg.norm(want)
    cos = float(got @ want / nrm) if nrm > 0 else 1.0
    assert rel <= BAND_MAX_ABS_REL, f"{what}: max_abs_diff/max|out| = {rel:.3g}"
    assert cos >= BAND_COSINE, f"{what}: cosine {cos:.8f}"
    assert rel <= REGRESSION_MAX_ABS_REL, \
        f"{what}: max_abs_diff/max|out| = {rel:.3g}, inside the band but above the regression bound"
    assert 1.0 - cos <= REGRESSION_ONE_MINUS_COS, \
        f"{what}: 1 - cosine = {1.0 - cos:.3g}, inside the band but above the regression bound"
    return rel, cos


def bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)
