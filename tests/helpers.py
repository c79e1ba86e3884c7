"""Shared test helpers: comparison against the oracle (no method arithmetic)."""

import numpy as np

BF16_TOL = 2e-2  # relative L2, bf16 inputs with float32 accumulation
F32_TOL = 1e-5   # relative L2, float32 inputs


def to64(t):
    """Exact float64 copy of a torch tensor (bf16 and fp32 upcast exactly)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def assert_close(got, ref, tol, what="", per_head_axes=2):
    """Relative L2 over the whole tensor and, for [B,H,...] tensors, for every
    (b, h) slice (so a fast-decaying head cannot hide behind a slow one)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = rel_l2(got, ref)
    assert err <= tol, f"{what}: rel L2 {err:.3e} > {tol:.1e}"
    if per_head_axes and got.ndim > per_head_axes:
        lead = got.shape[:per_head_axes]
        worst = 0.0
        for idx in np.ndindex(*lead):
            if np.linalg.norm(ref[idx]) > 0:
                worst = max(worst, rel_l2(got[idx], ref[idx]))
        assert worst <= tol, f"{what}: worst per-head rel L2 {worst:.3e} > {tol:.1e}"
    return err
