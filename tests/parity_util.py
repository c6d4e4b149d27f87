"""Helpers for comparing the HIP path against the oracle (no arithmetic of the method here)."""
import numpy as np

# Acceptance bars: fp32 outputs need both; bf16-input paths need the relative Frobenius bar,
# measured against the oracle run on the same bf16-rounded inputs.
F32_REL_FROB = 1e-5
F32_MAX_ABS = 1e-4
BF16_REL_FROB = 5e-3


def errors(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    diff = got - want
    denom = np.linalg.norm(want.ravel())
    rel = np.linalg.norm(diff.ravel()) / (denom if denom > 0 else 1.0)
    mx = float(np.abs(diff).max()) if diff.size else 0.0
    return float(rel), mx


def assert_f32(got, want, what=""):
    rel, mx = errors(got, want)
    print(f"    {what}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= F32_REL_FROB and mx <= F32_MAX_ABS, (what, rel, mx)


def assert_bf16(got, want, what=""):
    rel, mx = errors(got, want)
    print(f"    {what}: rel_frob={rel:.3e} max_abs={mx:.3e}", flush=True)
    assert rel <= BF16_REL_FROB, (what, rel, mx)
