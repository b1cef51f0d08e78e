"""Shared comparison helpers for the GPU parity tests.

Floating-point bar (reading of "max-abs 1e-2 / max-rel 2e-2", bf16 in/out,
fp32 accumulate): an output passes when, for every element,
    |gpu - ref| <= 1e-2 + 2e-2 * |ref|
and, over the whole tensor,
    max |gpu - ref| <= 2e-2 * max |ref|.
The second (norm-relative) term keeps the bar discriminating when outputs are
small; the negative controls in the tests must fail it.
"""
import numpy as np

ATOL = 1e-2
RTOL = 2e-2


def close_report(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    elem_ok = bool(np.all(err <= ATOL + RTOL * np.abs(ref)))
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    norm_ok = bool(err.max() <= RTOL * scale) if ref.size else True
    return elem_ok and norm_ok, float(err.max()) if ref.size else 0.0


def assert_close(got, ref, what=""):
    ok, e = close_report(got, ref)
    ref = np.asarray(ref)
    assert ok, f"{what}: max abs err {e:.3e} (ref max {np.abs(ref).max():.3e})"
    return e
