"""Parity metric between a device result and the fp64 oracle -- TEST INFRASTRUCTURE ONLY.

"Max relative error" is undefined where the oracle's value is near zero, and y
crosses zero (it is a signed sum over n), so each element's error is divided
by the larger of its own magnitude and the RMS of the oracle tensor it
belongs to:

    err = max_i |got_i - ref_i| / max(|ref_i|, rms(ref))

The same metric applies to final states.  `normwise` is the plain
max|got - ref| / max|ref| reported beside it.
"""
from __future__ import annotations

import numpy as np


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise ValueError(f"shape mismatch {got.shape} vs {ref.shape}")
    if ref.size == 0:
        return 0.0
    if not np.all(np.isfinite(got) == np.isfinite(ref)):
        return float("inf")
    fin = np.isfinite(ref)
    if not fin.all():
        if not np.array_equal(got[~fin], ref[~fin], equal_nan=True):
            return float("inf")
        got, ref = got[fin], ref[fin]
        if ref.size == 0:
            return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.abs(got - ref) / den))


def normwise(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    return float(np.max(np.abs(got - ref)) / m) if m > 0 else float(np.max(np.abs(got - ref), initial=0.0))


# Gates: fp32 inputs vs the oracle; bf16 inputs (fp32 state) vs the oracle run on
# the same bf16-rounded inputs.
TOL = {"f32": 1e-4, "bf16": 2e-2}
