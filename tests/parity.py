"""Parity criterion shared by the GPU tests (and by the mutation test that shows it has teeth).

Outputs of a bf16-in / fp32-accumulate attention are compared with the fp64
oracle by maximum absolute difference.  The bound 2e-2 on max|diff| is applied
relative to max(1, max|ref|), so for outputs of magnitude <= 1 it is exactly an
absolute 2e-2; a second term requires max|diff| <= 1% of max|ref| so that an
all-zero answer cannot pass when the outputs are small.  The mask is compared
bit for bit elsewhere.
"""
from __future__ import annotations

import numpy as np

ABS_TOL = 2e-2
REL_TOL = 1e-2
LSE_TOL = 1e-2


def out_errors(got, ref) -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(got - ref)
    max_abs = float(np.max(d)) if d.size else 0.0
    ref_max = float(np.max(np.abs(ref))) if ref.size else 0.0
    return dict(max_abs=max_abs, ref_max=ref_max,
                scaled=max_abs / max(1.0, ref_max),
                rel=max_abs / ref_max if ref_max > 0 else (0.0 if max_abs == 0 else np.inf),
                nan=bool(np.isnan(got).any()))


def out_passes(got, ref) -> tuple[bool, dict]:
    e = out_errors(got, ref)
    ok = (not e["nan"]) and e["scaled"] <= ABS_TOL and e["rel"] <= REL_TOL
    return ok, e


def lse_passes(got, ref) -> tuple[bool, float]:
    d = float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))))
    return (d <= LSE_TOL) and not np.isnan(d), d
