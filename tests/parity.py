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
BF16_U = 2.0 ** -8          # unit roundoff of bfloat16 (8 significant bits)
LSE_SLACK = 1e-3            # fp32 accumulation, exp2/log2 and split-merge rounding


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


def lse_tolerance(inp, heads=None) -> np.ndarray:
    """Per (node, head) bound on |lse_gpu - lse_ref| [T][H].

    The device rounds the absorbed query q_lat = W_UK^T q_nope to bfloat16 before the score MFMA (the other
    score operands are exact bf16 inputs).  That moves each score s_n by at most
    u * scale * sum_i |q_lat_i| |c_n,i| with u = 2^-8, and lse = ln sum exp(s) is 1-Lipschitz in the
    max-norm of s, so the same quantity, maximised over n, bounds the lse error; LSE_SLACK covers the fp32
    parts.  Rows over all cached positions bound the visible ones."""
    T, H = inp.T, inp.H
    heads = range(H) if heads is None else heads
    C = np.abs(inp.f32("c_kv")[inp.page_table].astype(np.float64))
    tol = np.full((T, H), np.nan)
    for h in heads:
        qlat = np.abs(inp.f32("q_nope")[:, h].astype(np.float64) @ inp.f32("w_uk")[h].astype(np.float64))
        tol[:, h] = BF16_U * inp.sm_scale * (qlat @ C.T).max(axis=1) + LSE_SLACK
    return tol


def lse_passes(got, ref, tol) -> tuple[bool, float]:
    """|diff| within the per-row bound everywhere; returns (ok, max |diff| / bound)."""
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    ratio = float(np.max(d / np.asarray(tol)))
    return (ratio <= 1.0) and not np.isnan(ratio), ratio
