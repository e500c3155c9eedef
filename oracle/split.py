"""Oracle for the split verify step: prefix attention, and the merge of two partial attention results.

TEST INFRASTRUCTURE ONLY (same rules as ``oracle/ref.py``): used by ``tests/``, never by the product package.

The pages' production arrangement hands the long prefix to a dense MLA decode kernel and only the small tree
tail to the tree kernel ("The Three Acts of Engineering: Diagnosis, Extension, and Analytical Pivot in a
Speculative Decoding Stack", section "References", item [1]).  The pages do not say how the two results are
joined; the reading taken here is the standard one for a softmax split over disjoint position sets: each
part carries the natural-log sum of exp of its scores (lse), and

    M = max(lse_a, lse_b),  w_x = exp(lse_x - M),
    out = (w_a out_a + w_b out_b) / (w_a + w_b),  lse = M + ln(w_a + w_b).

A part that saw no position has lse = -inf and weight 0; two such parts give out = 0, lse = -inf.
All arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

from .ref import gather_latent


def prefix_mla_absorbed(q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, L: int, sm_scale: float,
                        heads=None) -> tuple[np.ndarray, np.ndarray]:
    """Every (node, head) row attends to the L prefix positions page_table[0..L-1] and nothing else.

    Absorbed form as in ``ref.verify_mla_absorbed`` (q_lat = q_nope W_UK[h], out = W_UV[h] o_lat); no mask.
    Returns out [T][H][Dv] and lse [T][H]; heads not requested are NaN."""
    q_nope = np.asarray(q_nope)
    T, H, _ = q_nope.shape
    Dv = np.asarray(w_uv).shape[1]
    heads = range(H) if heads is None else heads
    C, Kp = gather_latent(c_kv, k_pe, np.asarray(page_table)[:L])   # [L][R], [L][Dr]
    out = np.full((T, H, Dv), np.nan)
    lse = np.full((T, H), np.nan)
    for h in heads:
        q_lat = np.asarray(q_nope[:, h], dtype=np.float64) @ np.asarray(w_uk[h], dtype=np.float64)
        s = sm_scale * (q_lat @ C.T + np.asarray(q_rope[:, h], dtype=np.float64) @ Kp.T)   # [T][L]
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        tot = e.sum(axis=1, keepdims=True)
        out[:, h] = ((e / tot) @ C) @ np.asarray(w_uv[h], dtype=np.float64).T
        lse[:, h] = (mx + np.log(tot))[:, 0]
    return out, lse


def merge_attn_states(out_a, lse_a, out_b, lse_b) -> tuple[np.ndarray, np.ndarray]:
    """Join two attention results over disjoint position sets (formula in the module docstring).

    out_x: [..., Dv]; lse_x: [...].  Returns (out, lse) in float64."""
    oa = np.asarray(out_a, dtype=np.float64)
    ob = np.asarray(out_b, dtype=np.float64)
    la = np.asarray(lse_a, dtype=np.float64)
    lb = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(la, lb)
    empty = m == -np.inf
    ms = np.where(empty, 0.0, m)
    wa = np.where(empty, 0.0, np.exp(la - ms))
    wb = np.where(empty, 0.0, np.exp(lb - ms))
    den = wa + wb
    safe = np.where(empty, 1.0, den)
    out = np.where(empty[..., None], 0.0, (wa[..., None] * oa + wb[..., None] * ob) / safe[..., None])
    lse = np.where(empty, -np.inf, ms + np.log(safe))
    return out, lse
