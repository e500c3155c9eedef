"""Plain fp64 CPU oracle for DDTree tree-verify MLA attention (absorbed and explicit forms).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares no
code with the HIP path (``speculative_decoding_tree_parent_amd``); the two meet
only in ``synth_inputs`` (seeded numbers, no attention arithmetic).

What is computed (sources are the three pages on the DDTree engine):

* Every draft-tree candidate is scored in parallel; each attends over the KV
  cache under a visibility mask that follows the tree ("The Architecture of
  Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 2).  A node sees
  the whole prefix, its ancestors and itself: the tokens it would follow if its
  root-to-node path were accepted.
* The cache is MLA's compressed latent, ``kv_lora_rank`` latent + ``qk_rope``
  rotary elements per token per layer ("From Diagnosis to Deployment...",
  section "The Second Thread: Pivoting to 200k Context"), addressed through a
  page table with one token per page ("The Architecture of Diagnosis...",
  section "The Discrepancy That Revealed the Truth").
* The kernel "absorbs the latent projection" (same item 2 above): the per-head
  key map W_UK is applied to the query (q_lat = W_UK[h]^T q_nope) instead of to
  every cached row, and the value map W_UV is applied once to the attention
  output instead of to every row.  ``verify_mla_explicit`` computes the
  un-absorbed form (K = W_UK c, V = W_UV c materialised per head) so that the
  two can be checked against each other.

Readings where the pages are silent:
  * node 0 is the root (parent -1); parent[i] < i (topological order);
  * tree node i's own latent row sits at logical position L + i;
  * q_rope and k_pe arrive after RoPE; the softmax scale is an argument;
  * a row whose parent is out of range is invalid: its mask holds only its own
    bit and the status is KDV_ERR_TREE (-3).

All arithmetic is float64 on values that are exactly the bf16 inputs.
Steps follow the plain definition in order: visibility, gather, score matmul,
mask to -inf, subtract the row max, exp, normalise, weighted sum, up-projection.
"""
from __future__ import annotations

import numpy as np

KDV_OK = 0
KDV_ERR_TREE = -3


# ----------------------------------------------------------------------------- tree structure
def _row_is_valid(parent: np.ndarray, i: int) -> bool:
    p = int(parent[i])
    if i == 0:
        return p == -1
    return 0 <= p < i


def ancestor_path(parent, t: int) -> list[int]:
    """Nodes on the path root..t (inclusive), in root-to-node order.

    Walking stops after an invalid row (its own node is still on the path),
    matching the mask rule for malformed trees.
    """
    parent = np.asarray(parent)
    path = [t]
    j = t
    while _row_is_valid(parent, j) and j != 0:
        j = int(parent[j])
        path.append(j)
    return path[::-1]


def tree_status(parent) -> int:
    parent = np.asarray(parent)
    return KDV_OK if all(_row_is_valid(parent, i) for i in range(parent.shape[0])) else KDV_ERR_TREE


def tree_mask(parent) -> tuple[np.ndarray, int]:
    """Ancestor bitmask: bit j of row i is set iff node j lies on the root-to-i path.

    Encoding: W = ceil(T/32) uint32 words per row, bit (j % 32) of word j // 32;
    every other bit (including the padding above T) is zero.
    Returns (mask [T][W] uint32, status).
    """
    parent = np.asarray(parent)
    T = parent.shape[0]
    W = (T + 31) // 32
    mask = np.zeros((T, W), dtype=np.uint32)
    for i in range(T):
        for j in ancestor_path(parent, i):
            mask[i, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return mask, tree_status(parent)


def visibility(parent, L: int) -> np.ndarray:
    """Boolean [T][L+T]: node t sees every prefix position and L + a for a on its root path."""
    parent = np.asarray(parent)
    T = parent.shape[0]
    vis = np.zeros((T, L + T), dtype=bool)
    vis[:, :L] = True
    for t in range(T):
        for a in ancestor_path(parent, t):
            vis[t, L + a] = True
    return vis


# ----------------------------------------------------------------------------- attention
def gather_latent(c_kv, k_pe, page_table) -> tuple[np.ndarray, np.ndarray]:
    """Logical rows of the paged cache: C[n] = c_kv[page_table[n]], Kp[n] = k_pe[page_table[n]] (fp64)."""
    idx = np.asarray(page_table, dtype=np.int64)
    return np.asarray(c_kv)[idx].astype(np.float64), np.asarray(k_pe)[idx].astype(np.float64)


def _masked_softmax(scores: np.ndarray, vis: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Row softmax over the visible entries; returns (probabilities, natural-log sum of exp)."""
    s = np.where(vis, scores, -np.inf)
    mx = s.max(axis=-1, keepdims=True)
    e = np.exp(s - mx)
    tot = e.sum(axis=-1, keepdims=True)
    return e / tot, (mx + np.log(tot))[..., 0]


def verify_mla_absorbed(q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, L: int, parent, sm_scale: float,
                        heads=None, nodes=None) -> tuple[np.ndarray, np.ndarray]:
    """Tree-verify MLA attention in absorbed form.

    Shapes: q_nope [T][H][Dn], q_rope [T][H][Dr], w_uk [H][Dn][R], w_uv [H][Dv][R],
    c_kv [P][R], k_pe [P][Dr], page_table [L+T].
    Returns out [T][H][Dv] and lse [T][H] (natural log of the sum of exp of scaled
    scores); entries for heads/nodes not requested are NaN.
    """
    q_nope = np.asarray(q_nope)
    T, H, _ = q_nope.shape
    Dv = np.asarray(w_uv).shape[1]
    heads = range(H) if heads is None else heads
    nodes = np.arange(T) if nodes is None else np.asarray(nodes)
    vis = visibility(parent, L)[nodes]                              # [t][N]
    C, Kp = gather_latent(c_kv, k_pe, page_table)                   # [N][R], [N][Dr]
    out = np.full((T, H, Dv), np.nan)
    lse = np.full((T, H), np.nan)
    for h in heads:
        Wk = np.asarray(w_uk[h], dtype=np.float64)                  # [Dn][R]
        Wv = np.asarray(w_uv[h], dtype=np.float64)                  # [Dv][R]
        qn = np.asarray(q_nope[nodes, h], dtype=np.float64)         # [t][Dn]
        qr = np.asarray(q_rope[nodes, h], dtype=np.float64)         # [t][Dr]
        q_lat = qn @ Wk                                             # absorption: [t][R]
        scores = sm_scale * (q_lat @ C.T + qr @ Kp.T)               # [t][N]
        p, lse_h = _masked_softmax(scores, vis)
        o_lat = p @ C                                               # [t][R]
        out[nodes, h] = o_lat @ Wv.T                                # up-projection: [t][Dv]
        lse[nodes, h] = lse_h
    return out, lse


def verify_mla_explicit(q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, page_table, L: int, parent, sm_scale: float,
                        heads=None, nodes=None) -> tuple[np.ndarray, np.ndarray]:
    """Same attention with per-head keys and values materialised (no absorption).

    K[n] = [W_UK[h] C[n] ; Kp[n]] (Dn+Dr), V[n] = W_UV[h] C[n] (Dv), q = [q_nope ; q_rope].
    """
    q_nope = np.asarray(q_nope)
    T, H, _ = q_nope.shape
    Dv = np.asarray(w_uv).shape[1]
    heads = range(H) if heads is None else heads
    nodes = np.arange(T) if nodes is None else np.asarray(nodes)
    vis = visibility(parent, L)[nodes]
    C, Kp = gather_latent(c_kv, k_pe, page_table)
    out = np.full((T, H, Dv), np.nan)
    lse = np.full((T, H), np.nan)
    for h in heads:
        Wk = np.asarray(w_uk[h], dtype=np.float64)
        Wv = np.asarray(w_uv[h], dtype=np.float64)
        K = np.concatenate([C @ Wk.T, Kp], axis=1)                  # [N][Dn+Dr]
        V = C @ Wv.T                                                # [N][Dv]
        q = np.concatenate([np.asarray(q_nope[nodes, h], dtype=np.float64),
                            np.asarray(q_rope[nodes, h], dtype=np.float64)], axis=1)
        p, lse_h = _masked_softmax(sm_scale * (q @ K.T), vis)
        out[nodes, h] = p @ V
        lse[nodes, h] = lse_h
    return out, lse


def verify_inputs(inp, form: str = "absorbed", heads=None, nodes=None):
    """Run the oracle on a ``synth_inputs.VerifyInputs`` (bf16 values widened exactly)."""
    fn = verify_mla_absorbed if form == "absorbed" else verify_mla_explicit
    return fn(inp.f32("q_nope"), inp.f32("q_rope"), inp.f32("w_uk"), inp.f32("w_uv"), inp.f32("c_kv"),
              inp.f32("k_pe"), inp.page_table, inp.L, inp.parent, inp.sm_scale, heads=heads, nodes=nodes)
