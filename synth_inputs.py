"""Seeded synthetic inputs for DDTree tree-verify MLA attention.

This module is the only code shared by the oracle (``oracle/``) and the HIP
path's tests and benchmark.  It draws numbers and lays them out; it holds none
of the attention arithmetic.

Workload shapes follow the pages' problem statement: the MLA latent cache holds
``kv_lora_rank`` (512) latent plus ``qk_rope`` (64) rotary elements per token
per layer ("From Diagnosis to Deployment...", section "The Second Thread:
Pivoting to 200k Context"), draft trees have 9-15 nodes and contexts of
13/1663/3333/5553 tokens ("From Diagnosis to Deployment...", section "The
Controlled Experiment That Changed Everything", context-sweep table), and the
cache is paged with one token per page ("The Architecture of Diagnosis...",
section "The Discrepancy That Revealed the Truth").  The pages run no public
dataset; every value here is drawn from a seeded normal distribution.

Draw order (fixed, one ``numpy.random.default_rng(seed)`` stream):
parent, q_nope, q_rope, W_UK, W_UV, c_kv, k_pe, page_table.
Values are drawn in float32 and rounded to bfloat16 with round-to-nearest-even,
the same rounding ``torch.Tensor.to(torch.bfloat16)`` applies.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

KIMI_DIMS = dict(num_heads=64, qk_nope_dim=128, qk_rope_dim=64, kv_lora_rank=512, v_head_dim=128)
TINY_DIMS = dict(num_heads=4, qk_nope_dim=32, qk_rope_dim=16, kv_lora_rank=64, v_head_dim=32)

DISTRIBUTIONS = ("literal", "unit", "peak4")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_u.size, step):
        c = flat_u[s:s + step].astype(np.uint64)
        r = (c + 0x7FFF + ((c >> 16) & 1)) >> 16
        nan = (c & 0x7FFFFFFF) > 0x7F800000
        r = np.where(nan, 0x7FC0, r)
        flat_o[s:s + step] = r.astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def random_parents(rng: np.random.Generator, T: int, depth_cap: int | None = None) -> np.ndarray:
    """Random recursive tree in topological order: parent[0] = -1, parent[i] ~ U{0..i-1}.

    With ``depth_cap`` (the longest root-to-node path, in nodes) the parent is
    drawn uniformly among earlier nodes whose depth leaves room for a child.
    """
    parent = np.full(T, -1, dtype=np.int32)
    if T <= 1:
        return parent
    if depth_cap is None:
        parent[1:] = rng.integers(0, np.arange(1, T)).astype(np.int32)
        return parent
    depth = np.zeros(T, dtype=np.int64)
    for i in range(1, T):
        cand = np.flatnonzero(depth[:i] < depth_cap - 1)
        p = int(cand[rng.integers(0, cand.size)])
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def accept_inputs(seed: int, T: int, vocab: int = 32000, follow: float = 0.7, dup: float = 0.0,
                  parent=None) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Seeded (parent, draft tokens, target predictions) for the tree-accept step; int32 arrays of length T.

    A random recursive tree (unless ``parent`` is given) with uniform draft tokens; with probability ``dup``
    a node copies an earlier sibling's token.  The target's prediction at a node is, with probability
    ``follow``, the draft token of one of its children drawn uniformly (so drafts get accepted), otherwise
    a uniform token.  Draw order: parent, tokens, duplicate choices, predictions.
    """
    rng = np.random.default_rng(seed)
    par = random_parents(rng, T) if parent is None else np.asarray(parent, dtype=np.int32)
    tok = rng.integers(0, vocab, size=T).astype(np.int32)
    for i in range(1, T):
        sib = [j for j in range(1, i) if par[j] == par[i]]
        if sib and rng.random() < dup:
            tok[i] = tok[sib[int(rng.integers(0, len(sib)))]]
    pred = rng.integers(0, vocab, size=T).astype(np.int32)
    for p in range(T):
        kids = [c for c in range(T) if par[c] == p]
        if kids and rng.random() < follow:
            pred[p] = tok[kids[int(rng.integers(0, len(kids)))]]
    return par, tok, pred


def draft_topk(seed: int, block: int, K: int, vocab: int = 32000, ties: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """Seeded drafter output for tree construction: (logp float32 [block][K], tok int32 [block][K]).

    Each position's K log-probabilities are drawn as minus exponential variates and sorted in decreasing
    order; with ``ties`` they are rounded to multiples of 1/4 so that equal scores occur.  Tokens are distinct
    within a position.  Draw order: log-probabilities, then tokens, position by position.
    """
    rng = np.random.default_rng(seed)
    logp = np.empty((block, K), dtype=np.float32)
    tok = np.empty((block, K), dtype=np.int32)
    for d in range(block):
        v = -rng.exponential(1.5, size=K)
        if ties:
            v = np.round(v * 4.0) / 4.0
        logp[d] = np.sort(v)[::-1].astype(np.float32)
    for d in range(block):
        tok[d] = rng.choice(vocab, size=K, replace=False).astype(np.int32)
    return logp, tok


@dataclass
class VerifyInputs:
    """One layer's worth of tree-verify inputs (bf16 bit patterns + their exact float32 values)."""
    H: int
    Dn: int
    Dr: int
    R: int
    Dv: int
    L: int
    T: int
    sm_scale: float
    parent: np.ndarray          # int32 [T]
    q_nope: np.ndarray          # uint16 bf16 [T][H][Dn]
    q_rope: np.ndarray          # uint16 bf16 [T][H][Dr]
    w_uk: np.ndarray            # uint16 bf16 [H][Dn][R]  (k_nope = W_UK[h] @ c)
    w_uv: np.ndarray            # uint16 bf16 [H][Dv][R]  (v = W_UV[h] @ c)
    c_kv: np.ndarray            # uint16 bf16 [P][R]
    k_pe: np.ndarray            # uint16 bf16 [P][Dr]
    page_table: np.ndarray      # int32 [L+T]
    seed: int = 0
    dist: str = "literal"
    _f32: dict = field(default_factory=dict, repr=False)

    @property
    def N(self) -> int:
        return self.L + self.T

    @property
    def pool_slots(self) -> int:
        return int(self.c_kv.shape[0])

    def f32(self, name: str) -> np.ndarray:
        """Exact float32 view of a bf16 input (cached)."""
        if name not in self._f32:
            self._f32[name] = bf16_bits_to_f32(getattr(self, name))
        return self._f32[name]

    def dims(self) -> dict:
        return dict(num_heads=self.H, qk_nope_dim=self.Dn, qk_rope_dim=self.Dr,
                    kv_lora_rank=self.R, v_head_dim=self.Dv, sm_scale=self.sm_scale)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def make_inputs(*, num_heads: int, qk_nope_dim: int, qk_rope_dim: int, kv_lora_rank: int, v_head_dim: int,
                L: int, T: int, seed: int = 0, parent=None, pool_slots: int | None = None,
                dist: str = "literal", poison_unused: bool = False, depth_cap: int | None = None,
                sm_scale: float | None = None) -> VerifyInputs:
    """Draw one layer of inputs.

    dist:
      "literal": weights N(0,1)/sqrt(kv_lora_rank); each activation N(0,1)/sqrt(its own last dim).
      "unit":    q, c_kv, k_pe ~ N(0,1); weights N(0,1)/sqrt(kv_lora_rank)  (score std ~1 at the Kimi shape).
      "peak4":   "unit" with both query parts multiplied by 4 (score std ~4, peaked softmax).
    pool_slots: None -> contiguous cache (pool of exactly L+T rows, identity page table);
                else page_table = first L+T entries of a random permutation of the pool.
    poison_unused: pool rows no page-table entry refers to are set to bf16 NaN.
    """
    if dist not in DISTRIBUTIONS:
        raise ValueError(f"unknown distribution {dist!r}")
    H, Dn, Dr, R, Dv = num_heads, qk_nope_dim, qk_rope_dim, kv_lora_rank, v_head_dim
    N = L + T
    rng = np.random.default_rng(seed)
    # 1. parent
    if parent is None:
        par = random_parents(rng, T, depth_cap)
    else:
        par = np.asarray(parent, dtype=np.int32).copy()
        if par.shape != (T,):
            raise ValueError("parent must have T entries")
    # 2-7. values
    if dist == "literal":
        s_qn, s_qr, s_c, s_kp = 1 / math.sqrt(Dn), 1 / math.sqrt(Dr), 1 / math.sqrt(R), 1 / math.sqrt(Dr)
    else:
        s_qn = s_qr = s_c = s_kp = 1.0
        if dist == "peak4":
            s_qn = s_qr = 4.0
    s_w = 1 / math.sqrt(R)
    P = N if pool_slots is None else int(pool_slots)
    if P < N:
        raise ValueError("pool smaller than L+T")
    q_nope = f32_to_bf16_bits(_normal(rng, (T, H, Dn), s_qn))
    q_rope = f32_to_bf16_bits(_normal(rng, (T, H, Dr), s_qr))
    w_uk = f32_to_bf16_bits(_normal(rng, (H, Dn, R), s_w))
    w_uv = f32_to_bf16_bits(_normal(rng, (H, Dv, R), s_w))
    c_kv = f32_to_bf16_bits(_normal(rng, (P, R), s_c))
    k_pe = f32_to_bf16_bits(_normal(rng, (P, Dr), s_kp))
    # 8. page table
    if pool_slots is None:
        page_table = np.arange(N, dtype=np.int32)
    else:
        page_table = rng.permutation(P)[:N].astype(np.int32)
    if poison_unused and P > N:
        unused = np.ones(P, dtype=bool)
        unused[page_table] = False
        c_kv[unused] = BF16_NAN
        k_pe[unused] = BF16_NAN
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(Dn + Dr)
    return VerifyInputs(H=H, Dn=Dn, Dr=Dr, R=R, Dv=Dv, L=L, T=T, sm_scale=float(sm_scale), parent=par,
                        q_nope=q_nope, q_rope=q_rope, w_uk=w_uk, w_uv=w_uv, c_kv=c_kv, k_pe=k_pe,
                        page_table=page_table, seed=seed, dist=dist)


def batch_inputs(dims: dict, Ls, Ts, seed: int = 0, dist: str = "literal", pool_slots: int | None = None,
                 parents=None) -> list[VerifyInputs]:
    """C requests of one layer: shared weights and latent pool, each request with its own queries, tree and page
    table (disjoint pool slots, drawn as one permutation of the pool).

    The shared arrays come from make_inputs(L=Ls[0], T=Ts[0], seed, pool_slots=P); request c's parent and
    queries are drawn from default_rng([seed, c + 1]) in the order parent, q_nope, q_rope, with the scales of
    `dist`.  Each returned VerifyInputs describes one request and refers to the shared arrays."""
    C = len(Ls)
    if len(Ts) != C or C < 1:
        raise ValueError("Ls and Ts must have the same length >= 1")
    total = int(sum(int(L) + int(T) for L, T in zip(Ls, Ts)))
    P = total if pool_slots is None else int(pool_slots)
    if P < total:
        raise ValueError("pool smaller than the requests' rows")
    base = make_inputs(**dims, L=int(Ls[0]), T=int(Ts[0]), seed=seed, dist=dist, pool_slots=P)
    H, Dn, Dr = base.H, base.Dn, base.Dr
    if dist == "literal":
        s_qn, s_qr = 1 / math.sqrt(Dn), 1 / math.sqrt(Dr)
    else:
        s_qn = s_qr = 4.0 if dist == "peak4" else 1.0
    perm = np.random.default_rng([seed, 0]).permutation(P)[:total].astype(np.int32)
    reqs, off = [], 0
    for c in range(C):
        L, T = int(Ls[c]), int(Ts[c])
        rng = np.random.default_rng([seed, c + 1])
        par = random_parents(rng, T) if parents is None else np.asarray(parents[c], dtype=np.int32).copy()
        q_nope = f32_to_bf16_bits(_normal(rng, (T, H, Dn), s_qn))
        q_rope = f32_to_bf16_bits(_normal(rng, (T, H, Dr), s_qr))
        reqs.append(VerifyInputs(H=H, Dn=Dn, Dr=Dr, R=base.R, Dv=base.Dv, L=L, T=T, sm_scale=base.sm_scale,
                                 parent=par, q_nope=q_nope, q_rope=q_rope, w_uk=base.w_uk, w_uv=base.w_uv,
                                 c_kv=base.c_kv, k_pe=base.k_pe, page_table=perm[off:off + L + T].copy(),
                                 seed=seed, dist=dist))
        off += L + T
    return reqs


# Named workloads (the shapes of the pages' verify workloads).
def tiny(seed: int = 0, dist: str = "literal", **kw) -> VerifyInputs:
    """4 heads, 32/16/64/32 dims, 128-token contiguous prefix, 7-node full binary tree."""
    args = dict(TINY_DIMS, L=128, T=7, seed=seed, parent=[-1, 0, 0, 1, 1, 2, 2], dist=dist)
    args.update(kw)
    return make_inputs(**args)


def kimi(L: int = 5553, T: int = 15, seed: int = 0, dist: str = "literal", **kw) -> VerifyInputs:
    """64 heads, 128/64/512/128 dims, random recursive tree, contiguous cache unless pool_slots given."""
    args = dict(KIMI_DIMS, L=L, T=T, seed=seed, dist=dist)
    args.update(kw)
    return make_inputs(**args)


def long_fragmented(seed: int = 0, dist: str = "literal", L: int = 200000, T: int = 15,
                    pool_slots: int = 262144, **kw) -> VerifyInputs:
    """64 heads, 200k-token prefix scattered over a 262144-slot pool (page_size = 1)."""
    return kimi(L=L, T=T, seed=seed, dist=dist, pool_slots=pool_slots, **kw)


FULL61_LAYERS = 61
FULL61_SHAPE = dict(num_heads=8, qk_nope_dim=128, qk_rope_dim=64, kv_lora_rank=512, v_head_dim=128)


def full61_shared(seed: int = 999, L: int = 131072, T: int = 32, pool_slots: int = 262144, depth_cap: int = 16):
    """Parent array and page table shared by all 61 layers of one verify step (8 heads per layer)."""
    rng = np.random.default_rng(seed)
    parent = random_parents(rng, T, depth_cap)
    page_table = rng.permutation(pool_slots)[:L + T].astype(np.int32)
    return parent, page_table


def full61_layer(layer: int, parent: np.ndarray, page_table: np.ndarray, L: int = 131072, T: int = 32,
                 pool_slots: int = 262144, dist: str = "literal") -> VerifyInputs:
    """One layer of the 61-layer verify step: per-layer seed 1000 + layer, shared parent and page table."""
    inp = make_inputs(**FULL61_SHAPE, L=L, T=T, seed=1000 + layer, parent=parent, pool_slots=pool_slots,
                      dist=dist)
    inp.page_table = np.asarray(page_table, dtype=np.int32).copy()
    return inp


def to_device(inp: VerifyInputs, device="cuda") -> dict:
    """Copy one layer's inputs to device tensors (bf16 bit patterns as int16; indices as int32)."""
    import torch

    def b16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)

    return dict(parent=torch.from_numpy(inp.parent.astype(np.int32)).to(device),
                q_nope=b16(inp.q_nope), q_rope=b16(inp.q_rope), w_uk=b16(inp.w_uk), w_uv=b16(inp.w_uv),
                c_kv=b16(inp.c_kv), k_pe=b16(inp.k_pe),
                page_table=torch.from_numpy(inp.page_table.astype(np.int32)).to(device))
