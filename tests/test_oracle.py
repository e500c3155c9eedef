"""Pins for the fp64 oracle, against facts that do not come from the oracle itself.

* worked examples derived by hand (tests/golden/*.json);
* closed forms (chain / star masks, uniform scores, L = 0 root);
* an algebraic identity (absorbed == explicit per-head K/V);
* brute force: ordinary causal attention over the explicit sequence prefix + root-to-node path;
* a library routine: torch scaled_dot_product_attention in float64 for chain trees and T = 1;
* invariants (mask rules, page-table permutation, scale equivalence);
* mutation: a mask planted wrong in the oracle fails the parity criterion.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import ref as oref
import synth_inputs as si
from tests.parity import out_passes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ------------------------------------------------------------------ mask
def test_mask_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "tiny_tree_mask.json")))
    mask, status = oracle.tree_mask(g["parent"])
    assert status == oracle.KDV_OK
    assert mask.shape == (7, 1)
    assert mask[:, 0].tolist() == g["mask"]


def _depth_by_walk(parent, i):
    d = 0
    while parent[i] != -1:
        i = parent[i]
        d += 1
    return d


@pytest.mark.parametrize("T", [1, 2, 7, 9, 15, 31, 32, 33, 63, 64])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mask_invariants_random_trees(T, seed):
    rng = np.random.default_rng(seed)
    parent = si.random_parents(rng, T)
    mask, status = oracle.tree_mask(parent)
    assert status == oracle.KDV_OK
    W = (T + 31) // 32
    assert mask.shape == (T, W) and mask.dtype == np.uint32
    bits = np.zeros((T, 32 * W), dtype=bool)
    for i in range(T):
        for w in range(W):
            for b in range(32):
                bits[i, 32 * w + b] = (int(mask[i, w]) >> b) & 1
    for i in range(T):
        assert bits[i, i]                                   # self
        assert bits[i, 0]                                   # root
        assert not bits[i, T:].any()                        # padding bits clear
        assert not bits[i, i + 1:].any()                    # topological order: no later node
        assert bits[i].sum() == _depth_by_walk(parent, i) + 1
        if i > 0:
            expect = bits[parent[i]].copy()
            expect[i] = True
            assert (bits[i] == expect).all()                # row i = row parent[i] | bit i


@pytest.mark.parametrize("T", [1, 5, 32, 33, 64])
def test_mask_closed_forms(T):
    chain = np.arange(-1, T - 1, dtype=np.int32)
    mask, _ = oracle.tree_mask(chain)
    for i in range(T):
        full = (1 << (i + 1)) - 1                           # bits 0..i
        got = sum(int(mask[i, w]) << (32 * w) for w in range(mask.shape[1]))
        assert got == full
    star = np.zeros(T, dtype=np.int32)
    star[0] = -1
    mask, _ = oracle.tree_mask(star)
    for i in range(T):
        got = sum(int(mask[i, w]) << (32 * w) for w in range(mask.shape[1]))
        assert got == (1 | (1 << i))


def test_mask_invalid_parents():
    # parent[0] != -1 -> row 0 invalid; parent[2] = 2 (not < 2) -> invalid; row 3 hangs off row 2.
    parent = np.array([0, 0, 2, 2, 1], dtype=np.int32)
    mask, status = oracle.tree_mask(parent)
    assert status == oracle.KDV_ERR_TREE
    assert mask[:, 0].tolist() == [0b1, 0b11, 0b100, 0b1100, 0b10011]
    parent = np.array([-1, 0, -1, 7], dtype=np.int32)       # parent[2] = -1 and parent[3] = 7 invalid
    mask, status = oracle.tree_mask(parent)
    assert status == oracle.KDV_ERR_TREE
    assert mask[:, 0].tolist() == [1, 3, 4, 8]


# ------------------------------------------------------------------ attention: hand example
def test_hand_worked_attention():
    g = json.load(open(os.path.join(GOLDEN, "hand_attention.json")))
    d = g["dims"]
    H, T, L = d["H"], d["T"], d["L"]
    ln = math.log
    c_logical = [0.0, ln(2), ln(3), ln(5)]
    kp_logical = [ln(4), 0.0, 0.0, ln(2)]
    P = 6
    c_kv = np.full((P, 1), np.nan)
    k_pe = np.full((P, 1), np.nan)
    for n, slot in enumerate(g["page_table"]):
        c_kv[slot, 0] = c_logical[n]
        k_pe[slot, 0] = kp_logical[n]
    q_nope = np.ones((T, H, 1))
    q_rope = np.zeros((T, H, 1))
    q_rope[:, 1, 0] = 1.0
    w_uk = np.array(g["w_uk"], dtype=np.float64)
    w_uv = np.array(g["w_uv"], dtype=np.float64)
    for fn in (oracle.verify_mla_absorbed, oracle.verify_mla_explicit):
        out, lse = fn(q_nope, q_rope, w_uk, w_uv, c_kv, k_pe, np.array(g["page_table"]), L, g["parent"],
                      d["sm_scale"])
        np.testing.assert_allclose(out[:, :, 0], np.array(g["expected_out"]), rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.array(g["expected_lse"]), rtol=0, atol=1e-13)


# ------------------------------------------------------------------ attention: brute force over paths
def _brute_force(inp, heads, nodes):
    """Ordinary causal attention: node t's query is the last position of the explicit sequence
    prefix rows + rows of its root..t path; K, V are materialised per head (no mask, no absorption)."""
    c = inp.f32("c_kv").astype(np.float64)
    kp = inp.f32("k_pe").astype(np.float64)
    qn = inp.f32("q_nope").astype(np.float64)
    qr = inp.f32("q_rope").astype(np.float64)
    wk = inp.f32("w_uk").astype(np.float64)
    wv = inp.f32("w_uv").astype(np.float64)
    out = {}
    for t in nodes:
        path = [t]
        while inp.parent[path[-1]] != -1:
            path.append(int(inp.parent[path[-1]]))
        path.reverse()
        seq = list(range(inp.L)) + [inp.L + a for a in path]
        slots = [int(inp.page_table[n]) for n in seq]
        for h in heads:
            K = np.array([np.concatenate([wk[h] @ c[s], kp[s]]) for s in slots])
            V = np.array([wv[h] @ c[s] for s in slots])
            q = np.concatenate([qn[t, h], qr[t, h]])
            s = inp.sm_scale * (K @ q)
            m = s.max()
            e = np.exp(s - m)
            out[(t, h)] = ((e / e.sum()) @ V, m + math.log(e.sum()))
    return out


@pytest.mark.parametrize("dist", ["literal", "unit", "peak4"])
def test_brute_force_tiny(dist):
    inp = si.tiny(seed=0, dist=dist)
    out, lse = oracle.verify_inputs(inp)
    bf = _brute_force(inp, range(inp.H), range(inp.T))
    for (t, h), (o, l) in bf.items():
        np.testing.assert_allclose(out[t, h], o, rtol=1e-10, atol=1e-12)
        assert abs(lse[t, h] - l) < 1e-10


@pytest.mark.parametrize("L", [0, 13])
def test_brute_force_kimi_shape(L):
    inp = si.kimi(L=L, T=15, seed=3, dist="unit")
    heads = [0, 17, 63]
    out, lse = oracle.verify_inputs(inp, heads=heads)
    bf = _brute_force(inp, heads, range(inp.T))
    for (t, h), (o, l) in bf.items():
        np.testing.assert_allclose(out[t, h], o, rtol=1e-10, atol=1e-12)
        assert abs(lse[t, h] - l) < 1e-10


def test_brute_force_permuted_pool():
    inp = si.tiny(seed=5, dist="unit", pool_slots=300, poison_unused=True)
    out, lse = oracle.verify_inputs(inp)
    assert not np.isnan(out).any()
    bf = _brute_force(inp, range(inp.H), range(inp.T))
    for (t, h), (o, l) in bf.items():
        np.testing.assert_allclose(out[t, h], o, rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------ algebraic identity
@pytest.mark.parametrize("maker,kw", [(si.tiny, dict(dist="literal")), (si.tiny, dict(dist="peak4")),
                                      (si.kimi, dict(L=200, T=9, dist="unit"))])
def test_absorbed_equals_explicit(maker, kw):
    inp = maker(seed=1, **kw)
    heads = None if inp.H <= 4 else [0, 5, 63]
    a, la = oracle.verify_inputs(inp, "absorbed", heads=heads)
    b, lb = oracle.verify_inputs(inp, "explicit", heads=heads)
    sel = ~np.isnan(a)
    scale = np.max(np.abs(b[sel]))
    assert np.max(np.abs(a[sel] - b[sel])) <= 1e-10 * scale
    np.testing.assert_allclose(la[~np.isnan(la)], lb[~np.isnan(lb)], rtol=0, atol=1e-10)


# ------------------------------------------------------------------ library routine: SDPA
def _explicit_qkv(inp, h):
    c = torch.from_numpy(inp.f32("c_kv").astype(np.float64))[torch.from_numpy(inp.page_table.astype(np.int64))]
    kp = torch.from_numpy(inp.f32("k_pe").astype(np.float64))[torch.from_numpy(inp.page_table.astype(np.int64))]
    wk = torch.from_numpy(inp.f32("w_uk")[h].astype(np.float64))
    wv = torch.from_numpy(inp.f32("w_uv")[h].astype(np.float64))
    K = torch.cat([c @ wk.T, kp], dim=1)
    V = c @ wv.T
    q = torch.cat([torch.from_numpy(inp.f32("q_nope")[:, h].astype(np.float64)),
                   torch.from_numpy(inp.f32("q_rope")[:, h].astype(np.float64))], dim=1)
    return q, K, V


@pytest.mark.parametrize("T,L", [(1, 0), (1, 37), (7, 0), (15, 50)])
def test_chain_tree_matches_sdpa(T, L):
    inp = si.make_inputs(**si.TINY_DIMS, L=L, T=T, seed=4, dist="unit", parent=np.arange(-1, T - 1))
    out, _ = oracle.verify_inputs(inp)
    for h in range(inp.H):
        q, K, V = _explicit_qkv(inp, h)
        # chain tree == causal attention of T queries appended after L keys
        allowed = torch.ones(T, L + T, dtype=torch.bool)
        allowed[:, L:] = torch.tril(torch.ones(T, T, dtype=torch.bool))
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None], V[None], attn_mask=allowed[None],
                                                               scale=inp.sm_scale)[0]
        np.testing.assert_allclose(out[:, h], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_star_tree_sees_prefix_root_self():
    T, L = 9, 21
    parent = np.zeros(T, dtype=np.int32)
    parent[0] = -1
    inp = si.make_inputs(**si.TINY_DIMS, L=L, T=T, seed=6, dist="unit", parent=parent)
    out, _ = oracle.verify_inputs(inp)
    for h in range(inp.H):
        q, K, V = _explicit_qkv(inp, h)
        allowed = torch.zeros(T, L + T, dtype=torch.bool)
        allowed[:, :L] = True
        allowed[:, L] = True
        allowed[torch.arange(T), L + torch.arange(T)] = True
        ref = torch.nn.functional.scaled_dot_product_attention(q[None], K[None], V[None], attn_mask=allowed[None],
                                                               scale=inp.sm_scale)[0]
        np.testing.assert_allclose(out[:, h], ref.numpy(), rtol=1e-10, atol=1e-12)


# ------------------------------------------------------------------ closed forms
def test_root_with_empty_prefix_is_its_own_value():
    # L = 0: the root sees only itself, so out = W_UV c_root and lse = its own score.
    inp = si.kimi(L=0, T=9, seed=7, dist="unit")
    out, lse = oracle.verify_inputs(inp, heads=[0, 1, 40])
    c0 = inp.f32("c_kv")[inp.page_table[0]].astype(np.float64)
    k0 = inp.f32("k_pe")[inp.page_table[0]].astype(np.float64)
    for h in [0, 1, 40]:
        wv = inp.f32("w_uv")[h].astype(np.float64)
        wk = inp.f32("w_uk")[h].astype(np.float64)
        np.testing.assert_allclose(out[0, h], wv @ c0, rtol=1e-12, atol=1e-14)
        s = inp.sm_scale * (inp.f32("q_nope")[0, h] @ (wk @ c0) + inp.f32("q_rope")[0, h] @ k0)
        assert abs(lse[0, h] - s) < 1e-10


def test_zero_query_gives_uniform_average():
    # q = 0 -> every visible row gets weight 1/n_t: out = W_UV mean(c_vis), lse = ln(n_t).
    inp = si.tiny(seed=8, dist="unit")
    z = np.zeros_like(inp.f32("q_nope"))
    zr = np.zeros_like(inp.f32("q_rope"))
    out, lse = oracle.verify_mla_absorbed(z, zr, inp.f32("w_uk"), inp.f32("w_uv"), inp.f32("c_kv"),
                                          inp.f32("k_pe"), inp.page_table, inp.L, inp.parent, inp.sm_scale)
    c = inp.f32("c_kv").astype(np.float64)
    depth = [0, 1, 1, 2, 2, 2, 2]
    paths = [[0], [0, 1], [0, 2], [0, 1, 3], [0, 1, 4], [0, 2, 5], [0, 2, 6]]
    for t in range(inp.T):
        rows = list(range(inp.L)) + [inp.L + a for a in paths[t]]
        n_t = inp.L + depth[t] + 1
        assert len(rows) == n_t
        mean_c = c[inp.page_table[rows]].mean(axis=0)
        for h in range(inp.H):
            np.testing.assert_allclose(out[t, h], inp.f32("w_uv")[h].astype(np.float64) @ mean_c, rtol=1e-12,
                                       atol=1e-14)
            assert abs(lse[t, h] - math.log(n_t)) < 1e-12


# ------------------------------------------------------------------ invariants
def test_page_permutation_invariance():
    a = si.tiny(seed=9, dist="unit")
    rng = np.random.default_rng(123)
    P = 500
    slots = rng.permutation(P)[:a.N]
    b_ckv = np.zeros((P, a.R), dtype=np.uint16)
    b_kpe = np.zeros((P, a.Dr), dtype=np.uint16)
    b_ckv[slots] = a.c_kv[a.page_table]
    b_kpe[slots] = a.k_pe[a.page_table]
    out_a, lse_a = oracle.verify_inputs(a)
    out_b, lse_b = oracle.verify_mla_absorbed(a.f32("q_nope"), a.f32("q_rope"), a.f32("w_uk"), a.f32("w_uv"),
                                              si.bf16_bits_to_f32(b_ckv), si.bf16_bits_to_f32(b_kpe),
                                              slots.astype(np.int32), a.L, a.parent, a.sm_scale)
    assert np.array_equal(out_a, out_b) and np.array_equal(lse_a, lse_b)


def test_scale_equivalence():
    inp = si.tiny(seed=10, dist="unit")
    out1, _ = oracle.verify_mla_absorbed(2 * inp.f32("q_nope"), 2 * inp.f32("q_rope"), inp.f32("w_uk"),
                                         inp.f32("w_uv"), inp.f32("c_kv"), inp.f32("k_pe"), inp.page_table, inp.L,
                                         inp.parent, inp.sm_scale)
    out2, _ = oracle.verify_mla_absorbed(inp.f32("q_nope"), inp.f32("q_rope"), inp.f32("w_uk"), inp.f32("w_uv"),
                                         inp.f32("c_kv"), inp.f32("k_pe"), inp.page_table, inp.L, inp.parent,
                                         2 * inp.sm_scale)
    np.testing.assert_allclose(out1, out2, rtol=1e-12, atol=1e-14)


def test_input_generator_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    bits = si.f32_to_bf16_bits(x)
    assert np.array_equal(bits, torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    assert np.array_equal(si.bf16_bits_to_f32(bits), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


# ------------------------------------------------------------------ mutation: the criterion catches a wrong mask
@pytest.mark.parametrize("L", [0, 13])
@pytest.mark.parametrize("mutation", ["drop_root_of_deepest", "add_non_ancestor"])
def test_mask_mutation_fails_parity(L, mutation, monkeypatch):
    inp = si.kimi(L=L, T=15, seed=11, dist="unit")
    heads = [0, 31]
    good, _ = oracle.verify_inputs(inp, heads=heads)
    depth = np.array([len(oracle.ancestor_path(inp.parent, t)) for t in range(inp.T)])
    deepest = int(np.argmax(depth))
    real = oref.visibility

    def mutated(parent, L_):
        vis = real(parent, L_).copy()
        if mutation == "drop_root_of_deepest":
            vis[deepest, L_ + 0] = False
        else:
            anc = set(oracle.ancestor_path(parent, deepest))
            j = next(j for j in range(len(parent)) if j not in anc)
            vis[deepest, L_ + j] = True
        return vis

    monkeypatch.setattr(oref, "visibility", mutated)
    bad, _ = oracle.verify_inputs(inp, heads=heads)
    ok, err = out_passes(bad[:, heads], good[:, heads])
    assert not ok, f"mutated mask passed parity: {err}"
