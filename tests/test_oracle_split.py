"""Pins for the split-step oracle (oracle/split.py): prefix attention and the merge of two partial results.

* identity: merging the prefix part with the tree-tail part reproduces the whole-cache verify attention
  (oracle/ref.py, itself pinned in tests/test_oracle.py);
* library routines: the prefix part equals a per-row softmax / logsumexp from scipy over explicitly
  materialised per-head keys and values; two single-position parts merge into scipy's two-way softmax and
  numpy's logaddexp;
* special cases: an empty part (lse = -inf) leaves the other untouched; two empty parts give 0 and -inf;
* invariants: the merge is symmetric and associative;
* mutation: a merge that ignores the weights fails the identity.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import synth_inputs as si

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _parts(inp, heads=None):
    f = inp.f32
    pre = oracle.prefix_mla_absorbed(f("q_nope"), f("q_rope"), f("w_uk"), f("w_uv"), f("c_kv"), f("k_pe"),
                                     inp.page_table, inp.L, inp.sm_scale, heads=heads)
    tail = oracle.verify_mla_absorbed(f("q_nope"), f("q_rope"), f("w_uk"), f("w_uv"), f("c_kv"), f("k_pe"),
                                      inp.page_table[inp.L:], 0, inp.parent, inp.sm_scale, heads=heads)
    full = oracle.verify_inputs(inp, heads=heads)
    return pre, tail, full


@pytest.mark.parametrize("maker,kw", [(si.tiny, dict(seed=0)), (si.tiny, dict(seed=3, dist="peak4")),
                                      (si.kimi, dict(L=200, T=15, seed=1)), (si.kimi, dict(L=1, T=9, seed=2))])
def test_prefix_tail_merge_is_whole_cache_attention(maker, kw):
    inp = maker(**kw)
    heads = None if inp.H <= 8 else [0, 17, 63]
    (po, pl), (to, tl), (fo, fl) = _parts(inp, heads)
    hs = list(range(inp.H)) if heads is None else heads
    mo, ml = oracle.merge_attn_states(po[:, hs], pl[:, hs], to[:, hs], tl[:, hs])
    np.testing.assert_allclose(mo, fo[:, hs], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ml, fl[:, hs], rtol=1e-12, atol=1e-12)


def test_prefix_matches_scipy_softmax_over_explicit_heads():
    inp = si.tiny(seed=5)
    f = inp.f32
    out, lse = oracle.prefix_mla_absorbed(f("q_nope"), f("q_rope"), f("w_uk"), f("w_uv"), f("c_kv"), f("k_pe"),
                                          inp.page_table, inp.L, inp.sm_scale)
    C = f("c_kv")[inp.page_table[:inp.L]].astype(np.float64)
    Kp = f("k_pe")[inp.page_table[:inp.L]].astype(np.float64)
    for h in range(inp.H):
        K = np.concatenate([C @ f("w_uk")[h].astype(np.float64).T, Kp], axis=1)   # per-head keys [L][Dn+Dr]
        V = C @ f("w_uv")[h].astype(np.float64).T                                 # per-head values [L][Dv]
        for t in range(inp.T):
            q = np.concatenate([f("q_nope")[t, h], f("q_rope")[t, h]]).astype(np.float64)
            s = inp.sm_scale * (K @ q)
            np.testing.assert_allclose(out[t, h], softmax(s) @ V, rtol=1e-10, atol=1e-12)
            assert abs(lse[t, h] - logsumexp(s)) < 1e-11


def test_two_single_position_parts_merge_to_two_way_softmax():
    rng = np.random.default_rng(7)
    s = rng.normal(0, 4, size=(50, 2))
    v = rng.normal(0, 1, size=(50, 2, 16))
    out, lse = oracle.merge_attn_states(v[:, 0], s[:, 0], v[:, 1], s[:, 1])
    p = softmax(s, axis=1)
    np.testing.assert_allclose(out, p[:, 0:1] * v[:, 0] + p[:, 1:2] * v[:, 1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, np.logaddexp(s[:, 0], s[:, 1]), rtol=1e-14, atol=1e-14)


def test_empty_parts():
    rng = np.random.default_rng(8)
    oa, ob = rng.normal(size=(6, 8)), rng.normal(size=(6, 8))
    la = rng.normal(size=6)
    ninf = np.full(6, -np.inf)
    out, lse = oracle.merge_attn_states(oa, la, ob, ninf)
    assert np.array_equal(out, oa) and np.array_equal(lse, la)
    out, lse = oracle.merge_attn_states(oa, ninf, ob, la)
    assert np.array_equal(out, ob) and np.array_equal(lse, la)
    out, lse = oracle.merge_attn_states(oa, ninf, ob, ninf)
    assert np.array_equal(out, np.zeros_like(oa)) and np.all(lse == -np.inf)


def test_merge_symmetric_and_associative():
    rng = np.random.default_rng(9)
    o = rng.normal(size=(3, 20, 8))
    l = rng.normal(0, 5, size=(3, 20))
    ab, lab = oracle.merge_attn_states(o[0], l[0], o[1], l[1])
    ba, lba = oracle.merge_attn_states(o[1], l[1], o[0], l[0])
    np.testing.assert_allclose(ab, ba, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lab, lba, rtol=1e-15, atol=0)
    left = oracle.merge_attn_states(ab, lab, o[2], l[2])
    bc, lbc = oracle.merge_attn_states(o[1], l[1], o[2], l[2])
    right = oracle.merge_attn_states(o[0], l[0], bc, lbc)
    np.testing.assert_allclose(left[0], right[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(left[1], right[1], rtol=1e-14, atol=1e-14)


def test_unweighted_merge_fails_identity():
    inp = si.tiny(seed=0)
    (po, pl), (to, tl), (fo, fl) = _parts(inp)
    assert not np.allclose(0.5 * (po + to), fo, rtol=1e-3, atol=1e-3)
    mo, _ = oracle.merge_attn_states(po, pl, to, tl)
    assert np.allclose(mo, fo, rtol=1e-10, atol=1e-12)
