"""Pins for the greedy tree-accept oracle (oracle/accept.py) against facts it does not compute itself.

* hand-worked cases (tests/golden/tree_accept.json);
* a closed form: on a chain tree the accepted length is the first draft/prediction mismatch;
* brute force: every root path is enumerated; with distinct sibling tokens the oracle's path is the unique
  longest path whose every edge carries the parent's prediction;
* properties with duplicate sibling tokens (accepted, maximal, lowest index at every step);
* malformed trees; a mistake planted in the oracle (prediction taken at the child) fails the hand cases.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import accept as oacc
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    return json.load(open(os.path.join(GOLDEN, "tree_accept.json")))["cases"]


@pytest.mark.parametrize("k", range(4))
def test_hand_cases(k):
    c = _cases()[k]
    path, nxt, status = oracle.tree_accept(c["parent"], c["tokens"], c["pred"])
    assert status == oracle.KDV_OK
    assert path == c["path"] and nxt == c["next_token"]


def _accepted_paths(parent, tokens, pred):
    """Every root path (root..t) whose edges all carry the parent's prediction."""
    out = []
    for t in range(len(parent)):
        path = oracle.ancestor_path(parent, t)
        if all(tokens[c] == pred[p] for p, c in zip(path[:-1], path[1:])):
            out.append(path)
    return out


@pytest.mark.parametrize("T", [1, 2, 5, 15, 32, 64])
@pytest.mark.parametrize("seed", range(4))
def test_chain_closed_form(T, seed):
    parent = np.arange(-1, T - 1, dtype=np.int32)
    _, tok, pred = si.accept_inputs(seed, T, vocab=4, follow=0.9, parent=parent)
    mism = np.flatnonzero(tok[1:] != pred[:-1])
    n_acc = int(mism[0]) if mism.size else T - 1
    path, nxt, status = oracle.tree_accept(parent, tok, pred)
    assert status == oracle.KDV_OK
    assert path == list(range(n_acc + 1))
    assert nxt == int(pred[n_acc])


@pytest.mark.parametrize("T", [2, 7, 15, 33, 64])
@pytest.mark.parametrize("seed", range(6))
def test_brute_force_distinct_siblings(T, seed):
    parent, tok, pred = si.accept_inputs(seed, T, vocab=1 << 20, follow=0.8)
    for p in range(T):  # make sibling tokens distinct so the accepted path is unique
        kids = [c for c in range(T) if parent[c] == p]
        assert len({int(tok[c]) for c in kids}) == len(kids)
    paths = _accepted_paths(parent, tok, pred)
    longest = max(len(pth) for pth in paths)
    best = [pth for pth in paths if len(pth) == longest]
    assert len(best) == 1
    path, nxt, _ = oracle.tree_accept(parent, tok, pred)
    assert path == best[0]
    assert nxt == int(pred[path[-1]])


@pytest.mark.parametrize("seed", range(10))
def test_duplicate_siblings_properties(seed):
    parent, tok, pred = si.accept_inputs(seed, 40, vocab=3, follow=0.9, dup=0.5)
    path, nxt, _ = oracle.tree_accept(parent, tok, pred)
    assert path[0] == 0
    for p, c in zip(path[:-1], path[1:]):
        assert parent[c] == p and tok[c] == pred[p]
        assert not any(parent[d] == p and tok[d] == pred[p] for d in range(c))  # lowest matching index
    last = path[-1]
    assert not any(parent[d] == last and tok[d] == pred[last] for d in range(40))  # maximal
    assert nxt == int(pred[last])


def test_malformed_tree():
    path, nxt, status = oracle.tree_accept([-1, 0, 5, 1], [1, 2, 3, 4], [2, 9, 9, 9])
    assert status == oracle.KDV_ERR_TREE and path == [0] and nxt == 2


def test_planted_mistake_fails(monkeypatch):
    """Taking the prediction at the child instead of at its parent must fail the hand cases."""
    def wrong(parent, tokens, pred):
        parent, tokens, pred = map(np.asarray, (parent, tokens, pred))
        path, cur = [0], 0
        while True:
            nxt = next((c for c in range(len(parent)) if parent[c] == cur and tokens[c] == pred[c]), None)
            if nxt is None:
                return path, int(pred[cur]), oracle.KDV_OK
            path.append(nxt)
            cur = nxt
    fails = 0
    for c in _cases():
        path, nxt, _ = wrong(c["parent"], c["tokens"], c["pred"])
        fails += (path != c["path"] or nxt != c["next_token"])
    assert fails > 0
