"""Greedy acceptance of a verified draft tree: the step that follows tree-verify attention.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Plain Python over small integer arrays.

Source: "The Architecture of Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 3: after the verify
forward pass the engine selects, greedily and on the device, the longest prefix of accepted tokens; the same
page's composition test chains build -> verify -> accept with no host round trip.

Readings where the page is silent:
  * node 0 is the root, the position whose token is already committed; parent[i] < i (as for the mask);
  * pred[t] is the target model's greedy prediction after the prefix that ends at node t (its argmax);
  * a child c of node p is accepted when its draft token equals pred[p]; the walk starts at the root and
    moves to an accepted child while one exists.  With distinct sibling tokens that child is unique and the
    walk yields the longest accepted root path; if several siblings carry the predicted token, the lowest
    node index is taken;
  * the committed tokens of the step are the draft tokens of path[1:] followed by pred[path[-1]] (the
    target's own token after the accepted prefix);
  * a malformed tree (the mask's rules) gives status KDV_ERR_TREE and the root alone.
"""
from __future__ import annotations

import numpy as np

from .ref import KDV_ERR_TREE, KDV_OK, tree_status


def tree_accept(parent, tokens, pred) -> tuple[list[int], int, int]:
    """Returns (path, next_token, status): path = node indices root -> last accepted node (path[0] = 0)."""
    parent = np.asarray(parent)
    tokens = np.asarray(tokens)
    pred = np.asarray(pred)
    T = parent.shape[0]
    if tree_status(parent) != KDV_OK:
        return [0], int(pred[0]), KDV_ERR_TREE
    path = [0]
    cur = 0
    while True:
        nxt = None
        for c in range(T):  # children in increasing index order: the first match wins
            if int(parent[c]) == cur and int(tokens[c]) == int(pred[cur]):
                nxt = c
                break
        if nxt is None:
            break
        path.append(nxt)
        cur = nxt
    return path, int(pred[cur]), KDV_OK
