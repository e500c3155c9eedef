"""Best-first construction of the draft tree from the drafter's per-position top-K log-probabilities.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).  Plain Python (heapq) with float32 scores.

Source: "The Architecture of Diagnosis...", section "Phase 1: Custom CUDA Kernels", item 1: the draft tree is
built best-first on the device instead of with a host-side priority queue; the session's DDTree settings are
block 16 and budget 32 ("Three Acts of Engineering...", the B300 projection).

Readings where the pages are silent:
  * the drafter gives, for each of the `block` positions after the committed token, its K best tokens tok[d][r]
    with log-probabilities logp[d][r], sorted so that logp[d][0] >= logp[d][1] >= ... (the top-k of each
    position's distribution); positions are independent, so a root path's score is the float32 sum of its
    nodes' log-probabilities, added from the root down;
  * node 0 is the root and carries the committed token; a node at depth d >= 1 takes a token of position d - 1;
  * the tree holds at most `budget` nodes, root included, and is grown best-first: the candidate with the
    highest score joins next.  Ties go to the smaller depth, then the smaller parent index, then the smaller
    rank.  A node joins only after its parent and its better-ranked siblings (their scores are >= its own),
    so node indices are in topological order and the tree is the `budget - 1` best nodes of the full
    K-ary tree of depth `block`;
  * when a node joins, its next sibling (rank + 1) and its first child (rank 0 at depth + 1) become candidates;
    this lazy expansion enumerates exactly the best-first order because each position's list is sorted.
"""
from __future__ import annotations

import heapq

import numpy as np


def _key(score: np.float32, depth: int, parent: int, rank: int):
    # heapq pops the smallest: negate the score; ties by depth, parent, rank ascending
    return (-float(score), depth, parent, rank)


def build_draft_tree(logp, tok, budget: int, root_token: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Returns (parent int32 [n], tokens int32 [n], score float32 [n]), n = min(budget, nodes available)."""
    logp = np.asarray(logp, dtype=np.float32)
    tok = np.asarray(tok)
    block, K = logp.shape
    parent, tokens, score, depth = [-1], [int(root_token)], [np.float32(0.0)], [0]
    heap = []
    if block > 0 and K > 0 and budget > 1:
        s = np.float32(np.float32(0.0) + logp[0, 0])
        heapq.heappush(heap, (_key(s, 1, 0, 0), s, 1, 0, 0))
    while heap and len(parent) < budget:
        _, s, d, p, r = heapq.heappop(heap)
        i = len(parent)
        parent.append(p)
        tokens.append(int(tok[d - 1, r]))
        score.append(s)
        depth.append(d)
        if r + 1 < K:  # next sibling: same parent, next-ranked token of the same position
            s2 = np.float32(score[p] + logp[d - 1, r + 1])
            heapq.heappush(heap, (_key(s2, d, p, r + 1), s2, d, p, r + 1))
        if d < block:  # first child: best token of the next position
            s3 = np.float32(s + logp[d, 0])
            heapq.heappush(heap, (_key(s3, d + 1, i, 0), s3, d + 1, i, 0))
    return (np.array(parent, dtype=np.int32), np.array(tokens, dtype=np.int32),
            np.array(score, dtype=np.float32))
