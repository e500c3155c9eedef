"""Pins for the best-first draft-tree oracle (oracle/build.py) against facts it does not compute itself.

* hand-worked cases, including exact ties (tests/golden/draft_tree.json);
* brute force: with continuous log-probabilities the tree is the budget - 1 highest-scoring nodes of the full
  K-ary tree of depth `block`, in decreasing score order (every node of that tree enumerated, float32 sums);
* K = 1 gives a chain; structural invariants; a mistake planted in the oracle (no sibling expansion) fails.
"""
import heapq
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    return json.load(open(os.path.join(GOLDEN, "draft_tree.json")))["cases"]


@pytest.mark.parametrize("k", range(3))
def test_hand_cases(k):
    c = _cases()[k]
    parent, tokens, _ = oracle.build_draft_tree(c["logp"], c["tok"], c["budget"], c["root_token"])
    assert parent.tolist() == c["parent"] and tokens.tolist() == c["tokens"]


def _all_nodes(logp):
    """Every node of the full K-ary tree: (rank path, float32 score accumulated from the root)."""
    block, K = logp.shape
    out = []
    for d in range(1, block + 1):
        for ranks in itertools.product(range(K), repeat=d):
            s = np.float32(0.0)
            for pos, r in enumerate(ranks):
                s = np.float32(s + logp[pos, r])
            out.append((ranks, s))
    return out


@pytest.mark.parametrize("block,K", [(1, 3), (2, 3), (3, 2), (4, 3), (5, 2), (3, 4)])
@pytest.mark.parametrize("budget", [1, 2, 5, 9, 17, 40])
@pytest.mark.parametrize("seed", range(3))
def test_brute_force_top_scores(block, K, budget, seed):
    logp, tok = si.draft_topk(seed, block, K)
    parent, tokens, score = oracle.build_draft_tree(logp, tok, budget, 99)
    nodes = sorted(_all_nodes(logp), key=lambda x: -float(x[1]))
    n = min(budget - 1, len(nodes))
    assert len(parent) == n + 1
    scores = [float(s) for _, s in nodes]
    assert len(set(scores)) == len(scores), "continuous draws are tie-free"
    # same scores, same order; and each node's token is the one its rank path ends with
    assert [float(x) for x in score[1:]] == scores[:n]
    path_of = {0: ()}
    for i in range(1, n + 1):
        path = path_of[int(parent[i])]
        want = nodes[i - 1][0]
        assert want[:-1] == path, "parent must be the node of the path minus its last rank"
        path_of[i] = want
        assert tokens[i] == tok[len(want) - 1, want[-1]]


@pytest.mark.parametrize("block,budget", [(1, 4), (5, 3), (16, 32), (16, 10)])
def test_k1_is_a_chain(block, budget):
    logp, tok = si.draft_topk(1, block, 1)
    parent, tokens, _ = oracle.build_draft_tree(logp, tok, budget, 3)
    n = min(budget, block + 1)
    assert parent.tolist() == list(range(-1, n - 1))
    assert tokens.tolist() == [3] + tok[: n - 1, 0].tolist()


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("ties", [False, True])
def test_invariants(seed, ties):
    block, K, budget = 16, 8, 32
    logp, tok = si.draft_topk(seed, block, K, ties=ties)
    parent, tokens, score = oracle.build_draft_tree(logp, tok, budget, 0)
    assert len(parent) == budget and parent[0] == -1
    depth = [0]
    for i in range(1, budget):
        assert 0 <= parent[i] < i
        depth.append(depth[parent[i]] + 1)
        assert depth[i] <= block
        assert tokens[i] in tok[depth[i] - 1]
        assert score[i] <= score[parent[i]]
    assert all(score[i] >= score[i + 1] for i in range(1, budget - 1))  # best-first: non-increasing
    assert oracle.tree_status(parent) == oracle.KDV_OK


def test_planted_mistake_fails():
    """Expanding only first children (no next sibling) must disagree with the brute-force order."""
    logp, tok = si.draft_topk(0, 3, 3)

    def wrong(budget):
        parent, heap = [-1], [(-float(logp[0, 0]), 1, 0, 0, np.float32(logp[0, 0]))]
        while heap and len(parent) < budget:
            _, d, p, r, s = heapq.heappop(heap)
            parent.append(p)
            if d < 3:
                s3 = np.float32(s + logp[d, 0])
                heapq.heappush(heap, (-float(s3), d + 1, len(parent) - 1, 0, s3))
        return parent
    good, _, _ = oracle.build_draft_tree(logp, tok, 9, 0)
    assert wrong(9) != good.tolist()
