"""GPU parity of best-first draft-tree construction (kdv_build_draft_tree) against the oracle: bit-exact
parent array, tokens and node count.  Cases: the hand-worked examples (exact ties), random drafter tables
with and without ties over block / K / budget edges (budget 1, trees smaller than the budget, 64 nodes), the
session's block 16 / budget 32 setting, and the full device pipeline build -> mask -> verify -> accept on one
stream.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from tests.parity import out_passes

pytestmark = pytest.mark.gpu

kdv = pytest.importorskip("speculative_decoding_tree_parent_amd")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def gpu_build(logp, tok, budget, root):
    lp = torch.from_numpy(np.ascontiguousarray(np.asarray(logp, dtype=np.float32))).cuda()
    tk = torch.from_numpy(np.ascontiguousarray(np.asarray(tok, dtype=np.int32))).cuda()
    rt = torch.tensor([root], dtype=torch.int32, device="cuda")
    parent, tokens, n = kdv.build_draft_tree(lp, tk, budget, rt)
    torch.cuda.synchronize()
    n = int(n.item())
    p, t = parent.cpu().numpy(), tokens.cpu().numpy()
    assert (p[n:] == -1).all() and (t[n:] == -1).all()
    return p[:n].tolist(), t[:n].tolist()


def check(logp, tok, budget, root=12345):
    got = gpu_build(logp, tok, budget, root)
    rp, rt, _ = oracle.build_draft_tree(logp, tok, budget, root)
    assert got == (rp.tolist(), rt.tolist())


@pytest.mark.parametrize("k", range(3))
def test_hand_cases(k):
    c = json.load(open(os.path.join(GOLDEN, "draft_tree.json")))["cases"][k]
    assert gpu_build(c["logp"], c["tok"], c["budget"], c["root_token"]) == (c["parent"], c["tokens"])


@pytest.mark.parametrize("block,K", [(1, 1), (1, 8), (3, 2), (4, 3), (16, 8), (16, 16), (63, 64), (40, 2)])
@pytest.mark.parametrize("budget", [1, 2, 15, 32, 33, 64])
@pytest.mark.parametrize("ties", [False, True])
def test_random_tables(block, K, budget, ties):
    for seed in range(2):
        logp, tok = si.draft_topk(seed, block, K, ties=ties)
        check(logp, tok, budget)


def test_session_setting_block16_budget32():
    for seed in range(20):
        logp, tok = si.draft_topk(100 + seed, 16, 8)
        check(logp, tok, 32)


def test_pipeline_build_mask_verify_accept():
    """build -> mask -> verify -> accept on one stream, device arrays only, one synchronisation at the end."""
    T = 15
    logp, tok = si.draft_topk(7, 16, 4)
    ref_parent, ref_tokens, _ = oracle.build_draft_tree(logp, tok, T, 42)
    inp = si.kimi(L=300, T=T, seed=5, dist="unit", parent=ref_parent)
    rng = np.random.default_rng(9)  # target predictions that follow a built child most of the time
    pred = rng.integers(0, 1 << 16, size=T).astype(np.int32)
    for p in range(T):
        kids = [c for c in range(T) if ref_parent[c] == p]
        if kids and rng.random() < 0.9:
            pred[p] = ref_tokens[kids[int(rng.integers(0, len(kids)))]]
    d = si.to_device(inp)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        lp = torch.from_numpy(logp).cuda()
        tk = torch.from_numpy(tok).cuda()
        root = torch.tensor([42], dtype=torch.int32, device="cuda")
        parent, tokens, _ = kdv.build_draft_tree(lp, tk, T, root, stream=stream)
        mask, mstatus = kdv.build_tree_mask(parent, stream=stream)
        out, _ = kdv.verify_mla_attn(kdv.make_dims(**inp.dims()), d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                     d["c_kv"], d["k_pe"], d["page_table"], inp.L, mask, stream=stream)
        pr = torch.from_numpy(pred).cuda()
        path, n_path, nxt, astatus = kdv.tree_accept(parent, tokens, pr, stream=stream)
    stream.synchronize()
    assert parent.cpu().numpy().tolist() == ref_parent.tolist()
    assert tokens.cpu().numpy().tolist() == ref_tokens.tolist()
    ref_mask, _ = oracle.tree_mask(ref_parent)
    assert (mask.cpu().numpy().view(np.uint32) == ref_mask).all()
    ok, err = out_passes(out.float().cpu().numpy().astype(np.float64), oracle.verify_inputs(inp)[0])
    assert ok, err
    ref_path, ref_next, _ = oracle.tree_accept(ref_parent, ref_tokens, pred)
    n = int(n_path.item())
    assert path.cpu().numpy()[:n].tolist() == ref_path and int(nxt.item()) == ref_next
    assert int(mstatus.item()) == 0 and int(astatus.item()) == 0
