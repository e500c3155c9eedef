"""GPU parity of greedy tree acceptance (kdv_tree_accept) against the oracle: bit-exact path, count, next
token and status.  Cases: the hand-worked examples, random trees at every size edge (1, 2, 32/33, 63, 64
nodes) with varied acceptance rates and duplicate sibling tokens, chains, malformed trees, and the
on-device composition mask -> verify -> accept on one stream with no host round trip in between.
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


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.int32))).cuda()


def gpu_accept(parent, tokens, pred):
    path, n_path, nxt, status = kdv.tree_accept(_dev(parent), _dev(tokens), _dev(pred))
    torch.cuda.synchronize()
    n = int(n_path.item())
    p = path.cpu().numpy()
    assert (p[n:] == -1).all(), "entries past n_path must be -1"
    return p[:n].tolist(), int(nxt.item()), int(status.item())


def check(parent, tokens, pred):
    got = gpu_accept(parent, tokens, pred)
    ref = oracle.tree_accept(parent, tokens, pred)
    assert got == (ref[0], ref[1], ref[2]), (got, ref)


@pytest.mark.parametrize("k", range(4))
def test_hand_cases(k):
    c = json.load(open(os.path.join(GOLDEN, "tree_accept.json")))["cases"][k]
    assert gpu_accept(c["parent"], c["tokens"], c["pred"]) == (c["path"], c["next_token"], oracle.KDV_OK)


@pytest.mark.parametrize("T", [1, 2, 7, 15, 31, 32, 33, 63, 64])
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("follow,dup,vocab", [(0.9, 0.0, 32000), (0.5, 0.0, 32000), (0.95, 0.6, 3)])
def test_random_trees(T, seed, follow, dup, vocab):
    check(*si.accept_inputs(seed, T, vocab=vocab, follow=follow, dup=dup))


@pytest.mark.parametrize("T", [2, 16, 64])
def test_chain_fully_accepted(T):
    parent = np.arange(-1, T - 1, dtype=np.int32)
    tokens = np.arange(T, dtype=np.int32) + 100
    pred = np.append(tokens[1:], 7).astype(np.int32)
    path, nxt, status = gpu_accept(parent, tokens, pred)
    assert path == list(range(T)) and nxt == 7 and status == oracle.KDV_OK


@pytest.mark.parametrize("parent", [[0, 0, 1], [-1, 2, 0], [-1, 0, -1], [-1, 0, 1, 70]])
def test_malformed_tree(parent):
    T = len(parent)
    check(parent, list(range(T)), [1] * T)


def test_composition_mask_verify_accept():
    """mask -> verify -> accept on one stream, device arrays only, one synchronisation at the end."""
    inp = si.kimi(L=600, T=15, seed=3, dist="unit")
    par, tok, pred = si.accept_inputs(11, inp.T, vocab=64, follow=0.9, parent=inp.parent)
    d = si.to_device(inp)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        mask, mstatus = kdv.build_tree_mask(d["parent"], stream=stream)
        out, _ = kdv.verify_mla_attn(kdv.make_dims(**inp.dims()), d["q_nope"], d["q_rope"], d["w_uk"], d["w_uv"],
                                     d["c_kv"], d["k_pe"], d["page_table"], inp.L, mask, stream=stream)
        path, n_path, nxt, astatus = kdv.tree_accept(d["parent"], _dev(tok), _dev(pred), stream=stream)
    stream.synchronize()
    ref_mask, _ = oracle.tree_mask(inp.parent)
    assert (mask.cpu().numpy().view(np.uint32) == ref_mask).all()
    ok, err = out_passes(out.float().cpu().numpy().astype(np.float64), oracle.verify_inputs(inp)[0])
    assert ok, err
    ref = oracle.tree_accept(inp.parent, tok, pred)
    n = int(n_path.item())
    assert path.cpu().numpy()[:n].tolist() == ref[0] and int(nxt.item()) == ref[1]
    assert int(mstatus.item()) == 0 and int(astatus.item()) == 0
