"""GPU tests of kdv_verify_mla_attn_tree: the verify call that builds the tree's ancestor mask itself.

Its mask and status must be bit-identical to the oracle's (and so to kdv_build_tree_mask's), and its output
and lse bit-identical to kdv_build_tree_mask followed by kdv_verify_mla_attn (same kernels, same plan), which
the parity tests hold to the fp64 oracle; one case is also checked against the oracle directly.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from tests.parity import out_passes

pytestmark = pytest.mark.gpu

kdv = pytest.importorskip("speculative_decoding_tree_parent_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def both(inp, parent=None):
    dev = si.to_device(inp)
    if parent is not None:
        dev["parent"] = torch.from_numpy(np.asarray(parent, dtype=np.int32)).cuda()
    dims = kdv.make_dims(**inp.dims())
    args = (dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"], dev["c_kv"], dev["k_pe"], dev["page_table"], inp.L)
    lse1 = torch.empty((inp.T, inp.H), dtype=torch.float32, device="cuda")
    out1, lse1, mask1, st1 = kdv.verify_mla_attn_tree(dims, *args, dev["parent"], lse=lse1)
    mask2, st2 = kdv.build_tree_mask(dev["parent"])
    lse2 = torch.empty((inp.T, inp.H), dtype=torch.float32, device="cuda")
    out2, lse2 = kdv.verify_mla_attn(dims, *args, mask2, lse=lse2)
    torch.cuda.synchronize()
    return (out1, lse1, mask1, st1), (out2, lse2, mask2, st2), dev


@pytest.mark.parametrize("maker,kw", [(si.tiny, dict(seed=0)), (si.kimi, dict(L=5553, T=15, seed=0)),
                                      (si.kimi, dict(L=100, T=33, seed=1)), (si.kimi, dict(L=0, T=64, seed=2)),
                                      (si.make_inputs, dict(**si.FULL61_SHAPE, L=1000, T=32, seed=3)),
                                      # one-tile sequences: the single short-sequence kernel builds the rows itself
                                      (si.kimi, dict(L=13, T=15, seed=5)), (si.kimi, dict(L=0, T=32, seed=6)),
                                      (si.kimi, dict(L=32, T=32, seed=7)),
                                      (si.make_inputs, dict(**si.TINY_DIMS, L=20, T=7, seed=8))])
def test_tree_call_equals_mask_then_verify(maker, kw):
    inp = maker(**kw)
    (o1, l1, m1, s1), (o2, l2, m2, s2), _ = both(inp)
    ref_mask, ref_status = oracle.tree_mask(inp.parent)
    assert int(s1.item()) == int(s2.item()) == ref_status == 0
    assert np.array_equal(m1.cpu().numpy().view(np.uint32), ref_mask)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_tree_call_matches_oracle():
    inp = si.kimi(L=777, T=15, seed=4, dist="peak4")
    (o1, _, _, _), _, _ = both(inp)
    ref, _ = oracle.verify_inputs(inp, heads=[0, 21, 63])
    ok, err = out_passes(o1.float().cpu().numpy()[:, [0, 21, 63]], ref[:, [0, 21, 63]])
    assert ok, err


@pytest.mark.parametrize("L", [128, 20])  # (20: the short-sequence kernel)
def test_tree_call_reports_malformed_tree(L):
    inp = si.make_inputs(**si.TINY_DIMS, L=L, T=7, seed=1)
    bad = [-1, 0, 5, 1, 1, 2, 2]  # node 2's parent is after it
    (o1, l1, m1, s1), (o2, l2, m2, s2), _ = both(inp, parent=bad)
    ref_mask, ref_status = oracle.tree_mask(bad)
    assert ref_status == oracle.KDV_ERR_TREE
    assert int(s1.item()) == int(s2.item()) == ref_status
    assert np.array_equal(m1.cpu().numpy().view(np.uint32), ref_mask)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("L", [300, 13])  # (13: the short-sequence kernel)
def test_tree_call_without_status(L):
    inp = si.kimi(L=L, T=15, seed=7)
    dev = si.to_device(inp)
    dims = kdv.make_dims(**inp.dims())
    T, H = inp.T, inp.H
    mask = torch.empty((T, 1), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, inp.Dv), dtype=torch.bfloat16, device="cuda")
    ws = torch.zeros((kdv.verify_workspace_bytes(dims, T, inp.L),), dtype=torch.uint8, device="cuda")
    rc = kdv.kdv_verify_mla_attn_tree(dims, *[dev[k].data_ptr() for k in ("q_nope", "q_rope", "w_uk", "w_uv", "c_kv",
                                                                         "k_pe")],
                                      inp.pool_slots, dev["page_table"].data_ptr(), inp.L, T,
                                      dev["parent"].data_ptr(), mask.data_ptr(), None, out.data_ptr(), None,
                                      ws.data_ptr(), ws.numel(), None)
    assert rc == kdv.KDV_OK
    torch.cuda.synchronize()
    ref_mask, _ = oracle.tree_mask(inp.parent)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), ref_mask)
    (o2, _, _, _), _, _ = both(inp)
    assert torch.equal(out, o2)
