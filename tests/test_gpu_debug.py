"""KDV_DEBUG=1: the page-table check in front of the verify kernels (include/kdv.h, pool_slots).

Every out-of-contract entry used here (>= pool_slots) still lies inside the allocated pool: pool_slots is
passed smaller than the pool, so even a missed check could not read outside the buffer.  A failed check must
leave the status KDV_ERR_PAGE in the workspace header and NaN in out and lse; a passing one KDV_OK and the
ordinary result.
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


@pytest.fixture
def debug_on(monkeypatch):
    monkeypatch.setenv("KDV_DEBUG", "1")


def _single(inp, pool_slots):
    dev = si.to_device(inp)
    mask, _ = kdv.build_tree_mask(dev["parent"])
    dims = kdv.make_dims(**inp.dims())
    ws = torch.zeros((kdv.verify_workspace_bytes(dims, inp.T, inp.L),), dtype=torch.uint8, device="cuda")
    ws[:4].fill_(0x55)  # neither status value
    lse = torch.zeros((inp.T, inp.H), dtype=torch.float32, device="cuda")
    out, lse = kdv.verify_mla_attn(dims, dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"], dev["c_kv"],
                                   dev["k_pe"], dev["page_table"], inp.L, mask, lse=lse, workspace=ws,
                                   pool_slots=pool_slots)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy(), kdv.debug_status(ws)


def test_valid_table_passes(debug_on):
    inp = si.kimi(L=700, T=15, seed=4, dist="unit")
    out, _, st = _single(inp, inp.pool_slots)
    assert st == kdv.KDV_OK
    ref, _ = oracle.verify_inputs(inp)
    assert out_passes(out, ref)[0]


@pytest.mark.parametrize("shape", ["kimi", "tiny"])
def test_entry_past_pool_slots_is_caught(debug_on, shape):
    # contiguous pool of exactly L + T rows; declaring one slot fewer puts the last tree row out of contract
    inp = si.kimi(L=700, T=15, seed=4, dist="unit") if shape == "kimi" else si.tiny(seed=2, dist="unit")
    out, lse, st = _single(inp, inp.pool_slots - 1)
    assert st == kdv.KDV_ERR_PAGE
    assert np.isnan(out).all() and np.isnan(lse).all()


def test_prefix_and_batch_checked(debug_on):
    inp = si.kimi(L=300, T=9, seed=6, dist="unit")
    dev = si.to_device(inp)
    dims = kdv.make_dims(**inp.dims())
    n = kdv.kdv_prefix_workspace_bytes(dims, inp.T, inp.L)
    ws = torch.zeros((n,), dtype=torch.uint8, device="cuda")
    pt = dev["page_table"][:inp.L].contiguous()
    out, lse = kdv.prefix_mla_attn(dims, dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"], dev["c_kv"],
                                   dev["k_pe"], pt, inp.L, workspace=ws, pool_slots=inp.L - 1)
    torch.cuda.synchronize()
    assert kdv.debug_status(ws) == kdv.KDV_ERR_PAGE and torch.isnan(out.float()).all()
    kdv.prefix_mla_attn(dims, dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"], dev["c_kv"], dev["k_pe"], pt,
                        inp.L, workspace=ws, pool_slots=inp.L)
    torch.cuda.synchronize()
    assert kdv.debug_status(ws) == kdv.KDV_OK

    reqs = si.batch_inputs(si.KIMI_DIMS, [200, 50], [7, 15], seed=3, dist="unit")
    b16 = lambda arrs: torch.from_numpy(np.ascontiguousarray(np.concatenate(arrs)).view(np.int16)).cuda()  # noqa
    P = reqs[0].pool_slots
    table = np.concatenate([r.page_table for r in reqs]).astype(np.int32)
    bad_pool = int(table.max())  # the request holding the largest slot is out of contract
    mask, _ = kdv.build_tree_masks([torch.from_numpy(r.parent.astype(np.int32)).cuda() for r in reqs])
    bdims = kdv.make_dims(**reqs[0].dims())
    args = (bdims, b16([r.q_nope for r in reqs]), b16([r.q_rope for r in reqs]), b16([reqs[0].w_uk]),
            b16([reqs[0].w_uv]), b16([reqs[0].c_kv]), b16([reqs[0].k_pe]), torch.from_numpy(table).cuda(),
            [r.L for r in reqs], [r.T for r in reqs], mask)
    ws = torch.zeros((kdv.verify_batch_workspace_bytes(bdims, args[8], args[9]),), dtype=torch.uint8, device="cuda")
    out, _ = kdv.verify_mla_attn_batch(*args, workspace=ws, pool_slots=bad_pool)
    torch.cuda.synchronize()
    assert kdv.debug_status(ws) == kdv.KDV_ERR_PAGE and torch.isnan(out.float()).all()
    out, _ = kdv.verify_mla_attn_batch(*args, workspace=ws, pool_slots=P)
    torch.cuda.synchronize()
    assert kdv.debug_status(ws) == kdv.KDV_OK
    got = out.float().cpu().numpy()
    off = 0
    for r in reqs:
        ref, _ = oracle.verify_inputs(r)
        assert out_passes(got[off:off + r.T], ref)[0]
        off += r.T


def test_debug_off_writes_no_status(monkeypatch):
    monkeypatch.delenv("KDV_DEBUG", raising=False)
    inp = si.tiny(seed=2, dist="unit")
    out, _, st = _single(inp, inp.pool_slots)
    assert st == 0x55555555
