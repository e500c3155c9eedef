"""GPU parity for the batched verify (kdv_verify_mla_attn_batch): several requests with their own prefix
lengths, trees, page tables and queries over one shared latent pool and one layer's weights, in one call.

Each request's slice of the output is compared with the fp64 oracle run on that request alone (the batched
call computes exactly the single-request attention for every request), with the criterion of
tests/parity.py; a batch of one is bit-identical to kdv_verify_mla_attn.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from tests.parity import lse_passes, lse_tolerance, out_passes

pytestmark = pytest.mark.gpu

kdv = pytest.importorskip("speculative_decoding_tree_parent_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _b16(arrs):
    return torch.from_numpy(np.ascontiguousarray(np.concatenate(arrs)).view(np.int16)).cuda()


def run_batch(reqs, splits=None):
    r0 = reqs[0]
    dims = kdv.make_dims(**r0.dims())
    Ls, Ts = [r.L for r in reqs], [r.T for r in reqs]
    dev = dict(q_nope=_b16([r.q_nope for r in reqs]), q_rope=_b16([r.q_rope for r in reqs]),
               w_uk=_b16([r0.w_uk]), w_uv=_b16([r0.w_uv]), c_kv=_b16([r0.c_kv]), k_pe=_b16([r0.k_pe]),
               page_table=torch.from_numpy(np.concatenate([r.page_table for r in reqs]).astype(np.int32)).cuda())
    parents = [torch.from_numpy(r.parent.astype(np.int32)).cuda() for r in reqs]
    old = os.environ.get("KDV_SPLITS")
    if splits is not None:
        os.environ["KDV_SPLITS"] = str(splits)
    try:
        mask, status = kdv.build_tree_masks(parents)
        lse = torch.empty((sum(Ts), r0.H), dtype=torch.float32, device="cuda")
        out, lse = kdv.verify_mla_attn_batch(dims, dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"],
                                             dev["c_kv"], dev["k_pe"], dev["page_table"], Ls, Ts, mask, lse=lse)
        torch.cuda.synchronize()
    finally:
        if splits is not None:
            if old is None:
                del os.environ["KDV_SPLITS"]
            else:
                os.environ["KDV_SPLITS"] = old
    assert np.all(status.cpu().numpy() == 0)
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy(), dev, mask


def check_batch(reqs, heads=None, splits=None):
    got, glse, _, _ = run_batch(reqs, splits)
    n0 = 0
    for c, r in enumerate(reqs):
        ref, rlse = oracle.verify_inputs(r, heads=heads)
        sel = slice(None) if heads is None else (slice(None), list(heads))
        g, gl = got[n0:n0 + r.T], glse[n0:n0 + r.T]
        ok, err = out_passes(g[sel], ref[sel])
        assert ok, f"request {c} (L={r.L}, T={r.T}): output parity failed: {err}"
        lok, ratio = lse_passes(gl[sel], rlse[sel], lse_tolerance(r, heads)[sel])
        assert lok, f"request {c}: lse parity failed: max |dlse| / bound = {ratio:.3f}"
        n0 += r.T


@pytest.mark.parametrize("dist", si.DISTRIBUTIONS)
def test_tiny_mixed_requests(dist):
    check_batch(si.batch_inputs(si.TINY_DIMS, [128, 0, 65], [7, 1, 33], seed=1, dist=dist))


@pytest.mark.parametrize("seed", [0, 1])
def test_tiny_sixteen_requests(seed):
    rng = np.random.default_rng(100 + seed)
    Ls = rng.integers(0, 300, size=16).tolist()
    Ts = rng.integers(1, 65, size=16).tolist()
    check_batch(si.batch_inputs(si.TINY_DIMS, Ls, Ts, seed=seed, dist="unit"))


@pytest.mark.parametrize("splits", [1, 3])
def test_tiny_forced_splits(splits):
    check_batch(si.batch_inputs(si.TINY_DIMS, [200, 64, 1, 130], [7, 15, 2, 64], seed=3, dist="unit"),
                splits=splits)


def test_kimi_two_requests():
    check_batch(si.batch_inputs(si.KIMI_DIMS, [5553, 100], [15, 9], seed=4), heads=[0, 33, 63])


def test_kimi_uneven_requests():
    """Requests of 1, 15, 64 and 9 nodes over prefixes of 0, 4000, 13 and 700 tokens: under the batch plan the
    groups have 64 workgroups (one per query tile of the 64-node request), the runs are 20 KV tiles, the last
    run touches three requests, most members skip the smaller requests, and the combine takes 16-node blocks."""
    check_batch(si.batch_inputs(si.KIMI_DIMS, [0, 4000, 13, 700], [1, 15, 64, 9], seed=8, dist="unit"),
                heads=[0, 31, 63])


def test_kimi_ten_streams():
    """Ten concurrent 15-node trees over 1000-token prefixes (the pages' C = 10 serving level)."""
    check_batch(si.batch_inputs(si.KIMI_DIMS, [1000] * 10, [15] * 10, seed=5), heads=[0, 63])


def test_kimi_ten_requests_timed_workload():
    """The ten-request workload the benchmark times: ten 15-node trees over 5553-token prefixes.  The batch plan
    takes 17 groups of 15 workgroups and runs of 52 of the 870 KV tiles, so every request is split over 2 or 3
    runs, and the combine takes 16-node blocks."""
    check_batch(si.batch_inputs(si.KIMI_DIMS, [5553] * 10, [15] * 10, seed=10, dist="unit"), heads=[0, 37, 63])


def test_kimi_sixteen_requests():
    """The largest batch (16 requests) at full Kimi dims: ten 15-node trees over 5553-token prefixes, as in the
    timed ten-request workload, plus six more requests of 64, 1, 33, 9, 15 and 2 nodes over 0 to 3333 tokens.
    Under the batch plan the groups have 64 workgroups (one per query tile of the 64-node request), four runs
    of 239 of the 955 KV tiles, each touching 3 to 8 requests; members past a request's query tiles skip it."""
    Ls = [5553] * 10 + [0, 1, 64, 3333, 1663, 13]
    Ts = [15] * 10 + [64, 1, 33, 9, 15, 2]
    check_batch(si.batch_inputs(si.KIMI_DIMS, Ls, Ts, seed=9, dist="unit"), heads=[0, 63])


def test_batch_of_one_is_the_single_call():
    reqs = si.batch_inputs(si.KIMI_DIMS, [777], [15], seed=6)
    got, glse, dev, mask = run_batch(reqs)
    r = reqs[0]
    lse = torch.empty((r.T, r.H), dtype=torch.float32, device="cuda")
    out, lse = kdv.verify_mla_attn(kdv.make_dims(**r.dims()), dev["q_nope"], dev["q_rope"], dev["w_uk"],
                                   dev["w_uv"], dev["c_kv"], dev["k_pe"], dev["page_table"], r.L, mask, lse=lse)
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), got.astype(np.float32))
    assert np.array_equal(lse.cpu().numpy(), glse)
