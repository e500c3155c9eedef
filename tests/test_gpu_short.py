"""GPU parity of the short-sequence verify path: one request whose L + T KV rows fit in one 64-row tile and whose
tree has at most 32 nodes runs as one kernel, short_verify_kernel (the query absorption, the scores, a one-tile
softmax, P V and the W_UV product), instead of the query absorption, the split-KV pass and the combine.

Cases: the tile's edges (N = 1, N = 64 with T = 15 and with T = 32, and the first shapes past them, which take the
split path), head counts 1..128, chain and star trees, both score distributions, the 64-wide test shape, a pool
scattered with NaN in every unused slot, the tree-building entry point, the no-allocation entry point, a forced
split count (which always takes the split path), graph replay, and KDV_DEBUG.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from tests.parity import lse_passes, lse_tolerance, out_passes_qlat
from tests.test_gpu_parity import check, run_gpu
from tests.test_zz_no_alloc import _run_both

pytestmark = pytest.mark.gpu

kdv = pytest.importorskip("speculative_decoding_tree_parent_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def kernels(inp):
    return kdv.kdv_verify_kernel_count(kdv.make_dims(**inp.dims()), inp.T, inp.L)


@pytest.mark.parametrize("L,T,n", [(0, 1, 1), (13, 15, 1), (49, 15, 1), (50, 15, 3), (32, 32, 1), (33, 32, 3),
                                   (0, 33, 3), (13, 9, 1), (5553, 15, 3)])
def test_kernel_count(L, T, n):
    assert kdv.kdv_verify_kernel_count(kdv.make_dims(**si.KIMI_DIMS, sm_scale=0.072), T, L) == n


@pytest.mark.parametrize("L,T", [(0, 1), (0, 15), (13, 9), (13, 15), (49, 15), (32, 32), (0, 32), (20, 16),
                                 (50, 15), (33, 32)])
@pytest.mark.parametrize("dist", ["unit", "peak4"])
def test_kimi_tile_edges(L, T, dist):
    inp = si.kimi(L=L, T=T, seed=L * 64 + T, dist=dist)
    check(inp)


@pytest.mark.parametrize("H", [1, 3, 8, 100, 128])
def test_kimi_head_counts(H):
    inp = si.make_inputs(**dict(si.KIMI_DIMS, num_heads=H), L=13, T=15, seed=H, dist="unit")
    assert kernels(inp) == 1
    check(inp)


@pytest.mark.parametrize("shape", ["chain", "star"])
@pytest.mark.parametrize("T", [15, 32])
def test_chain_and_star(shape, T):
    parent = np.arange(-1, T - 1) if shape == "chain" else np.r_[-1, np.zeros(T - 1, dtype=np.int64)]
    check(si.kimi(L=64 - T, T=T, seed=T, dist="peak4", parent=parent))


@pytest.mark.parametrize("L", [0, 1, 30, 57])
@pytest.mark.parametrize("dist", si.DISTRIBUTIONS)
def test_tiny_shape(L, dist):
    inp = si.make_inputs(**si.TINY_DIMS, L=L, T=7, seed=L, dist=dist, parent=[-1, 0, 0, 1, 1, 2, 2])
    assert kernels(inp) == 1
    check(inp)


def test_scattered_nan_pool_bit_identical():
    """Contiguous rows and the same rows scattered over a pool whose other slots hold NaN give identical bits
    (a NaN in the output would mean an unused slot was read, the rows past N included)."""
    a = si.kimi(L=13, T=15, seed=44, dist="unit")
    b = si.kimi(L=13, T=15, seed=44, dist="unit")
    P = 4096
    slots = np.random.default_rng(9).permutation(P)[:a.N].astype(np.int32)
    c = np.full((P, a.R), si.BF16_NAN, dtype=np.uint16)
    k = np.full((P, a.Dr), si.BF16_NAN, dtype=np.uint16)
    c[slots] = a.c_kv[a.page_table]
    k[slots] = a.k_pe[a.page_table]
    b.c_kv, b.k_pe, b.page_table = c, k, slots
    b._f32.clear()
    oa, la = run_gpu(a)
    ob, lb = run_gpu(b)
    oa2, la2 = run_gpu(a)
    assert not np.isnan(ob).any()
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    assert np.array_equal(oa, oa2) and np.array_equal(la, la2)


def test_forced_splits_take_the_split_path(monkeypatch):
    inp = si.kimi(L=13, T=15, seed=3, dist="unit")
    monkeypatch.setenv("KDV_SPLITS", "1")
    assert kernels(inp) == 3
    monkeypatch.delenv("KDV_SPLITS")
    assert kernels(inp) == 1
    check(inp, splits=1)
    check(inp)


def _tree_call(inp, dev, mask, status, out, lse, ws):
    dims = kdv.make_dims(**inp.dims())
    p = lambda t: t.data_ptr()  # noqa: E731
    rc = kdv.kdv_verify_mla_attn_tree(dims, p(dev["q_nope"]), p(dev["q_rope"]), p(dev["w_uk"]), p(dev["w_uv"]),
                                      p(dev["c_kv"]), p(dev["k_pe"]), inp.pool_slots, p(dev["page_table"]), inp.L,
                                      inp.T, p(dev["parent"]), p(mask), p(status), p(out), p(lse), p(ws), ws.numel(),
                                      torch.cuda.current_stream().cuda_stream)
    assert rc == kdv.KDV_OK


def test_tree_building_entry_and_graph_replay():
    """The call that builds its own mask, eagerly and as a captured graph replayed three times with eager work
    between the replays: every replay bit-identical to the eager result, which passes parity."""
    inp = si.kimi(L=13, T=15, seed=12, dist="unit")
    dev = si.to_device(inp)
    dims = kdv.make_dims(**inp.dims())
    ws = torch.zeros((kdv.verify_workspace_bytes(dims, inp.T, inp.L),), dtype=torch.uint8, device="cuda")
    mask = torch.empty((inp.T, 1), dtype=torch.int32, device="cuda")
    status = torch.full((1,), -99, dtype=torch.int32, device="cuda")
    out = torch.empty((inp.T, inp.H, inp.Dv), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((inp.T, inp.H), dtype=torch.float32, device="cuda")
    _tree_call(inp, dev, mask, status, out, lse, ws)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    eager_o, eager_l = out.clone(), lse.clone()
    ref, rlse = oracle.verify_inputs(inp)
    got = eager_o.float().cpu().numpy().astype(np.float64)
    assert out_passes_qlat(got, ref, inp)[0]
    assert lse_passes(eager_l.cpu().numpy(), rlse, lse_tolerance(inp))[0]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _tree_call(inp, dev, mask, status, out, lse, ws)
    for _ in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l)


def test_no_alloc_entry_matches():
    """The no-allocation entry point takes the same path: bit-identical to the workspace entry point."""
    inp = si.kimi(L=40, T=15, seed=8, dist="unit")
    (o_ws, l_ws), (o_na, l_na) = _run_both(inp)
    assert np.array_equal(o_ws, o_na) and np.array_equal(l_ws, l_na)
    ref, _ = oracle.verify_inputs(inp)
    assert out_passes_qlat(o_na.astype(np.float64), ref, inp)[0]


@pytest.mark.parametrize("shape", ["kimi", "tiny"])
def test_debug_check_short(monkeypatch, shape):
    """KDV_DEBUG=1 on the short path: an entry >= pool_slots (still inside the allocated pool) gives NaN results
    and KDV_ERR_PAGE; a valid table gives the ordinary result."""
    monkeypatch.setenv("KDV_DEBUG", "1")
    inp = (si.kimi(L=13, T=15, seed=4, dist="unit") if shape == "kimi" else
           si.make_inputs(**si.TINY_DIMS, L=20, T=7, seed=4, dist="unit", parent=[-1, 0, 0, 1, 1, 2, 2]))
    assert kernels(inp) == 1
    dev = si.to_device(inp)
    mask, _ = kdv.build_tree_mask(dev["parent"])
    dims = kdv.make_dims(**inp.dims())
    ws = torch.zeros((kdv.verify_workspace_bytes(dims, inp.T, inp.L),), dtype=torch.uint8, device="cuda")
    for pool, expect in ((inp.pool_slots - 1, kdv.KDV_ERR_PAGE), (inp.pool_slots, kdv.KDV_OK)):
        lse = torch.zeros((inp.T, inp.H), dtype=torch.float32, device="cuda")
        out, lse = kdv.verify_mla_attn(dims, dev["q_nope"], dev["q_rope"], dev["w_uk"], dev["w_uv"], dev["c_kv"],
                                       dev["k_pe"], dev["page_table"], inp.L, mask, lse=lse, workspace=ws,
                                       pool_slots=pool)
        torch.cuda.synchronize()
        assert kdv.debug_status(ws) == expect
        o = out.float().cpu().numpy()
        if expect == kdv.KDV_ERR_PAGE:
            assert np.isnan(o).all() and np.isnan(lse.cpu().numpy()).all()
        else:
            ref, _ = oracle.verify_inputs(inp)
            assert out_passes_qlat(o.astype(np.float64), ref, inp)[0]
