"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Mask: bit-exact.  Outputs: tests/parity.py (max|diff| <= 2e-2 relative to max(1, max|ref|) and <= 1% of
max|ref|); lse within the bf16-rounding bound derived in tests/parity.py.  Sizes span several 64-row KV tiles
with ragged tails, every tree-size edge (1, 32/33 -> two mask words, 64 = maximum), head counts that leave a partial 64-row query tile, forced
split counts, the full Kimi-shape workload (64 heads, 15 nodes, 5553-token prefix) in the launch
configuration the benchmark times, the context sweep (also over seeds 0-9 with unit and peaked scores, and a
one-bit mask mutation caught at 16384 tokens), a 200k-token prefix scattered over a 262144-slot
pool with unused slots poisoned to NaN (sampled heads), and one layer of the 8-head / 32-node /
131072-token verify step.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from tests.parity import lse_passes, lse_tolerance, out_errors, out_passes, out_passes_qlat

pytestmark = pytest.mark.gpu

kdv = pytest.importorskip("speculative_decoding_tree_parent_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _as_u32(t):
    return t.cpu().numpy().view(np.uint32)


def gpu_mask(parent):
    p = torch.from_numpy(np.asarray(parent, dtype=np.int32)).cuda()
    mask, status = kdv.build_tree_mask(p)
    torch.cuda.synchronize()
    return _as_u32(mask), int(status.item())


def run_gpu(inp, splits=None, mask_np=None, with_lse=True, dev=None):
    dev = dev or si.to_device(inp)
    old = os.environ.get("KDV_SPLITS")
    if splits is not None:
        os.environ["KDV_SPLITS"] = str(splits)
    try:
        if mask_np is None:
            mask, status = kdv.build_tree_mask(dev["parent"])
        else:
            mask = torch.from_numpy(np.ascontiguousarray(mask_np).view(np.int32)).cuda()
            status = None
        lse = torch.empty((inp.T, inp.H), dtype=torch.float32, device="cuda") if with_lse else None
        out, lse = kdv.verify_mla_attn(kdv.make_dims(**inp.dims()), dev["q_nope"], dev["q_rope"], dev["w_uk"],
                                       dev["w_uv"], dev["c_kv"], dev["k_pe"], dev["page_table"], inp.L, mask,
                                       lse=lse)
        torch.cuda.synchronize()
    finally:
        if splits is not None:
            if old is None:
                del os.environ["KDV_SPLITS"]
            else:
                os.environ["KDV_SPLITS"] = old
    if status is not None:
        assert int(status.item()) == 0
    return out.float().cpu().numpy().astype(np.float64), (None if lse is None else lse.cpu().numpy())


def check(inp, heads=None, **kw):
    got, glse = run_gpu(inp, **kw)
    ref, rlse = oracle.verify_inputs(inp, heads=heads)
    sel = slice(None) if heads is None else (slice(None), list(heads))
    ok, err = out_passes_qlat(got[sel], ref[sel], inp, heads)
    assert ok, f"output parity failed: {err}"
    if glse is not None:
        tol = lse_tolerance(inp, heads)
        lok, ratio = lse_passes(glse[sel], rlse[sel], tol[sel])
        assert lok, f"lse parity failed: max |dlse| / bound = {ratio:.3f}"
    return err


# ----------------------------------------------------------------------------------------------- mask
def test_mask_worked_example():
    mask, status = gpu_mask([-1, 0, 0, 1, 1, 2, 2])
    assert status == 0
    assert mask[:, 0].tolist() == [1, 3, 5, 11, 19, 37, 69]


@pytest.mark.parametrize("T", [1, 2, 7, 9, 15, 31, 32, 33, 63, 64])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mask_random_trees_bit_exact(T, seed):
    parent = si.random_parents(np.random.default_rng(seed), T)
    mask, status = gpu_mask(parent)
    ref, rstatus = oracle.tree_mask(parent)
    assert status == rstatus == 0
    assert np.array_equal(mask, ref)


@pytest.mark.parametrize("T", [16, 64])
def test_mask_chain_and_star(T):
    for parent in (np.arange(-1, T - 1), np.r_[-1, np.zeros(T - 1, dtype=np.int64)]):
        mask, status = gpu_mask(parent)
        ref, _ = oracle.tree_mask(parent)
        assert status == 0 and np.array_equal(mask, ref)


@pytest.mark.parametrize("parent", [[0, 0, 2, 2, 1], [-1, 0, -1, 7], [-1, 5, 1], [3]])
def test_mask_invalid_parents(parent):
    mask, status = gpu_mask(parent)
    ref, rstatus = oracle.tree_mask(parent)
    assert rstatus == oracle.KDV_ERR_TREE
    assert status == rstatus
    assert np.array_equal(mask, ref)


# ----------------------------------------------------------------------------------------------- tiny shape
@pytest.mark.parametrize("dist", si.DISTRIBUTIONS)
def test_tiny(dist):
    check(si.tiny(seed=0, dist=dist))


@pytest.mark.parametrize("L", [0, 1, 63, 64, 65, 200])
@pytest.mark.parametrize("splits", [None, 1, 3])
def test_tiny_prefix_lengths(L, splits):
    check(si.make_inputs(**si.TINY_DIMS, L=L, T=7, seed=L, dist="unit", parent=[-1, 0, 0, 1, 1, 2, 2]),
          splits=splits)


# ----------------------------------------------------------------------------------------------- Kimi shape
@pytest.mark.parametrize("dist", si.DISTRIBUTIONS)
def test_kimi_headline_workload(dist):
    """64 heads, 15 nodes, 5553-token prefix, default split plan (what the benchmark times)."""
    err = check(si.kimi(L=5553, T=15, seed=0, dist=dist))
    print(f"kimi L=5553 T=15 {dist}: max|d|={err['max_abs']:.3e} rel={err['rel']:.3e}")


@pytest.mark.parametrize("L", [0, 13, 51, 64, 113, 1663])
@pytest.mark.parametrize("T", [9, 15])
def test_kimi_small_prefix(L, T):
    check(si.kimi(L=L, T=T, seed=L + T, dist="unit"))


@pytest.mark.parametrize("L", [13, 1663, 3333, 5553, 16384])
@pytest.mark.parametrize("T", [9, 15])
def test_context_sweep(L, T):
    seed = [13, 1663, 3333, 5553, 16384].index(L) * 2 + (T == 15)
    check(si.kimi(L=L, T=T, seed=seed, dist="literal"))


# The context sweep over seeds 0-9 with the unit and peaked score distributions.  Above 13 tokens the oracle runs
# on four sampled heads (the kernel computes all 64; a head's rows span every query tile boundary class).
SWEEP_HEADS = (0, 21, 42, 63)


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("dist", ["unit", "peak4"])
@pytest.mark.parametrize("L", [13, 1663, 3333, 5553, 16384])
@pytest.mark.parametrize("T", [9, 15])
def test_context_sweep_seeds(L, T, dist, seed):
    check(si.kimi(L=L, T=T, seed=100 + seed, dist=dist), heads=None if L == 13 else SWEEP_HEADS)


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 64])
def test_kimi_tree_sizes(T):
    check(si.kimi(L=300, T=T, seed=100 + T, dist="unit"))


@pytest.mark.parametrize("H,T", [(1, 15), (3, 9), (8, 32), (16, 32), (32, 15), (100, 15), (128, 64)])
def test_kimi_head_counts(H, T):
    """Also covers each node-block size of the combine: 1 node per workgroup (8 heads x 32 nodes), 2 (16 x 32,
    32 x 15) and 4 (100 x 15, 128 x 64)."""
    inp = si.make_inputs(**dict(si.KIMI_DIMS, num_heads=H), L=700, T=T, seed=H, dist="unit")
    check(inp, heads=None if H <= 8 else [0, 1, H // 2, H - 1])


@pytest.mark.parametrize("T,splits", [(7, None), (33, None), (33, 5), (64, 9)])
def test_tiny_combine_node_blocks(T, splits):
    """64-wide shape, 4 heads: 7 nodes -> 1 node per combine workgroup, 33 and 64 -> 2 (the batched tests cover
    4); forced split counts give the combine's split groups unequal numbers of splits."""
    inp = si.make_inputs(**si.TINY_DIMS, L=300, T=T, seed=T, dist="unit")
    check(inp, splits=splits)


@pytest.mark.parametrize("shape", ["chain", "star"])
def test_kimi_chain_and_star(shape):
    T = 15
    parent = np.arange(-1, T - 1) if shape == "chain" else np.r_[-1, np.zeros(T - 1, dtype=np.int64)]
    check(si.kimi(L=900, T=T, seed=7, dist="peak4", parent=parent))


@pytest.mark.parametrize("splits", [1, 2, 3, 5, 13, 27])
def test_forced_split_counts(splits):
    check(si.kimi(L=1663, T=15, seed=21, dist="unit"), splits=splits)


def test_permuted_pool_bit_identical_and_deterministic():
    """Same logical rows, contiguous vs scattered over a NaN-poisoned pool: identical bits.  Any NaN in the
    output would mean a row was gathered from an unused slot."""
    a = si.kimi(L=2500, T=15, seed=31, dist="unit")
    b = si.kimi(L=2500, T=15, seed=31, dist="unit")
    P = 8192
    rng = np.random.default_rng(5)
    slots = rng.permutation(P)[:a.N].astype(np.int32)
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


def test_long_fragmented_200k():
    """200000-token prefix over a random permutation of a 262144-slot pool, unused slots NaN; sampled heads."""
    inp = si.long_fragmented(seed=0, dist="literal", poison_unused=True)
    err = check(inp, heads=[0, 29, 63])
    print(f"200k fragmented: max|d|={err['max_abs']:.3e} rel={err['rel']:.3e}")


def test_long_fragmented_200k_unit():
    inp = si.long_fragmented(seed=1, dist="unit", poison_unused=True)
    check(inp, heads=[5, 40])


@pytest.mark.parametrize("layer", [0, 60])
def test_full61_layer(layer):
    """One layer of the 61-layer verify step: 8 heads, 32 nodes (depth <= 16), 131072-token scattered prefix."""
    parent, table = si.full61_shared()
    inp = si.full61_layer(layer, parent, table)
    check(inp)


def test_lse_optional():
    inp = si.tiny(seed=3, dist="unit")
    got, lse = run_gpu(inp, with_lse=False)
    assert lse is None
    ref, _ = oracle.verify_inputs(inp)
    assert out_passes(got, ref)[0]


@pytest.mark.parametrize("mutation", ["drop_root_of_deepest", "add_non_ancestor"])
def test_mutated_mask_fails_parity(mutation):
    """The parity criterion has teeth on the device path: a one-bit mask error is caught at L=13."""
    inp = si.kimi(L=13, T=15, seed=11, dist="unit")
    mask, _ = oracle.tree_mask(inp.parent)
    depth = [len(oracle.ancestor_path(inp.parent, t)) for t in range(inp.T)]
    t = int(np.argmax(depth))
    bad = mask.copy()
    if mutation == "drop_root_of_deepest":
        bad[t, 0] &= ~np.uint32(1)
    else:
        anc = set(oracle.ancestor_path(inp.parent, t))
        j = next(j for j in range(inp.T) if j not in anc)
        bad[t, 0] |= np.uint32(1) << np.uint32(j)
    got, _ = run_gpu(inp, mask_np=bad)
    ref, _ = oracle.verify_inputs(inp)
    ok, err = out_passes(got, ref)
    assert not ok, f"mutated mask passed: {err}"
    good, _ = run_gpu(inp)
    assert out_passes(good, ref)[0]


def _plant_peak(inp, t, j, h=0, alpha=16.0):
    """Make tree key j score about alpha above every prefix key for node t in head h: its latent and rotary rows
    become alpha times node t's unit-normalised absorbed query (the same modified inputs go to the oracle)."""
    qlat = inp.f32("q_nope")[t, h].astype(np.float64) @ inp.f32("w_uk")[h].astype(np.float64)
    qr = inp.f32("q_rope")[t, h].astype(np.float64)
    norm = np.sqrt(qlat @ qlat + qr @ qr)
    row = inp.page_table[inp.L + j]
    inp.c_kv[row] = si.f32_to_bf16_bits((alpha * qlat / norm).astype(np.float32))
    inp.k_pe[row] = si.f32_to_bf16_bits((alpha * qr / norm).astype(np.float32))
    inp._f32.clear()


@pytest.mark.parametrize("mutation", ["drop_root_of_deepest", "add_non_ancestor"])
def test_mutated_mask_fails_parity_long_context(mutation):
    """A one-bit mask error is caught at 16384 prefix tokens too, where one tree key is a small share of the
    softmax mass: the key the mutation concerns is made to dominate the affected node's scores in head 0."""
    inp = si.kimi(L=16384, T=15, seed=12, dist="unit")
    mask, _ = oracle.tree_mask(inp.parent)
    depth = [len(oracle.ancestor_path(inp.parent, t)) for t in range(inp.T)]
    t = int(np.argmax(depth))
    anc = set(oracle.ancestor_path(inp.parent, t))
    bad = mask.copy()
    if mutation == "drop_root_of_deepest":
        j = 0
        bad[t, 0] &= ~np.uint32(1)
    else:
        j = next(j for j in range(inp.T) if j not in anc)
        bad[t, 0] |= np.uint32(1) << np.uint32(j)
    _plant_peak(inp, t, j)
    ref, _ = oracle.verify_inputs(inp, heads=[0])
    got, _ = run_gpu(inp, mask_np=bad)
    ok, err = out_passes(got[:, [0]], ref[:, [0]])
    assert not ok, f"mutated mask passed: {err}"
    good, _ = run_gpu(inp)
    assert out_passes(good[:, [0]], ref[:, [0]])[0]


def test_invalid_tree_reports_status():
    p = torch.tensor([-1, 0, 5, 1], dtype=torch.int32, device="cuda")
    _, status = kdv.build_tree_mask(p)
    torch.cuda.synchronize()
    assert int(status.item()) == kdv.KDV_ERR_TREE
