"""GPU parity over seeded random shapes: each case draws the shape (64-wide test dims or the Kimi dims with 1..128
heads), the prefix length (0..3000, with a bias to one-tile and tile-boundary lengths), the tree size (1..64), the
score distribution, a forced split count (sometimes), and a contiguous or scattered, NaN-poisoned pool.  Each
output and lse is checked against the oracle on up to four sampled heads, under the same bounds as the other
parity tests.  The cases cover the three-kernel path, the single short-sequence kernel and forced split plans
without naming them.  Twelve more cases draw batches of 2..16 requests with their own prefix lengths and tree sizes.
"""
import numpy as np
import pytest
import torch

import synth_inputs as si
from tests.test_gpu_parity import check

pytestmark = pytest.mark.gpu

kdv = pytest.importorskip("speculative_decoding_tree_parent_amd")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def draw_case(k: int):
    rng = np.random.default_rng([2026, k])
    kimi = rng.random() < 0.7
    dims = dict(si.KIMI_DIMS, num_heads=int(rng.choice([1, 2, 5, 8, 16, 33, 64, 100, 128]))) if kimi \
        else dict(si.TINY_DIMS)
    T = int(rng.choice([1, 2, 7, 9, 15, 16, 31, 32, 33, 48, 64]))
    pick = rng.random()
    if pick < 0.35:
        L = int(rng.integers(0, max(1, 65 - T)))  # one tile (the short path when T <= 32)
    elif pick < 0.6:
        L = int(rng.choice([63, 64, 65, 127, 128, 129])) - T  # around tile boundaries
        L = max(L, 0)
    else:
        L = int(rng.integers(0, 3000))
    dist = str(rng.choice(si.DISTRIBUTIONS))
    splits = int(rng.choice([1, 2, 3, 7])) if rng.random() < 0.2 else None
    scattered = rng.random() < 0.3
    H = dims["num_heads"]
    heads = None if H <= 4 else sorted({0, H - 1, *map(int, rng.choice(H, size=2, replace=False))})
    return dims, L, T, dist, splits, scattered, heads


@pytest.mark.parametrize("k", range(40))
def test_random_shape(k):
    dims, L, T, dist, splits, scattered, heads = draw_case(k)
    pool = None
    if scattered:
        pool = int(np.random.default_rng([7, k]).integers(L + T, 2 * (L + T) + 64))
    inp = si.make_inputs(**dims, L=L, T=T, seed=1000 + k, dist=dist, pool_slots=pool, poison_unused=scattered)
    print(f"case {k}: H={dims['num_heads']} R={dims['kv_lora_rank']} L={L} T={T} {dist} splits={splits} "
          f"scattered={scattered} heads={heads}", flush=True)
    check(inp, heads=heads, splits=splits)


# Batches: 2..16 requests with their own prefix lengths (0..2000) and tree sizes (1..64) over one pool, each request's
# slice against the oracle run on that request alone; sometimes with a forced split count.
@pytest.mark.parametrize("k", range(12))
def test_random_batch(k):
    from tests.test_gpu_batch import check_batch
    rng = np.random.default_rng([2027, k])
    dims = dict(si.KIMI_DIMS, num_heads=int(rng.choice([1, 8, 16, 64]))) if rng.random() < 0.6 else dict(si.TINY_DIMS)
    C = int(rng.integers(2, 17))
    Ts = [int(t) for t in rng.choice([1, 3, 9, 15, 32, 33, 64], size=C)]
    Ls = [int(x) for x in (rng.integers(0, 2000, size=C) * (rng.random(C) < 0.8))]
    dist = str(rng.choice(["literal", "unit"]))
    splits = int(rng.choice([2, 5])) if rng.random() < 0.25 else None
    H = dims["num_heads"]
    heads = None if H <= 4 else [0, H - 1]
    print(f"batch {k}: H={H} R={dims['kv_lora_rank']} C={C} L={Ls} T={Ts} {dist} splits={splits}", flush=True)
    check_batch(si.batch_inputs(dims, Ls, Ts, seed=2000 + k, dist=dist), heads=heads, splits=splits)
