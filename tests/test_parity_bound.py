"""The lse tolerance of the GPU parity tests (tests/parity.py), checked on the CPU.

- bf16_round_f64 rounds exactly as torch's float32 -> bfloat16 conversion on float32 values, ties included;
- at the 64-head, 15-node, 5553-token shape the bound is the size of the bf16 rounding of the absorbed
  query alone (well under the flat 1e-2 the lse was first compared with on unit scores);
- an lse off by twice the bound fails, and the device's own rounding of q_lat, emulated here on the CPU
  (float32 accumulation, bf16 round to nearest even, exact scores), passes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from tests.parity import LSE_SLACK, bf16_round_f64, lse_passes, lse_tolerance


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    # exact ties: the bf16 midpoint between two neighbours (bit 15 set, low 15 bits zero)
    ties = ((rng.integers(0x3000, 0x4F00, 4000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got, ulp, dist = bf16_round_f64(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.all(np.abs(got - x) <= ulp / 2)
    assert np.all(dist[len(x) - 2 * len(ties):] == 0)


@pytest.mark.parametrize("dist,lo,hi", [("unit", 0.005, 0.015), ("peak4", 0.02, 0.06), ("literal", 1e-3, 1.2e-3)])
def test_bound_size_at_headline_shape(dist, lo, hi):
    inp = si.kimi(L=5553, T=15, seed=0, dist=dist)
    tol = lse_tolerance(inp, heads=[0, 31, 63])[:, [0, 31, 63]]
    assert np.all(tol >= LSE_SLACK)
    assert lo <= tol.min() and tol.max() <= hi, (tol.min(), tol.max())


@pytest.mark.parametrize("dist", ["unit", "peak4"])
def test_emulated_device_rounding_passes_and_planted_error_fails(dist):
    inp = si.kimi(L=700, T=15, seed=3, dist=dist)
    heads = [0, 9, 63]
    tol = lse_tolerance(inp, heads)[:, heads]
    _, ref = oracle.verify_inputs(inp, heads=heads)
    ref = ref[:, heads]
    mask, _ = oracle.tree_mask(inp.parent)
    C = inp.f32("c_kv")[inp.page_table].astype(np.float64)
    Kp = inp.f32("k_pe")[inp.page_table].astype(np.float64)
    emu = np.empty_like(ref)
    for j, h in enumerate(heads):
        ql32 = inp.f32("q_nope")[:, h] @ inp.f32("w_uk")[h]
        qb = si.bf16_bits_to_f32(si.f32_to_bf16_bits(ql32)).astype(np.float64)
        s = inp.sm_scale * (qb @ C.T + inp.f32("q_rope")[:, h].astype(np.float64) @ Kp.T)
        for t in range(inp.T):
            vis = np.r_[np.ones(inp.L, bool), [(int(mask[t, 0]) >> i) & 1 == 1 for i in range(inp.T)]]
            sv = s[t, vis]
            emu[t, j] = sv.max() + np.log(np.exp(sv - sv.max()).sum())
    ok, ratio = lse_passes(emu, ref, tol)
    assert ok and ratio < 0.5, ratio
    bad = emu.copy()
    bad[4, 1] = ref[4, 1] + 2 * tol[4, 1]
    assert not lse_passes(bad, ref, tol)[0]
