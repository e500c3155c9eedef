"""The lse tolerance of the GPU parity tests (tests/parity.py), checked on the CPU.

- bf16_round_f64 rounds exactly as torch's float32 -> bfloat16 conversion on float32 values, ties included;
- at the 64-head, 15-node, 5553-token shape the bound is the size of the bf16 rounding of the absorbed
  query alone (well under the flat 1e-2 the lse was first compared with on unit scores);
- an lse off by twice the bound fails, and the device's own rounding of q_lat, emulated here on the CPU
  (float32 accumulation, bf16 round to nearest even, exact scores), passes.
"""
import copy

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from tests import parity
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


# ------------------------------------------------------------------ output effect of the q_lat rounding
def _scaled_identity_inputs(scale_w: float, seed: int = 5):
    """Oracle-only inputs (Dn = R) whose W_UK[h] is scale_w times the identity, so that q_lat = scale_w q_nope."""
    inp = si.make_inputs(num_heads=3, qk_nope_dim=64, qk_rope_dim=16, kv_lora_rank=64, v_head_dim=32, L=40, T=7,
                         seed=seed, dist="peak4")
    w = np.zeros((inp.H, inp.Dn, inp.R), dtype=np.float32)
    for h in range(inp.H):
        w[h] = scale_w * np.eye(inp.Dn, inp.R, dtype=np.float32)
    inp.w_uk = si.f32_to_bf16_bits(w)
    inp._f32.clear()
    return inp


def test_qlat_output_effect_matches_the_oracle_on_rounded_queries():
    # q_lat = 3 q_nope is not a bfloat16 value in general; the same oracle on W_UK = I and q_nope = bf16(3 q_nope)
    # sees exactly the rounded q_lat, so the difference of the two oracle outputs is the effect to predict.
    inp = _scaled_identity_inputs(3.0)
    rounded = copy.deepcopy(inp)
    q3 = 3.0 * inp.f32("q_nope").astype(np.float64)
    rounded.q_nope = si.f32_to_bf16_bits(bf16_round_f64(q3)[0].astype(np.float32))
    rounded.w_uk = si.f32_to_bf16_bits(np.stack([np.eye(inp.Dn, inp.R, dtype=np.float32)] * inp.H))
    rounded._f32.clear()
    base, _ = oracle.verify_inputs(inp)
    moved, _ = oracle.verify_inputs(rounded)
    eff = parity.qlat_output_effect(inp)
    assert np.abs(moved - base).max() > 1e-4            # the rounding matters on these inputs
    np.testing.assert_allclose(eff, moved - base, rtol=0, atol=1e-12)


def test_qlat_output_effect_vanishes_for_representable_queries():
    inp = _scaled_identity_inputs(1.0)                   # q_lat = q_nope: already bfloat16
    assert np.abs(parity.qlat_output_effect(inp)).max() == 0.0


def test_qlat_criterion_still_rejects_wrong_outputs():
    inp = si.kimi(L=300, T=9, seed=108, dist="peak4")
    heads = (0, 63)
    ref, _ = oracle.verify_inputs(inp, heads=heads)
    sel = (slice(None), list(heads))
    bad = ref.copy()
    bad[4, 63] *= 1.05
    assert not parity.out_passes_qlat(bad[sel], ref[sel], inp, heads)[0]
    assert not parity.out_passes_qlat(np.zeros_like(ref[sel]), ref[sel], inp, heads)[0]
    assert parity.out_passes_qlat(ref[sel], ref[sel], inp, heads)[0]
