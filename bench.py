#!/usr/bin/env python3
"""Benchmark of DDTree tree-verify MLA attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload kimi5553|long200k|full61|kimi:L:T] [--no-extra]

A step is one pass of the whole hot path over one batch of synthetic input: the ancestor mask of the draft
tree and tree-verify attention for one layer (kdv_verify_mla_attn: q absorption, split-KV MFMA pass, split
combine fused with the W_UV up-projection); for `full61` a step is one mask and 61 layers.

The default run measures the headline workload (64 heads, 15 nodes, 5553-token prefix) for the line's `value`,
then every other configuration of the metric with the same measurement, under `configs`: the context sweep
(prefix 13 / 1663 / 3333 / 5553 / 16384 x trees of 9 / 15 nodes), the 200000-token prefix over a scattered
262144-slot pool, and the 61-layer step (8 heads, 32 nodes, 131072 tokens).  `--no-extra` measures one workload.

Timing: W eager warm-up steps, then the K timed steps are captured in one HIP graph (so host launch cost is
not counted) and replayed once between two device synchronisations, timed with HIP events on the stream the
kernels run on.  "Cold" rotates the steps over distinct copies of the layer's buffers (together more than
512 MiB, twice the 256 MiB Infinity Cache, as a real multi-layer model would; `buffers` states how much the K
timed steps touched); "hot" reuses one copy.  Each kernel's own time comes from HIP events that the launch itself
stamps with the kernel's start and end (hipExtLaunchKernelGGL, through kdv_verify_mla_attn_profiled), over eager
launches of the same cold steps; those also give the per-layer p10 / p50 / p90.
Work counts are algorithmic: masked tree entries and padding are not counted.

Profile evidence (bash profile_bench.sh [workload]) is summarised by `--summarize-profile DIR`;
`roofline.traffic` is read from the committed counter summary only while its hash of the kernel source matches.

Prints ONE JSON line.  Inputs are seeded synthetic data with the shapes of the pages' workloads.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import csv
import hashlib
import re
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tree-verify MLA attn µs/layer + TFLOP/s (% MFMA peak), 64 heads, 15 nodes, ctx 5553"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA, vendor figure
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, vendor figure
COLD_BYTES = 576 << 20
KERNEL_SOURCES = ("speculative_decoding_tree_parent_amd/csrc/verify.hip",
                  "speculative_decoding_tree_parent_amd/csrc/common.h",
                  "speculative_decoding_tree_parent_amd/csrc/tree_mask.h",
                  "speculative_decoding_tree_parent_amd/csrc/tree.hip")
KERNELS = ("tree_mask_kernel", "q_absorb_kernel", "splitkv_kernel", "combine_up_kernel", "short_verify_kernel",
           "tree_accept_kernel", "draft_tree_kernel", "merge_states_kernel")
KERNEL_NAMES = ["q_absorb", "splitkv", "combine_up"]
SHORT_KERNEL_NAMES = ["short_verify"]  # a call whose L + T rows fit in one KV tile (T <= 32): one kernel


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------------------ work model
def depths(parent):
    d = []
    for t in range(len(parent)):
        k, j = 0, t
        while parent[j] != -1:
            j = int(parent[j])
            k += 1
        d.append(k)
    return np.array(d)


def work(H, Dn, Dr, R, Dv, L, T, parent):
    """Algorithmic FLOPs and HBM bytes of one layer (visible rows only)."""
    n_t = L + depths(parent) + 1
    sn = float(n_t.sum())
    f_absorb = 2.0 * H * T * Dn * R
    f_scores = 2.0 * H * sn * (R + Dr)
    f_pv = 2.0 * H * sn * R
    f_up = 2.0 * H * T * R * Dv
    N = L + T
    b = N * (R + Dr) * 2 + H * (Dn + Dv) * R * 2 + T * H * (Dn + Dr) * 2 + T * H * Dv * 2 + 4 * N
    return dict(flops=f_absorb + f_scores + f_pv + f_up, flops_splitkv=f_scores + f_pv, bytes=float(b),
                bytes_splitkv=float(N * (R + Dr) * 2 + T * H * (R + Dr) * 2 + 4 * N))


# ------------------------------------------------------------------------------------------------ HIP events
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")  # by soname: the runtime torch already loaded
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(e))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return e.value

    def record(self, e, stream):
        rc = self.lib.hipEventRecord(e, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        ms = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)


# ------------------------------------------------------------------------------------------------ workloads
SWEEP_L = (13, 1663, 3333, 5553, 16384)
SWEEP_T = (9, 15)


def clone_layer(t):
    return {k: v.clone() for k, v in t.items()}


def parse_workload(name):
    """(kind, L, T, seed) for a workload name: kimi5553, long200k, full61, or kimi:L:T (64 heads, contiguous cache,
    the sweep's seed for that point: 2 * index(L) + index(T) when (L, T) is a sweep point, else 0)."""
    if name in ("kimi5553", "long200k", "full61"):
        return name, None, None, None
    parts = name.split(":")
    if len(parts) == 3 and parts[0] == "kimi":
        L, T = int(parts[1]), int(parts[2])
        seed = 2 * SWEEP_L.index(L) + SWEEP_T.index(T) if (L in SWEEP_L and T in SWEEP_T) else 0
        return "kimi", L, T, seed
    raise SystemExit(f"unknown workload {name!r} (kimi5553, long200k, full61, sweep, or kimi:L:T)")


def profile_tag(workload):
    """File-name form of a workload name (profiles/<kernel>_<tag>_*.md)."""
    return workload.replace(":", "_L", 1).replace(":", "_T", 1)


class Setup:
    """Device buffers of one workload: the layer buffer sets of the cold rotation, the hot set, and the shared
    page table and tree."""


def setup_workload(name, torch, si, dev):
    kind, Lk, Tk, seed = parse_workload(name)
    S = Setup()
    S.name = name
    if kind == "full61":
        parent_np, table_np = si.full61_shared()
        S.H, S.Dn, S.Dr, S.R, S.Dv = 8, 128, 64, 512, 128
        S.L, S.T, P = 131072, 32, 262144
        S.scale = 1.0 / math.sqrt(S.Dn + S.Dr)
        S.desc = ("verify-step attention, 61 layers x 8 heads, 32-node tree (depth <= 16), 131072-token prefix "
                  "scattered over a 262144-slot pool, per-layer buffers")
        gen = torch.Generator(device=dev)
        layers = []
        for layer in range(61):
            gen.manual_seed(1000 + layer)

            def rnd(shape, std):
                x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std
                return x.to(torch.bfloat16).view(torch.int16)
            layers.append(dict(q_nope=rnd((S.T, S.H, S.Dn), S.Dn ** -0.5), q_rope=rnd((S.T, S.H, S.Dr), S.Dr ** -0.5),
                               w_uk=rnd((S.H, S.Dn, S.R), S.R ** -0.5), w_uv=rnd((S.H, S.Dv, S.R), S.R ** -0.5),
                               c_kv=rnd((P, S.R), S.R ** -0.5), k_pe=rnd((P, S.Dr), S.Dr ** -0.5)))
        S.layers_per_step = 61
        S.cold_sets, S.hot_sets = [layers], [layers[:1] * 61]
        S.parent_t = torch.from_numpy(parent_np.astype(np.int32)).to(dev)
        S.table_t = torch.from_numpy(table_np.astype(np.int32)).to(dev)
        S.pool_slots, S.parent_np, S.inp = P, parent_np, None
        per_layer = sum(v.numel() * v.element_size() for v in layers[0].values())
        S.n_cold, S.set_bytes = 1, 61 * per_layer
        return S
    if kind == "kimi5553":
        inp = si.kimi(L=5553, T=15, seed=0, dist="literal")
        S.desc = ("tree-verify MLA attention (absorbed), 64 heads, 15-node random tree, 5553-token prefix, "
                  "contiguous bf16 latent cache, dims nope/rope/rank/v = 128/64/512/128")
    elif kind == "long200k":
        inp = si.long_fragmented(seed=0, dist="literal")
        S.desc = ("tree-verify MLA attention (absorbed), 64 heads, 15-node random tree, 200000-token prefix "
                  "scattered over a 262144-slot page_size=1 pool")
    else:
        inp = si.kimi(L=Lk, T=Tk, seed=seed, dist="literal")
        S.desc = (f"tree-verify MLA attention (absorbed), 64 heads, {Tk}-node random tree, {Lk}-token prefix, "
                  f"contiguous bf16 latent cache (seed {seed})")
    S.inp = inp
    S.H, S.Dn, S.Dr, S.R, S.Dv, S.L, S.T = inp.H, inp.Dn, inp.Dr, inp.R, inp.Dv, inp.L, inp.T
    S.parent_np, S.scale, S.pool_slots = inp.parent, inp.sm_scale, inp.pool_slots
    d0 = si.to_device(inp, dev)
    S.parent_t, S.table_t = d0.pop("parent"), d0.pop("page_table")
    S.set_bytes = sum(v.numel() * v.element_size() for v in d0.values())
    S.n_cold = max(2, math.ceil(COLD_BYTES / S.set_bytes))
    cold = [d0] + [clone_layer(d0) for _ in range(S.n_cold - 1)]
    S.cold_sets, S.hot_sets = [[c] for c in cold], [[d0]]
    S.layers_per_step = 1
    return S


def measure(S, args, torch, kdv, dev, hip, stream, sh, note, K, Wm, full=True, reps=1):
    """Times one workload: K steps of the cold rotation and of one hot buffer set, each captured in one HIP graph,
    and the kernels of each call over eager cold steps (kernel-stamped HIP events).  With reps > 1 each graph is
    replayed reps times after its untimed replay and the median replay is taken (the other configurations of the
    metric, whose K steps last well under a millisecond).  Returns (result dict, state for the extra rows of the
    headline)."""
    H, Dn, Dr, R, Dv, L, T = S.H, S.Dn, S.Dr, S.R, S.Dv, S.L, S.T
    lps = S.layers_per_step
    dims = kdv.make_dims(H, Dn, Dr, R, Dv, S.scale)
    W = (T + 31) // 32
    mask_t = torch.empty((T, W), dtype=torch.int32, device=dev)
    status_t = torch.zeros((1,), dtype=torch.int32, device=dev)
    out_t = torch.empty((T, H, Dv), dtype=torch.bfloat16, device=dev)
    lse_t = torch.empty((T, H), dtype=torch.float32, device=dev)
    ws_bytes = kdv.verify_workspace_bytes(dims, T, L)
    ws_t = torch.zeros((ws_bytes,), dtype=torch.uint8, device=dev)
    splits = kdv.kdv_verify_num_splits(dims, T, L)
    nk = kdv.kdv_verify_kernel_count(dims, T, L)
    names = KERNEL_NAMES if nk == 3 else SHORT_KERNEL_NAMES
    assert nk == len(names)
    wk = work(H, Dn, Dr, R, Dv, L, T, S.parent_np)

    def ptrs(t):
        return [t["q_nope"].data_ptr(), t["q_rope"].data_ptr(), t["w_uk"].data_ptr(), t["w_uv"].data_ptr(),
                t["c_kv"].data_ptr(), t["k_pe"].data_ptr()]
    cold_ptrs = [[ptrs(t) for t in s] for s in S.cold_sets]
    hot_ptrs = [[ptrs(t) for t in s] for s in S.hot_sets]
    fx = dict(pt=S.table_t.data_ptr(), mask=mask_t.data_ptr(), out=out_t.data_ptr(), lse=lse_t.data_ptr(),
              ws=ws_t.data_ptr(), parent=S.parent_t.data_ptr(), status=status_t.data_ptr())
    ps = S.pool_slots

    def step(set_ptrs):
        # The first layer's call builds the step's tree mask (one extra block of its first kernel); the other
        # layers of the step reuse it.
        for i, lp in enumerate(set_ptrs):
            if i == 0:
                rc = kdv.kdv_verify_mla_attn_tree(dims, *lp, ps, fx["pt"], L, T, fx["parent"], fx["mask"],
                                                  fx["status"], fx["out"], fx["lse"], fx["ws"], ws_bytes, sh)
            else:
                rc = kdv.kdv_verify_mla_attn(dims, *lp, ps, fx["pt"], L, T, fx["mask"], fx["out"], fx["lse"],
                                             fx["ws"], ws_bytes, sh)
            if rc:
                raise kdv.KdvError(rc, "kdv_verify_mla_attn")

    def run_steps(sets, n, fn=step):
        for i in range(n):
            fn(sets[i % len(sets)])

    def timed(sets, n, fn=step, r=1):
        """Device time (ms) of n steps: graph-captured unless --no-graph; the median of r timed replays."""
        e0, e1 = hip.event(), hip.event()
        if args.no_graph:
            torch.cuda.synchronize()
            hip.record(e0, sh)
            run_steps(sets, n, fn)
            hip.record(e1, sh)
            return hip.elapsed_ms(e0, e1)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run_steps(sets, n, fn)
        g.replay()                       # untimed replay: graph upload, first-touch
        torch.cuda.synchronize()
        ms = []
        for _ in range(r):
            hip.record(e0, sh)
            g.replay()
            hip.record(e1, sh)
            ms.append(hip.elapsed_ms(e0, e1))
        torch.cuda.synchronize()
        return float(np.median(ms))

    per_step = {n: lps for n in names}  # (the mask is built inside the first call)
    per_step_eager = dict(tree_mask=1, **per_step)

    def note_timed(what, counts, n, r=1):
        if args.no_graph:
            note(f"{S.name}: {what}, eager", counts, n)
        else:
            note(f"{S.name}: graph {what}, upload replay", counts, n)
            note(f"{S.name}: graph {what}, timed replay", counts, n * r)

    log(f"[bench] {S.name}: warmup {Wm} steps")
    torch.cuda.synchronize()
    run_steps(cold_ptrs, Wm)
    torch.cuda.synchronize()
    if int(status_t.item()) != 0:
        raise SystemExit("tree status not OK")
    note(f"{S.name}: warm-up", per_step, Wm)
    log(f"[bench] {S.name}: timing {K} steps (cold)")
    ms_cold = timed(cold_ptrs, K, r=reps)
    note_timed("cold", per_step, K, reps)
    log(f"[bench] {S.name}: timing {K} steps (hot)")
    ms_hot = timed(hot_ptrs, K, r=reps)
    note_timed("hot", per_step, K, reps)

    # per-kernel device time and per-step spread: events stamped by each kernel's own dispatch, eager launches
    # queued behind a spin kernel so that they run back to back as in the graph
    log(f"[bench] {S.name}: per-kernel timing")
    EvArr = ctypes.c_void_p * (2 * nk)
    Kp = min(K, max(1, 400 // lps))
    ev_list = [EvArr(*[hip.event() for _ in range(2 * nk)]) for _ in range(Kp * lps)]

    def step_ev(set_ptrs, evs):
        rc = kdv.kdv_build_tree_mask(fx["parent"], T, fx["mask"], fx["status"], sh)
        if rc:
            raise kdv.KdvError(rc, "kdv_build_tree_mask")
        for lp, ev in zip(set_ptrs, evs):
            rc = kdv.kdv_verify_mla_attn_profiled(dims, *lp, ps, fx["pt"], L, T, fx["mask"], fx["out"], fx["lse"],
                                                  fx["ws"], ws_bytes, sh, ctypes.addressof(ev))
            if rc:
                raise kdv.KdvError(rc, "kdv_verify_mla_attn_profiled")
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2.4e9 * 0.05))
    for i in range(Kp):
        step_ev(cold_ptrs[i % len(cold_ptrs)], ev_list[i * lps:(i + 1) * lps])
    torch.cuda.synchronize()
    note(f"{S.name}: eager cold, kernel events", per_step_eager, Kp)
    samples = {n: [] for n in names}
    for ev in ev_list:
        for k, n in enumerate(names):
            samples[n].append(1e3 * hip.elapsed_ms(ev[2 * k], ev[2 * k + 1]))
    # a layer's span: first kernel's start to last kernel's end (per layer of every eager step)
    spans = [1e3 * hip.elapsed_ms(ev[0], ev[2 * nk - 1]) for ev in ev_list]
    kern_us = {n: float(np.mean(v)) for n, v in samples.items()}
    kern_pct = {n: [round(float(np.percentile(v, 10)), 3), round(float(np.percentile(v, 90)), 3)]
                for n, v in samples.items()}

    us_cold = 1e3 * ms_cold / (K * lps)
    us_hot = 1e3 * ms_hot / (K * lps)
    tf_cold = wk["flops"] / (us_cold * 1e-6) / 1e12
    tf_hot = wk["flops"] / (us_hot * 1e-6) / 1e12
    gbs = wk["bytes"] / (us_cold * 1e-6) / 1e9
    touched = min(K, S.n_cold) * S.set_bytes if lps == 1 else S.set_bytes
    res = {
        "workload": S.desc, "heads": H, "tree_nodes": T, "prefix_len": L, "layers_per_step": lps,
        "kv_splits": splits, "kernels_per_call": nk,
        "us_per_layer": round(us_cold, 3),
        "tflops": round(tf_cold, 3), "frac_bf16_peak": round(tf_cold / PEAK_BF16_TFLOPS, 4),
        "hbm_gbs": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "us_per_layer_eager_p10_p50_p90": [round(float(np.percentile(spans, q)), 3) for q in (10, 50, 90)],
        "hot": {"us_per_layer": round(us_hot, 3), "tflops": round(tf_hot, 3),
                "frac_bf16_peak": round(tf_hot / PEAK_BF16_TFLOPS, 4)},
        "kernels_us": {k: round(v, 3) for k, v in kern_us.items()},
        "kernels_us_p10_p90": kern_pct,
        "work_per_layer": {"gflop": round(wk["flops"] / 1e9, 4), "mbytes": round(wk["bytes"] / 1e6, 3)},
        "buffers": (f"cold: {S.n_cold} distinct layer buffer sets of {S.set_bytes / 2**20:.1f} MiB in rotation, "
                    f"{touched / 2**20:.0f} MiB touched by the {K} timed steps; hot: one set" if lps == 1 else
                    f"cold: 61 distinct layers ({S.set_bytes / 2**30:.2f} GiB) per step; hot: layer 0 61 times"),
        "timing": ("eager" if args.no_graph else "one HIP graph of K steps" if reps == 1 else
                   f"one HIP graph of K steps, median of {reps} replays") +
                  "; eager p10/p50/p90: first kernel's start to last kernel's end of each layer, kernel-stamped events",
    }
    state = dict(dims=dims, fx=fx, ws_bytes=ws_bytes, cold_ptrs=cold_ptrs, out_t=out_t, lse_t=lse_t, wk=wk,
                 kern_us=kern_us, timed=timed, step=step, note_timed=note_timed, run_steps=run_steps, names=names)
    return res, state


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="kimi5553",
                    help="kimi5553 (default, with the other configurations as extra keys), long200k, full61, or "
                         "kimi:L:T (64 heads, L-token contiguous prefix, T-node tree)")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline workload only: no context sweep, 200k and 61-layer rows, no batched row")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of one HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (the reference for FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="print the markdown summaries of a profile_bench.sh run and exit (no GPU needed)")
    args = ap.parse_args()
    parse_workload(args.workload)
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.workload)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the tree-verify attention of one layer runs on a single "
                                   "MI355X; splitting it over several GPUs (heads, or the KV sequence with one "
                                   "exchange of split partials) is not implemented", "n_gpus": args.gpus}),
              flush=True)
        sys.exit(2)

    import torch
    import synth_inputs as si
    import speculative_decoding_tree_parent_amd as kdv

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (gfx950)")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        copy_calibration(torch, dev)
        return
    hip = Hip()
    stream = torch.cuda.Stream(device=dev)      # default priority; graphs cannot capture the null stream
    sh = stream.cuda_stream
    with torch.cuda.stream(stream):
        run(args, torch, si, kdv, dev, hip, stream, sh)


def run(args, torch, si, kdv, dev, hip, stream, sh):
    ledger = []

    def note(phase, counts, n=1):
        names = {p for p, _ in ledger}
        name, i = phase, 2
        while name in names:  # phase names are unique keys
            name, i = f"{phase} #{i}", i + 1
        ledger.append([name, {f"{k}_kernel": v * n for k, v in counts.items() if v}])

    K, Wm = args.steps, args.warmup
    log(f"[bench] workload {args.workload}: building inputs")
    S = setup_workload(args.workload, torch, si, dev)
    res, st = measure(S, args, torch, kdv, dev, hip, stream, sh, note, K, Wm)
    H, Dn, Dr, R, Dv, L, T = S.H, S.Dn, S.Dr, S.R, S.Dv, S.L, S.T
    lps = S.layers_per_step
    dims, fx, ws_bytes, wk, kern_us = st["dims"], st["fx"], st["ws_bytes"], st["wk"], st["kern_us"]
    ps = S.pool_slots

    # The prefix/tail split of the same step: per layer, a prefix-only call over the L prefix rows, the tree call
    # over the T tail rows (L = 0) and the LSE merge of the two (one stream, so they share a workspace).
    split_bufs = [torch.empty_like(st["out_t"]), torch.empty_like(st["lse_t"]), torch.empty_like(st["out_t"]),
                  torch.empty_like(st["lse_t"])]
    split_ptr = [t.data_ptr() for t in split_bufs]

    def split_step(set_ptrs):
        rc = kdv.kdv_build_tree_mask(fx["parent"], T, fx["mask"], fx["status"], sh)
        if rc:
            raise kdv.KdvError(rc, "kdv_build_tree_mask")
        for lp in set_ptrs:
            rc = kdv.kdv_prefix_mla_attn(dims, *lp, ps, fx["pt"], L, T, split_ptr[0], split_ptr[1], fx["ws"],
                                         ws_bytes, sh)
            if rc:
                raise kdv.KdvError(rc, "kdv_prefix_mla_attn")
            rc = kdv.kdv_verify_mla_attn(dims, *lp, ps, fx["pt"] + 4 * L, 0, T, fx["mask"], split_ptr[2],
                                         split_ptr[3], fx["ws"], ws_bytes, sh)
            if rc:
                raise kdv.KdvError(rc, "kdv_verify_mla_attn")
            rc = kdv.kdv_merge_attn_states(split_ptr[0], split_ptr[1], split_ptr[2], split_ptr[3], T * H, Dv,
                                           fx["out"], fx["lse"], sh)
            if rc:
                raise kdv.KdvError(rc, "kdv_merge_attn_states")
    # the prefix-only pass always takes the split path; the tail pass (L = 0) may take the short-sequence kernel
    tail_names = KERNEL_NAMES if kdv.kdv_verify_kernel_count(dims, T, 0) == 3 else SHORT_KERNEL_NAMES
    per_split_step = dict(tree_mask=1, merge_states=lps)
    for n in KERNEL_NAMES + tail_names:
        per_split_step[n] = per_split_step.get(n, 0) + lps
    ms_split = None
    if L >= 1:
        log(f"[bench] timing {K} steps of the prefix/tail split (cold)")
        st["run_steps"](st["cold_ptrs"], 2, split_step)
        note("split warm-up", per_split_step, 2)
        ms_split = st["timed"](st["cold_ptrs"], K, split_step)
        st["note_timed"]("split cold", per_split_step, K)

    # The tree mask (once per verify step) and the greedy tree accept that follows verification: launch-bound,
    # timed as one HIP graph of many launches.
    def graph_us(launch, n=200, counts=None, label=None):
        """Device time per launch of a graph of n launches (`counts`: dispatches of one launch, for the
        ledger; uploading replay + timed replay)."""
        note(label or "launch-timing graph: " + ", ".join(counts or {}), counts or {}, 2 * n)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(n):
                launch()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, sh)
        g.replay()
        hip.record(e1, sh)
        return 1e3 * hip.elapsed_ms(e0, e1) / n

    def mask_launch():
        rc = kdv.kdv_build_tree_mask(fx["parent"], T, fx["mask"], fx["status"], sh)
        if rc:
            raise kdv.KdvError(rc, "kdv_build_tree_mask")
    kern_us["tree_mask"] = graph_us(mask_launch, counts=dict(tree_mask=1))
    _, acc_tok, acc_pred = si.accept_inputs(0, T, follow=0.8, parent=S.parent_np)
    acc_in = [torch.from_numpy(a.astype(np.int32)).to(dev) for a in (acc_tok, acc_pred)]
    acc_out = [torch.empty((n,), dtype=torch.int32, device=dev) for n in (T, 1, 1, 1)]

    def accept_launch():
        rc = kdv.kdv_tree_accept(fx["parent"], acc_in[0].data_ptr(), acc_in[1].data_ptr(), T,
                                 *[t.data_ptr() for t in acc_out], sh)
        if rc:
            raise kdv.KdvError(rc, "kdv_tree_accept")
    accept_us = graph_us(accept_launch, counts=dict(tree_accept=1))
    torch.cuda.synchronize()
    n_path = int(acc_out[1].item())
    # best-first draft tree at the session's block 16 / budget 32 (top-8 per position)
    b_logp, b_tok = si.draft_topk(0, 16, 8)
    b_in = [torch.from_numpy(b_logp).to(dev), torch.from_numpy(b_tok).to(dev),
            torch.tensor([7], dtype=torch.int32, device=dev)]
    b_out = [torch.empty((n,), dtype=torch.int32, device=dev) for n in (32, 32, 1)]

    def build_launch():
        rc = kdv.kdv_build_draft_tree(b_in[0].data_ptr(), b_in[1].data_ptr(), 16, 8, 32, b_in[2].data_ptr(),
                                      *[t.data_ptr() for t in b_out], sh)
        if rc:
            raise kdv.KdvError(rc, "kdv_build_draft_tree")
    build_us = graph_us(build_launch, counts=dict(draft_tree=1))
    torch.cuda.synchronize()

    def merge_launch():
        rc = kdv.kdv_merge_attn_states(split_ptr[0], split_ptr[1], split_ptr[2], split_ptr[3], T * H, Dv,
                                       fx["out"], fx["lse"], sh)
        if rc:
            raise kdv.KdvError(rc, "kdv_merge_attn_states")
    merge_us = graph_us(merge_launch, counts=dict(merge_states=1)) if L >= 1 else None
    torch.cuda.synchronize()

    batch_row = None
    if args.workload != "full61" and not args.no_extra:
        batch_row = batched_verify_row(torch, si, kdv, dev, sh, graph_us, note, st["names"])

    mfma_peak = measured_mfma_peak(torch, kdv, dev, hip, sh, note)
    # the dominant kernel: the split-KV pass (MFMA-bound), or for a one-tile sequence the single short-sequence
    # kernel, which is the whole call and streams the layer's weights (HBM-bound)
    if "splitkv" in kern_us:
        dom, bound, unit, peak = "splitkv", "mfma", "TFLOP/s", PEAK_BF16_TFLOPS
        dom_work = wk["flops_splitkv"]
        achieved = dom_work / (kern_us[dom] * 1e-6) / 1e12
    else:
        dom, bound, unit, peak = "short_verify", "hbm", "GB/s", PEAK_HBM_GBS
        dom_work = wk["bytes"]
        achieved = dom_work / (kern_us[dom] * 1e-6) / 1e9

    result = {
        "metric": METRIC,
        "value": res["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(res["us_per_layer"] * lps / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": S.desc, "heads": H, "tree_nodes": T, "prefix_len": L, "kv_lora_rank": R,
                   "qk_rope_dim": Dr, "qk_nope_dim": Dn, "v_head_dim": Dv, "layers_per_step": lps,
                   "kv_splits": res["kv_splits"], "timing": res["timing"], "buffers": res["buffers"]},
    }
    for k in ("us_per_layer", "frac_bf16_peak", "hbm_gbs", "frac_hbm_peak", "us_per_layer_eager_p10_p50_p90", "hot",
              "kernels_us", "kernels_us_p10_p90", "work_per_layer"):
        result[k] = res[k]
    result["kernels_us"]["tree_mask"] = round(kern_us["tree_mask"], 3)
    result.update({
        "kernel_timing": "eager, kernel-stamped HIP events, queued behind a spin kernel",
        "roofline": {"bound": bound, "kernel": dom, "achieved": round(achieved, 2),
                     "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
                     "traffic": traffic_from_profile(args.workload, dom),
                     **({"measured_mfma_peak": round(mfma_peak, 1),
                         "frac_of_measured_peak": round(achieved / mfma_peak, 4),
                         "work_per_launch_gflop": round(dom_work / 1e9, 4)} if bound == "mfma" else
                        {"work_per_launch_mbytes": round(dom_work / 1e6, 4)})},
        "cpu_baseline": None,
        "dispatch_phases": ledger,
        "next_rows": {"tree_accept": {"us": round(accept_us, 3), "nodes": T, "accepted_path_nodes": n_path,
                                      "timing": "one HIP graph of 200 launches", "bound": "launch latency"},
                      "draft_tree": {"us": round(build_us, 3), "block": 16, "topk": 8, "budget": 32,
                                     "nodes": int(b_out[2].item()), "timing": "one HIP graph of 200 launches",
                                     "bound": "latency of 31 dependent wave-wide selections"}},
    })
    if batch_row is not None:
        result["next_rows"]["batched_verify"] = batch_row
    if ms_split is not None:
        result["next_rows"]["prefix_tail_split"] = {
            "us_per_layer": round(1e3 * ms_split / (K * lps), 3),
            "single_call_us_per_layer": res["us_per_layer"],
            "merge_us": round(merge_us, 3),
            "parts": "prefix-only attention over L rows + tree attention over the T tail rows + LSE merge",
            "timing": "one HIP graph of K steps, cold rotation; merge alone: one HIP graph of 200 launches"}

    # The other configurations of the measured metric, each with its own inputs and the same measurement
    extra = {}
    if args.workload == "kimi5553" and not args.no_extra:
        del S, st
        torch.cuda.empty_cache()
        Ke, We = min(K, 20), min(Wm, 3)
        sweep = []
        for Lx in SWEEP_L:
            for Tx in SWEEP_T:
                Sx = setup_workload(f"kimi:{Lx}:{Tx}", torch, si, dev)
                r, _ = measure(Sx, args, torch, kdv, dev, hip, stream, sh, note, Ke, We, reps=5)
                r["bound"] = "hbm (weight streaming)" if Lx <= 1663 else "mfma"
                sweep.append(r)
                del Sx
                torch.cuda.empty_cache()
        extra["context_sweep"] = sweep
        for wname in ("long200k", "full61"):
            Sx = setup_workload(wname, torch, si, dev)
            r, _ = measure(Sx, args, torch, kdv, dev, hip, stream, sh, note, min(Ke, 10) if wname == "full61" else Ke,
                           min(We, 2), reps=3)
            extra[wname] = r
            del Sx
            torch.cuda.empty_cache()
        result["configs"] = extra

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, S_inp(args, si), wk, lps, extra)
    print(json.dumps(result), flush=True)


def S_inp(args, si):
    kind, Lk, Tk, seed = parse_workload(args.workload)
    if kind == "kimi5553":
        return si.kimi(L=5553, T=15, seed=0, dist="literal")
    if kind == "long200k":
        return si.long_fragmented(seed=0, dist="literal")
    if kind == "full61":
        return None
    return si.kimi(L=Lk, T=Tk, seed=seed, dist="literal")


def measured_mfma_peak(torch, kdv, dev, hip, sh, note, iters=2048):
    """bf16 MFMA issue-rate ceiling on this GPU, TFLOP/s: two 4-wave workgroups per CU, each wave four
    independent 32x32x16 chains (kdv_mfma_probe), timed with HIP events on the bench stream."""
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus
    sink = torch.empty((blocks * 256,), dtype=torch.float32, device=dev)
    for _ in range(2):  # the first launch is untimed
        e0, e1 = hip.event(), hip.event()
        hip.record(e0, sh)
        rc = kdv.kdv_mfma_probe(iters, sink.data_ptr(), blocks, sh)
        if rc:
            raise kdv.KdvError(rc, "kdv_mfma_probe")
        hip.record(e1, sh)
        torch.cuda.synchronize()
        ms = hip.elapsed_ms(e0, e1)
    note("mfma probe", {}, 0)
    return blocks * 4 * iters * 4 * 32768 / (ms * 1e-3) / 1e12


def batched_verify_row(torch, si, kdv, dev, sh, graph_us, note, single_names, C=10, L=5553, T=15):
    """Ten concurrent 15-node trees over 5553-token prefixes (the pages' C = 10 serving level, at the headline
    shape): one kdv_verify_mla_attn_batch call against the same requests as C single calls (hot buffers)."""
    log(f"[bench] batched verify: {C} requests")
    reqs = si.batch_inputs(si.KIMI_DIMS, [L] * C, [T] * C, seed=11)
    r0 = reqs[0]

    def b16(arrs):
        return torch.from_numpy(np.ascontiguousarray(np.concatenate(arrs)).view(np.int16)).to(dev)
    qn, qr = b16([r.q_nope for r in reqs]), b16([r.q_rope for r in reqs])
    wuk, wuv, ckv, kpe = b16([r0.w_uk]), b16([r0.w_uv]), b16([r0.c_kv]), b16([r0.k_pe])
    pt = torch.from_numpy(np.concatenate([r.page_table for r in reqs]).astype(np.int32)).to(dev)
    mask, status = kdv.build_tree_masks([torch.from_numpy(r.parent.astype(np.int32)).to(dev) for r in reqs])
    note("batch: tree masks", dict(tree_mask=C))
    dims = kdv.make_dims(**r0.dims())
    H, Dv = r0.H, r0.Dv
    out = torch.empty((C * T, H, Dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((C * T, H), dtype=torch.float32, device=dev)
    Ls, Ts = [L] * C, [T] * C
    ws_b = kdv.verify_batch_workspace_bytes(dims, Ls, Ts)
    ws = torch.zeros((ws_b,), dtype=torch.uint8, device=dev)
    la, lp = kdv._host_i32(Ls)
    ta, tp = kdv._host_i32(Ts)
    base = [t.data_ptr() for t in (wuk, wuv, ckv, kpe)]
    W = (T + 31) // 32

    def batch_launch():
        rc = kdv.kdv_verify_mla_attn_batch(dims, C, lp, tp, qn.data_ptr(), qr.data_ptr(), *base, ckv.shape[0],
                                           pt.data_ptr(), mask.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                           ws.data_ptr(), ws_b, sh)
        if rc:
            raise kdv.KdvError(rc, "kdv_verify_mla_attn_batch")

    ws1 = kdv.verify_workspace_bytes(dims, T, L)

    def singles_launch():
        for c in range(C):
            rc = kdv.kdv_verify_mla_attn(dims, qn.data_ptr() + c * T * H * r0.Dn * 2,
                                         qr.data_ptr() + c * T * H * r0.Dr * 2, *base, ckv.shape[0],
                                         pt.data_ptr() + 4 * c * (L + T), L, T, mask.data_ptr() + 4 * c * T * W,
                                         out.data_ptr() + c * T * H * Dv * 2, lse.data_ptr() + 4 * c * T * H,
                                         ws.data_ptr(), ws1, sh)
            if rc:
                raise kdv.KdvError(rc, "kdv_verify_mla_attn")
    call = dict(q_absorb=1, splitkv=1, combine_up=1)
    batch_us = graph_us(batch_launch, n=20, counts=call, label="batch: graph of batched calls")
    single_us = graph_us(singles_launch, n=20, counts={k: C for k in single_names},
                         label="batch: graph of single calls")
    torch.cuda.synchronize()
    assert int(status.sum().item()) == 0
    flops = sum(work(H, r0.Dn, r0.Dr, r0.R, Dv, L, T, r.parent)["flops"] for r in reqs)
    return {"requests": C, "prefix_len": L, "tree_nodes": T, "us_per_layer": round(batch_us, 3),
            "sequential_single_calls_us": round(single_us, 3), "speedup": round(single_us / batch_us, 3),
            "tflops": round(flops / (batch_us * 1e-6) / 1e12, 2),
            "frac_bf16_peak": round(flops / (batch_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "timing": "one HIP graph of 20 calls, hot buffers (shared pool of the ten requests: 64 MiB)"}


def _cpu_info():
    """Host CPU as the machine reports it: model name, family / model numbers, logical CPUs."""
    info = {"cpu_model": "unknown", "cpu_family": None, "cpu_model_number": None, "host_cpus": os.cpu_count()}
    try:
        for ln in open("/proc/cpuinfo"):
            k, _, v = ln.partition(":")
            k, v = k.strip(), v.strip()
            if k == "model name" and info["cpu_model"] == "unknown":
                info["cpu_model"] = v
            elif k == "cpu family" and info["cpu_family"] is None:
                info["cpu_family"] = int(v)
            elif k == "model" and info["cpu_model_number"] is None:
                info["cpu_model_number"] = int(v)
    except Exception:
        pass
    return info


def _blas():
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in pools] or [1])
        name = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in pools})) or "unknown"
        return threads, name
    except Exception:
        return os.cpu_count(), "unknown"


def _time_oracle(fn, seconds, max_calls=200):
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds or n >= max_calls:
            return el / n, n, el


def cpu_baseline(args, inp, wk, layers_per_step, extra):
    """The fp64 oracle, as it stands, on the host cores, over bounded samples of the measured workloads; the
    headline layer also on one thread; the heapq tree builder at the GPU builder's settings."""
    import oracle
    import synth_inputs as si
    threads, blas = _blas()
    if inp is None:  # full61: one layer of the same shape, generated on the host
        parent, table = si.full61_shared()
        inp = si.full61_layer(0, parent, table)
        heads = [0, 1]
        sample = f"oracle on heads {heads} of one 8-head layer (all 32 nodes, 131072-token prefix)"
    elif inp.L > 100000:
        heads = [0, 1]
        sample = f"oracle on heads {heads} of the layer (all nodes)"
    else:
        heads = None
        sample = "oracle on whole layers of the timed workload"
    frac = 1.0 if heads is None else len(heads) / inp.H
    log("[bench] cpu baseline (oracle)")
    sec, n, el = _time_oracle(lambda: oracle.verify_inputs(inp, heads=heads), args.cpu_seconds)
    s_per_layer = sec / frac
    wk1 = work(inp.H, inp.Dn, inp.Dr, inp.R, inp.Dv, inp.L, inp.T, inp.parent)
    res = {"value": round(wk1["flops"] / s_per_layer / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
           **_cpu_info(), "blas": blas,
           "kind": "oracle", "sample": f"{sample}; {n} calls in {el:.1f} s",
           "seconds_per_layer": round(s_per_layer, 4)}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            sec1, n1, el1 = _time_oracle(lambda: oracle.verify_inputs(inp, heads=heads), args.cpu_seconds / 2)
        res["single_thread"] = {"seconds_per_layer": round(sec1 / frac, 4),
                                "value": round(wk1["flops"] / (sec1 / frac) / 1e12, 6), "cores": 1,
                                "sample": f"{sample}; {n1} calls in {el1:.1f} s, BLAS limited to one thread"}
    except Exception as e:  # threadpoolctl missing: say so
        res["single_thread"] = {"error": repr(e)}
    # the other configurations: seconds per layer of the oracle on a small sample each
    if extra:
        per_cfg = {}
        for r in extra.get("context_sweep", []):
            L, T = r["prefix_len"], r["tree_nodes"]
            xi = si.kimi(L=L, T=T, seed=2 * SWEEP_L.index(L) + SWEEP_T.index(T), dist="literal")
            sx, nx, _ = _time_oracle(lambda: oracle.verify_inputs(xi, heads=[0, 1, 2, 3]), 1.0, 20)
            per_cfg[f"kimi:{L}:{T}"] = {"seconds_per_layer": round(sx * xi.H / 4, 4),
                                        "sample": f"heads 0-3 of the layer, {nx} calls"}
        if "long200k" in extra:
            xi = si.long_fragmented(seed=0, dist="literal")
            sx, nx, _ = _time_oracle(lambda: oracle.verify_inputs(xi, heads=[0]), 1.0, 5)
            per_cfg["long200k"] = {"seconds_per_layer": round(sx * xi.H, 3), "sample": f"head 0, {nx} calls"}
        if "full61" in extra:
            parent, table = si.full61_shared()
            xi = si.full61_layer(0, parent, table)
            sx, nx, _ = _time_oracle(lambda: oracle.verify_inputs(xi, heads=[0]), 1.0, 5)
            per_cfg["full61"] = {"seconds_per_layer": round(sx * xi.H, 3), "seconds_per_step": round(61 * sx * xi.H, 2),
                                 "sample": f"head 0 of layer 0, {nx} calls"}
        res["configs_seconds_per_layer"] = per_cfg
    # the best-first tree builder (heapq, pure Python) at the GPU builder's settings: block 16, top-8, budget 32
    b_logp, b_tok = si.draft_topk(0, 16, 8)
    sb, nb, _ = _time_oracle(lambda: oracle.build_draft_tree(b_logp, b_tok, 32, 7), 1.0, 20000)
    res["draft_tree"] = {"us_per_tree": round(sb * 1e6, 2), "us_per_batch_of_64": round(64 * sb * 1e6, 1),
                         "cores": 1, "sample": f"oracle.build_draft_tree (heapq, one thread), {nb} trees"}
    return res


# ------------------------------------------------------------------------------------------------ profiles
COPY_BYTES = 256 << 20
COPY_REPS = 3


def copy_calibration(torch, dev):
    """A plain device-to-device copy of known size: what FETCH_SIZE / WRITE_SIZE read for it gives the
    factor from counter units to bytes."""
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    for _ in range(COPY_REPS):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": COPY_REPS}), flush=True)


def source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_profile_path(workload, kernel):
    return os.path.join(ROOT, "profiles", f"{kernel}_{profile_tag(workload)}_hbm_traffic.md")


def traffic_from_profile(workload, kernel):
    """HBM bytes per launch of the dominant kernel from the committed counter summary, or None when there is none
    or the kernel source has changed since the counters were taken."""
    path = traffic_profile_path(workload, kernel)
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(path).read(), re.S)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256") != source_hash():
        return None
    return rec["traffic_bytes_per_launch"]


def _kernel_key(name):
    for k in KERNELS:
        if k in name:
            return k
    return None


def _read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _phases(bench, kernel):
    """Dispatch index ranges of one kernel in each phase of a bench.py run (its dispatch ledger), in order."""
    out, a = {}, 0
    for name, counts in bench["dispatch_phases"]:
        c = counts.get(kernel, 0)
        out[name] = (a, a + c)
        a += c
    return out, a


def _counter_per_dispatch(d, counter, kernel_pred):
    rows = [r for r in _read_csv(os.path.join(d, "run_counter_collection.csv")) if r["Counter_Name"] == counter]
    by = {}
    for r in rows:
        k = kernel_pred(r["Kernel_Name"])
        if k:
            by.setdefault(k, []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return {k: [v for _, v in sorted(lst)] for k, lst in by.items()}


def summarize_profile(d, workload):
    """Writes <kernel>_<workload>_kernel_trace.md and splitkv_<workload>_hbm_traffic.md into d/summaries."""
    cmds = open(os.path.join(d, "commands.txt")).read().strip()
    out_dir = os.path.join(d, "summaries")
    os.makedirs(out_dir, exist_ok=True)

    # kernel trace: per-kernel durations by bench phase, next to bench.py's own event timings
    bench = json.loads(open(os.path.join(d, "trace_bench.json")).read().strip().splitlines()[-1])
    plain = json.loads(open(os.path.join(d, "plain_bench.json")).read().strip().splitlines()[-1])
    trace = _read_csv(os.path.join(d, "trace", "run_kernel_trace.csv"))
    durs = {}
    for r in trace:
        k = _kernel_key(r["Kernel_Name"])
        if k:
            durs.setdefault(k, []).append((int(r["Dispatch_Id"]), int(r["Start_Timestamp"]),
                                           int(r["End_Timestamp"])))
    lines = [f"# Kernel trace: tree-verify MLA attention, workload `{workload}`", "",
             f"Kernel source sha256 (first 16 hex): `{source_hash()}`", "",
             "Commands (from the repository root on the GPU machine; `bash profile_bench.sh` runs them):", "",
             "```", cmds, "```", "",
             f"bench.py without the tracer: {plain['us_per_layer']} us/layer cold, "
             f"{plain['hot']['us_per_layer']} us/layer hot, {plain['value']} {plain['unit']}; under the tracer: "
             f"{bench['us_per_layer']} us/layer cold.", "",
             "Average kernel duration (us) from rocprofv3 `--kernel-trace`, by phase of the bench run (phases "
             "from the run's dispatch ledger; the 'batch' phases run the ten-request workload, the 'split' phases "
             "the prefix/tail split, so their durations are of other shapes):", "",
             "| kernel | phase | dispatches | average us |", "|---|---|---|---|"]
    ev = {f"{k}_kernel": v for k, v in plain["kernels_us"].items()}
    eager = {}
    for k in KERNELS:
        if k not in durs:
            continue
        lst = sorted(durs[k])
        ph, total = _phases(bench, k)
        if len(lst) != total:
            raise SystemExit(f"{k}: {len(lst)} dispatches traced, {total} expected")
        for name, (a, b) in ph.items():
            seg = lst[a:b]
            if seg:
                avg = sum(e - s for _, s, e in seg) / len(seg) / 1e3
                lines.append(f"| {k} | {name} | {len(seg)} | {avg:.2f} |")
                if name == f"{workload}: eager cold, kernel events":
                    eager[k] = avg
    lines += ["", "Eager cold launches under the tracer against bench.py's kernel-stamped HIP events without it:", "",
              "| kernel | traced average us | bench.py events us |", "|---|---|---|"]
    for k, v in eager.items():
        lines.append(f"| {k} | {v:.2f} | {ev.get(k, float('nan')):.2f} |")
    # step span in the timed cold replay (includes gaps between kernels): the call's first kernel starts every layer
    qa_a, qa_b = _phases(bench, "q_absorb_kernel")[0].get(f"{workload}: graph cold, timed replay", (0, 0))
    first = "q_absorb_kernel" if qa_b > qa_a else "short_verify_kernel"
    tm = sorted(durs[first])
    ph, _ = _phases(bench, first)
    a, b = ph[f"{workload}: graph cold, timed replay"]
    lps = bench["config"]["layers_per_step"]
    span = lps * (tm[b - 1][1] - tm[a][1]) / (b - a - 1) / 1e3 if b - a > 1 else float("nan")
    lines += ["", f"Cold timed replay: one step every {span:.2f} us under the tracer "
              f"(bench.py without the tracer: {1e3 * plain['ms_per_step']:.2f} us per step).", "",
              "In the timed steps the tree mask is built by an extra block of the first layer's q_absorb launch "
              "(kdv_verify_mla_attn_tree); the eager per-kernel launches and the split phases use the separate "
              "mask kernel.  bench.py's kernel-stamped HIP events are taken over its eager cold launches without "
              "the tracer (the tracer lengthens event-bracketed launches).", ""]
    with open(os.path.join(out_dir, f"verify_{profile_tag(workload)}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM traffic of the split-KV kernel: FETCH_SIZE and WRITE_SIZE, scaled by the copy calibration
    def kp(name):
        return _kernel_key(name)

    def copy_pred(name):
        return "copy" if "copyBuffer" in name else None
    fb = json.loads(open(os.path.join(d, "fetch_bench.json")).read().strip().splitlines()[-1])
    fetch = _counter_per_dispatch(os.path.join(d, "fetch"), "FETCH_SIZE", kp)
    write = _counter_per_dispatch(os.path.join(d, "write"), "WRITE_SIZE", kp)
    cf = _counter_per_dispatch(os.path.join(d, "copy_fetch"), "FETCH_SIZE", copy_pred)["copy"]
    cw = _counter_per_dispatch(os.path.join(d, "copy_write"), "WRITE_SIZE", copy_pred)["copy"]
    copy_kib = COPY_BYTES / 1024
    f_fac = copy_kib / (sum(cf) / len(cf))
    w_fac = copy_kib / (sum(cw) / len(cw))
    lines = [f"# HBM traffic per dispatch: tree-verify MLA attention, workload `{workload}`", "",
             "Commands (from the repository root on the GPU machine; `bash profile_bench.sh` runs them):", "",
             "```", cmds, "```", "",
             f"Calibration: a plain {COPY_BYTES >> 20} MiB device copy (`bench.py --copy-calibration`) reads "
             f"FETCH_SIZE {sum(cf) / len(cf):.0f} KiB and WRITE_SIZE {sum(cw) / len(cw):.0f} KiB per dispatch "
             f"for {copy_kib:.0f} KiB moved each way: bytes = FETCH_SIZE x {f_fac:.3f} KiB, "
             f"WRITE_SIZE x {w_fac:.3f} KiB.", "",
             "Per dispatch, averaged over the eager cold launches of the counted run "
             f"(`--steps {fb['steps']} --warmup {fb['warmup']}`):", "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB |", "|---|---|---|---|---|"]
    rec = None
    # the workload's own dominant kernel: split-KV, or the short-sequence kernel when the call has no split-KV pass
    sk_ph, _ = _phases(fb, "splitkv_kernel")
    sk_a, sk_b = sk_ph.get(f"{workload}: eager cold, kernel events", (0, 0))
    dom_kernel = "splitkv_kernel" if sk_b > sk_a else "short_verify_kernel"
    for k in KERNELS:
        if k not in fetch or k not in write:
            continue
        ph, total = _phases(fb, k)
        a, b = ph[f"{workload}: eager cold, kernel events"]
        fv, wv = fetch[k][a:b], write[k][a:b]
        if len(fetch[k]) != total or len(write[k]) != total:
            raise SystemExit(f"{k}: counter dispatch count mismatch")
        if not fv:  # a kernel of the other measurements only (not launched by the verify call)
            continue
        fk, wk_ = sum(fv) / len(fv), sum(wv) / len(wv)
        fb_bytes, wb_bytes = fk * f_fac * 1024, wk_ * w_fac * 1024
        lines.append(f"| {k} | {fk:.1f} | {wk_:.1f} | {fb_bytes / 1e6:.3f} | {wb_bytes / 1e6:.3f} |")
        if k == dom_kernel:
            rec = {"kernel": k, "workload": workload, "source_sha256": source_hash(),
                   "fetch_kib_per_dispatch": round(fk, 2), "write_kib_per_dispatch": round(wk_, 2),
                   "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4),
                   "traffic_bytes_per_launch": round(fb_bytes + wb_bytes)}
    lines += ["", "Record read by bench.py (`roofline.traffic`, used only while the kernel source hash matches):",
              "", "```json", json.dumps(rec), "```", ""]
    with open(os.path.join(out_dir, f"{dom_kernel[:-len('_kernel')]}_{profile_tag(workload)}_hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if os.path.isdir(os.path.join(d, "mfma")):
        _summarize_mfma(d, workload, cmds, bench, durs, out_dir)
    print(out_dir)


def _summarize_mfma(d, workload, cmds, trace_bench, durs, out_dir):
    """MFMA instructions and busy cycles per dispatch (counter run) against the traced durations."""
    mb = json.loads(open(os.path.join(d, "mfma_bench.json")).read().strip().splitlines()[-1])
    insts = _counter_per_dispatch(os.path.join(d, "mfma"), "SQ_INSTS_MFMA", _kernel_key)
    busy = _counter_per_dispatch(os.path.join(d, "mfma"), "SQ_VALU_MFMA_BUSY_CYCLES", _kernel_key)
    agent = [r for r in _read_csv(os.path.join(d, "mfma", "run_agent_info.csv")) if r.get("Name", "").startswith("gfx")]
    simds = int(agent[0]["Simd_Count"]) if agent else 1024
    mhz = float(agent[0]["Max_Engine_Clk_Fcompute"]) if agent else 2400.0
    lines = [f"# MFMA use per dispatch: tree-verify MLA attention, workload `{workload}`", "",
             "Commands (from the repository root on the GPU machine; `bash profile_bench.sh` runs them):", "",
             "```", cmds, "```", "",
             f"Counters from `rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES` over the eager cold launches "
             f"of the counted run (`--steps {mb['steps']} --warmup {mb['warmup']}`); durations from the kernel "
             f"trace of the same phase.  Every MFMA here is a 32x32x16 bf16 (32768 flop, 32 busy cycles).  "
             f"Busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / ({simds} SIMDs x duration x {mhz:.0f} MHz, the "
             "agent's maximum engine clock): the share of the kernel's time the matrix cores were busy, "
             "against the clock the vendor peak assumes.", "",
             "| kernel | MFMA instructions | MFMA GFLOP | traced us | TFLOP/s from counters | MFMA busy fraction |",
             "|---|---|---|---|---|---|"]
    for k in KERNELS:
        if k not in insts or k not in busy or k not in durs:
            continue
        ph, total = _phases(mb, k)
        a, b = ph[f"{workload}: eager cold, kernel events"]
        iv, bv = insts[k][a:b], busy[k][a:b]
        if len(insts[k]) != total or not iv:
            continue
        tph, _ = _phases(trace_bench, k)
        ta, tb = tph[f"{workload}: eager cold, kernel events"]
        seg = sorted(durs[k])[ta:tb]
        us = sum(e - s_ for _, s_, e in seg) / len(seg) / 1e3
        n = sum(iv) / len(iv)
        cyc = sum(bv) / len(bv)
        gflop = n * 32768 / 1e9
        frac = cyc / (simds * us * 1e-6 * mhz * 1e6)
        lines.append(f"| {k} | {n:.0f} | {gflop:.3f} | {us:.2f} | {gflop / (us * 1e-6) / 1e3:.1f} | {frac:.3f} |")
    with open(os.path.join(out_dir, f"verify_{profile_tag(workload)}_mfma.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
