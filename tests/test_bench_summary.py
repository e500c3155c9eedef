"""CPU tests of bench.py's host logic: the profile summaries split a trace by the dispatch ledger that the
bench run records, and the HBM-traffic record is what roofline.traffic reads back.  A synthetic profile
directory (the CSV columns rocprofv3 writes) stands in for a GPU run; no GPU is touched."""
import csv
import json
import os

import pytest

import bench

PHASES = [["kimi5553: warm-up", {"q_absorb_kernel": 2, "splitkv_kernel": 2, "combine_up_kernel": 2}],
          ["kimi5553: graph cold, upload replay", {"q_absorb_kernel": 3, "splitkv_kernel": 3, "combine_up_kernel": 3}],
          ["kimi5553: graph cold, timed replay", {"q_absorb_kernel": 3, "splitkv_kernel": 3, "combine_up_kernel": 3}],
          ["kimi5553: eager cold, kernel events", {"tree_mask_kernel": 2, "q_absorb_kernel": 2, "splitkv_kernel": 2,
                                                   "combine_up_kernel": 2}],
          ["launch-timing graph: tree_mask", {"tree_mask_kernel": 4}]]
NAMES = {"tree_mask_kernel": "kdv::tree_mask_kernel(int const*, int, unsigned int*, int*)",
         "q_absorb_kernel": "void kdv::q_absorb_kernel<128, 512, 64>(...)",
         "splitkv_kernel": "void kdv::splitkv_kernel<512, 64, 1>(...)",
         "combine_up_kernel": "void kdv::combine_up_kernel<512, 128, 1>(...)"}
# per-kernel duration (ns) by phase: the eager phase is what the counter tables average over
DUR = {"tree_mask_kernel": 2000, "q_absorb_kernel": 5000, "splitkv_kernel": 24000, "combine_up_kernel": 8000}


def _bench_json(steps=3, warmup=2):
    return {"metric": "m", "value": 300.0, "unit": "TFLOP/s", "us_per_layer": 38.0, "hot": {"us_per_layer": 36.0},
            "ms_per_step": 0.038, "steps": steps, "warmup": warmup, "kernel_calls": 2,
            "config": {"layers_per_step": 1}, "dispatch_phases": PHASES,
            "kernels_us": {"tree_mask": 1.6, "q_absorb": 5.6, "splitkv": 24.4, "combine_up": 8.2}}


def _dispatches():
    """Launch order of the synthetic run: phases in order, kernels interleaved per step."""
    out = []
    for _, counts in PHASES:
        left = dict(counts)
        while any(left.values()):
            for k in ("tree_mask_kernel", "q_absorb_kernel", "splitkv_kernel", "combine_up_kernel"):
                if left.get(k, 0):
                    out.append(k)
                    left[k] -= 1
    return out


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _counter_dir(path, counter, per_kernel):
    rows = []
    for i, k in enumerate(_dispatches()):
        rows.append({"Dispatch_Id": i + 1, "Kernel_Name": NAMES[k], "Counter_Name": counter,
                     "Counter_Value": per_kernel[k]})
    _write_csv(os.path.join(path, "run_counter_collection.csv"), rows)


@pytest.fixture
def profile_dir(tmp_path):
    d = tmp_path / "profile_kimi5553"
    d.mkdir()
    (d / "commands.txt").write_text("cd /tmp && TMPDIR=/tmp python3 $REPO/bench.py --workload kimi5553\n")
    for name in ("plain_bench.json", "trace_bench.json", "fetch_bench.json", "write_bench.json", "mfma_bench.json"):
        (d / name).write_text(json.dumps(_bench_json()) + "\n")
    t, rows = 1000, []
    for i, k in enumerate(_dispatches()):
        rows.append({"Dispatch_Id": i + 1, "Kernel_Name": NAMES[k], "Start_Timestamp": t,
                     "End_Timestamp": t + DUR[k]})
        t += DUR[k] + 500
    _write_csv(str(d / "trace" / "run_kernel_trace.csv"), rows)
    _counter_dir(str(d / "fetch"), "FETCH_SIZE", {"tree_mask_kernel": 2, "q_absorb_kernel": 4000,
                                                  "splitkv_kernel": 7500, "combine_up_kernel": 12000})
    _counter_dir(str(d / "write"), "WRITE_SIZE", {"tree_mask_kernel": 0, "q_absorb_kernel": 1000,
                                                  "splitkv_kernel": 14500, "combine_up_kernel": 270})
    _counter_dir(str(d / "mfma"), "SQ_INSTS_MFMA", {"tree_mask_kernel": 0, "q_absorb_kernel": 8192,
                                                    "splitkv_kernel": 354960, "combine_up_kernel": 32768})
    # the mfma directory holds both counters
    rows = list(csv.DictReader(open(d / "mfma" / "run_counter_collection.csv")))
    for r in list(rows):
        rows.append(dict(r, Counter_Name="SQ_VALU_MFMA_BUSY_CYCLES", Counter_Value=32 * int(r["Counter_Value"])))
    _write_csv(str(d / "mfma" / "run_counter_collection.csv"), rows)
    _write_csv(str(d / "mfma" / "run_agent_info.csv"), [{"Name": "gfx950", "Simd_Count": 1024,
                                                         "Max_Engine_Clk_Fcompute": 2400}])
    copy_kib = bench.COPY_BYTES // 1024
    for sub, counter, val in (("copy_fetch", "FETCH_SIZE", copy_kib // 2), ("copy_write", "WRITE_SIZE", copy_kib)):
        _write_csv(str(d / sub / "run_counter_collection.csv"),
                   [{"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                     "Counter_Value": val}])
    return str(d)


def test_phases_follow_the_ledger():
    ph, total = bench._phases(_bench_json(), "splitkv_kernel")
    assert total == 10
    assert ph["kimi5553: graph cold, timed replay"] == (5, 8)
    assert ph["kimi5553: eager cold, kernel events"] == (8, 10)
    assert ph["launch-timing graph: tree_mask"] == (10, 10)
    ph, total = bench._phases(_bench_json(), "tree_mask_kernel")
    assert total == 6 and ph["kimi5553: eager cold, kernel events"] == (0, 2)


def test_summaries_from_a_synthetic_profile(profile_dir):
    bench.summarize_profile(profile_dir, "kimi5553")
    out = os.path.join(profile_dir, "summaries")
    assert sorted(os.listdir(out)) == ["splitkv_kimi5553_hbm_traffic.md", "verify_kimi5553_kernel_trace.md",
                                      "verify_kimi5553_mfma.md"]
    trace = open(os.path.join(out, "verify_kimi5553_kernel_trace.md")).read()
    assert "| splitkv_kernel | kimi5553: graph cold, timed replay | 3 | 24.00 |" in trace
    assert "| splitkv_kernel | 24.00 | 24.40 |" in trace  # traced eager average beside bench.py's events
    traffic = open(os.path.join(out, "splitkv_kimi5553_hbm_traffic.md")).read()
    rec = json.loads(traffic.split("```json\n")[1].split("\n```")[0])
    # calibration: FETCH_SIZE reads half the copied bytes (factor 2), WRITE_SIZE all of them (factor 1)
    assert rec["fetch_factor"] == pytest.approx(2.0, rel=1e-4) and rec["write_factor"] == pytest.approx(1.0)
    assert rec["traffic_bytes_per_launch"] == pytest.approx((7500 * 2 + 14500) * 1024, rel=1e-4)
    assert rec["source_sha256"] == bench.source_hash()
    mfma = open(os.path.join(out, "verify_kimi5553_mfma.md")).read()
    # 354960 MFMAs x 32768 flop over 24 us; busy = 32 cycles each over 1024 SIMDs x 24 us x 2.4 GHz
    busy = 354960 * 32 / (1024 * 24e-6 * 2400e6)
    assert f"| splitkv_kernel | 354960 | 11.631 | 24.00 | 484.6 | {busy:.3f} |" in mfma


def test_workload_names():
    assert bench.parse_workload("kimi5553")[0] == "kimi5553"
    assert bench.parse_workload("kimi:13:9") == ("kimi", 13, 9, 0)
    assert bench.parse_workload("kimi:16384:15") == ("kimi", 16384, 15, 9)
    assert bench.profile_tag("kimi:16384:15") == "kimi_L16384_T15"
    with pytest.raises(SystemExit):
        bench.parse_workload("sweep:1")


def test_committed_profiles_match_the_kernel_source():
    """The kernel-trace and HBM-traffic summaries under profiles/ were taken from the kernel source as it stands:
    each names the source hash it was measured on, and roofline.traffic is only read back while that hash
    matches.  A kernel change makes this fail until the profiles are taken again (profile_bench.sh on the GPU)."""
    pdir = os.path.join(bench.ROOT, "profiles")
    names = sorted(f for f in os.listdir(pdir) if f.endswith("_kernel_trace.md") or f.endswith("_hbm_traffic.md"))
    assert len(names) >= 2, "no profile summaries"
    want = bench.source_hash()
    for name in names:
        text = open(os.path.join(pdir, name)).read()
        if name.endswith("_kernel_trace.md"):
            assert f"Kernel source sha256 (first 16 hex): `{want}`" in text, name
        else:
            rec = json.loads(text.split("```json\n", 1)[1].split("\n```", 1)[0])
            assert rec["source_sha256"] == want, name
    assert bench.traffic_from_profile("kimi5553", "splitkv") is not None
