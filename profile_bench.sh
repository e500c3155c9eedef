#!/bin/bash
# rocprofv3 evidence behind bench.py's roofline object, for one workload (default kimi5553):
#   1. a bench run without the profiler, then the same run under a kernel trace (per-kernel durations,
#      compared with bench.py's own event timings from the run without the profiler);
#   2. FETCH_SIZE, then WRITE_SIZE, then the MFMA instruction and busy-cycle counts, each in a counter run of
#      its own, on a shorter bench run;
#   3. the same two counters on a plain 256 MiB device copy, the calibration of counter units to bytes.
# Raw output goes to $O (profile_<workload>/ under the output folder); the markdown summaries to $O/summaries/.
# Run from anywhere on the GPU machine: bash profile_bench.sh [workload]
R=$(cd "$(dirname "$0")" && pwd)
W=${1:-kimi5553}
O=$R/gpurun_out/profile_${W//:/_}
mkdir -p "$O"
: > "$O/commands.txt"
cd /tmp && export TMPDIR=/tmp

run() {  # run <seconds> <stdout file> <command...>: log the command, stop the script on any failure
  local secs=$1 outf=$2
  shift 2
  echo "cd /tmp && TMPDIR=/tmp $*" | sed "s#$R#\$REPO#g" >> "$O/commands.txt"
  echo "[profile] $*" >&2
  timeout -k 10 "$secs" "$@" > "$outf" 2> "$outf.err"
  local rc=$?
  if [ $rc -ne 0 ]; then
    echo "[profile] failed with status $rc: $*" >&2
    tail -20 "$outf.err" >&2
    exit $rc
  fi
}

run 300 "$O/plain_bench.json" python3 "$R/bench.py" --workload "$W" --steps 50 --warmup 5 --no-cpu-baseline --no-extra
run 300 "$O/trace_bench.json" rocprofv3 --kernel-trace --stats -f csv -d "$O/trace" -o run -- \
  python3 "$R/bench.py" --workload "$W" --steps 50 --warmup 5 --no-cpu-baseline --no-extra
run 120 "$O/fetch_bench.json" rocprofv3 --pmc FETCH_SIZE -f csv -d "$O/fetch" -o run -- \
  python3 "$R/bench.py" --workload "$W" --steps 10 --warmup 2 --no-cpu-baseline --no-extra
run 120 "$O/write_bench.json" rocprofv3 --pmc WRITE_SIZE -f csv -d "$O/write" -o run -- \
  python3 "$R/bench.py" --workload "$W" --steps 10 --warmup 2 --no-cpu-baseline --no-extra
run 120 "$O/mfma_bench.json" rocprofv3 --pmc SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES -f csv -d "$O/mfma" -o run -- \
  python3 "$R/bench.py" --workload "$W" --steps 10 --warmup 2 --no-cpu-baseline --no-extra
run 120 "$O/copy_fetch.json" rocprofv3 --pmc FETCH_SIZE -f csv -d "$O/copy_fetch" -o run -- \
  python3 "$R/bench.py" --copy-calibration
run 120 "$O/copy_write.json" rocprofv3 --pmc WRITE_SIZE -f csv -d "$O/copy_write" -o run -- \
  python3 "$R/bench.py" --copy-calibration
echo "python3 \$REPO/bench.py --workload $W --summarize-profile gpurun_out/profile_${W//:/_}" >> "$O/commands.txt"
python3 "$R/bench.py" --workload "$W" --summarize-profile "$O"
