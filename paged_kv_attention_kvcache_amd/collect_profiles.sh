#!/bin/bash
# Collects, on an MI355X, the rocprofv3 runs behind profiles/ and writes their
# summaries there. Run from the repository root with the library built:
#   bash paged_kv_attention_kvcache_amd/collect_profiles.sh OUT [STEP ...]
# OUT receives the raw rocprofv3 output (large; not committed). Every run is
# one of the commands named in the summaries' headers. With STEP names only
# those runs are made (the raw output of several invocations can be gathered
# into one OUT); the last step, "summaries", needs every run in OUT and
# needs no GPU.
set -o pipefail
OUT=${1:?usage: collect_profiles.sh OUT [STEP ...]}
shift
ONLY=" $* "
R=$(pwd)
mkdir -p "$OUT"
export TMPDIR=${TMPDIR:-/tmp}
want() { [ "$ONLY" = "  " ] || [[ "$ONLY" == *" $1 "* ]]; }
step() {
  local name=$1
  shift
  want "$name" || return 0
  echo "== $name $(date +%T)"
  "$@" > "$OUT/$name.log" 2>&1 || { echo "$name failed"; tail -20 "$OUT/$name.log"; exit 1; }
}
pmc() {
  local name=$1 counters=$2
  shift 2
  step "$name" timeout -s KILL 400 rocprofv3 --pmc $counters --output-format csv \
    -d "$OUT/$name" -o run -- "$@"
}
# Kernel durations: the default benchmark, exactly as the driver runs it.
step stats_default timeout -k 10 900 rocprofv3 --kernel-trace --stats --output-format csv \
  -d "$OUT/stats_default" -o run -- python3 "$R/bench.py"
# HBM bytes: a plain copy of 1 GiB calibrates the counters, then one step of
# every workload (bytes per launch do not depend on the number of steps).
pmc copy_fetch FETCH_SIZE python3 "$R/bench.py" --probe copy
pmc copy_write WRITE_SIZE python3 "$R/bench.py" --probe copy
pmc all_fetch FETCH_SIZE python3 "$R/bench.py" --steps 1 --warmup 1 --no-cpu-baseline
pmc all_write WRITE_SIZE python3 "$R/bench.py" --steps 1 --warmup 1 --no-cpu-baseline
# Matrix-core and instruction counters of the prefill kernels, L2 hit rates.
pmc prefill_engine "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_WAIT_INST_ANY SQ_WAVE_CYCLES SQ_BUSY_CYCLES" \
  python3 "$R/bench.py" --prefill-only --no-cpu-baseline
# What the prefill step waits on: engine clock, matrix-core and LDS activity, waits.
pmc prefill_pipeline "SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_WAIT_ANY SQ_WAVE_CYCLES" \
  python3 "$R/bench.py" --prefill-only --no-cpu-baseline
pmc all_l2 "TCC_HIT_sum TCC_MISS_sum" python3 "$R/bench.py" --steps 1 --warmup 1 --no-cpu-baseline
# What bounds the decode kernels: L1->L2 and L2->memory read latency, TLB
# misses, instruction counts and waits (decode workloads only).
pmc decode_tcp "TCP_TCC_READ_REQ_LATENCY_sum TCP_TCC_READ_REQ_sum TCP_UTCL1_TRANSLATION_MISS_sum TCP_UTCL1_REQUEST_sum" \
  python3 "$R/bench.py" --steps 1 --warmup 1 --no-cpu-baseline --no-prefill
pmc decode_tcc "TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_LEVEL_sum" \
  python3 "$R/bench.py" --steps 1 --warmup 1 --no-cpu-baseline --no-prefill
pmc decode_sq "SQ_INSTS_VALU SQ_INSTS_VMEM_RD SQ_INST_LEVEL_VMEM SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_BUSY_CYCLES SQ_WAVES" \
  python3 "$R/bench.py" --steps 1 --warmup 1 --no-cpu-baseline --no-prefill
want summaries || exit 0
echo "== summaries $(date +%T)"
python3 -m paged_kv_attention_kvcache_amd.rocprof_summary write "$OUT" --profiles "$R/profiles"
