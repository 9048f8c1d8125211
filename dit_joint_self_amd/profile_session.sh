#!/bin/bash
# Measurement session behind profiles/: the bench line as the full test run
# takes it, then rocprofv3 kernel traces and HBM / SQ counters of each kernel
# family, each from the bench command of its workload.  Outputs go to
# gpurun_out/ (raw) on the GPU machine.  Usage (repo root): bash dit_joint_self_amd/profile_session.sh
set -o pipefail
export TMPDIR=/tmp
O=gpurun_out/session
mkdir -p $O
step() { echo "[step] $1"; }
run() {  # run <name> <limit s> <cmd...>: one GPU step, its own time limit, stop the session on failure
    local name=$1 lim=$2; shift 2
    step "$name"
    timeout -k 10 "$lim" "$@" > "$O/$name.log" 2>&1 || { echo "FAILED: $name"; tail -20 "$O/$name.log"; exit 1; }
}
pmc() {  # pmc <name> <counters> -- <cmd...>
    local name=$1 ctr=$2; shift 3
    step "pmc $name"
    timeout -s KILL 180 rocprofv3 --pmc $ctr --output-format csv -d "$O/$name" -o run -- "$@" > "$O/$name.log" 2>&1 \
        || { echo "FAILED: pmc $name"; tail -20 "$O/$name.log"; exit 1; }
}
B="python -u bench.py --no-cpu-baseline --no-library-baseline --single-config"
P="--steps 2 --warmup 1 --prewarm-s 0"
run bench_line 600 python -u bench.py --gpus 1 --steps 20 --warmup 5
run trace_flux2048 300 rocprofv3 --kernel-trace --stats --output-format csv -d $O/trace_flux2048 -o run -- $B --workload flux2048 --steps 20 --warmup 5
pmc fetch_flux2048 FETCH_SIZE -- $B --workload flux2048 $P
pmc write_flux2048 WRITE_SIZE -- $B --workload flux2048 $P
pmc sq_flux2048 "SQ_BUSY_CYCLES SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE" -- $B --workload flux2048 $P
pmc fetch_copy FETCH_SIZE -- python -u bench.py --copy-mib 1024 --steps 2 --warmup 1
pmc write_copy WRITE_SIZE -- python -u bench.py --copy-mib 1024 --steps 2 --warmup 1
run bench_fp8 300 $B --workload flux2048_fp8 --steps 20 --warmup 5
run trace_fp8 300 rocprofv3 --kernel-trace --stats --output-format csv -d $O/trace_fp8 -o run -- $B --workload flux2048_fp8 --steps 20 --warmup 5
pmc fetch_fp8 FETCH_SIZE -- $B --workload flux2048_fp8 $P
pmc write_fp8 WRITE_SIZE -- $B --workload flux2048_fp8 $P
pmc sq_fp8 "SQ_BUSY_CYCLES SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE" -- $B --workload flux2048_fp8 $P
run bench_ring2 300 python -u bench.py --workload flux2048 --ring 2 --steps 20 --warmup 5
run trace_ring2 300 rocprofv3 --kernel-trace --stats --output-format csv -d $O/trace_ring2 -o run -- python -u bench.py --workload flux2048 --ring 2 --steps 20 --warmup 5
run bench_qkv 300 python -u bench.py --workload flux2048_qkv --steps 20 --warmup 5 --cpu-seconds 10
run trace_qkv 300 rocprofv3 --kernel-trace --stats --output-format csv -d $O/trace_qkv -o run -- $B --workload flux2048_qkv --steps 20 --warmup 5
pmc fetch_qkv FETCH_SIZE -- $B --workload flux2048_qkv $P
pmc write_qkv WRITE_SIZE -- $B --workload flux2048_qkv $P
pmc sq_qkv "SQ_BUSY_CYCLES SQ_WAIT_INST_LDS SQ_WAIT_ANY SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE" -- $B --workload flux2048_qkv $P
run bench_residual 300 python -u bench.py --workload flux2048_residual --steps 20 --warmup 5 --cpu-seconds 10
run trace_residual 300 rocprofv3 --kernel-trace --stats --output-format csv -d $O/trace_residual -o run -- $B --workload flux2048_residual --steps 20 --warmup 5
pmc fetch_residual FETCH_SIZE -- $B --workload flux2048_residual $P
pmc write_residual WRITE_SIZE -- $B --workload flux2048_residual $P
step done
