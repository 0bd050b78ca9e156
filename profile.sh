#!/bin/bash
# rocprofv3 runs behind the committed summaries under profiles/: a kernel trace of
# the benchmark, then one counter pass each for FETCH_SIZE and WRITE_SIZE (with the
# 512 MiB calibration copy of bench.py --profile), three passes of SQ counters
# (matrix-core and VALU activity, LDS traffic and conflicts, at most 8 SQ counters a
# pass), then the summaries.
# Usage, from the repository root on a machine with the GPU:  bash profile.sh OUTDIR [bench args]
set -u
OUT=$(realpath -m "${1:?usage: profile.sh OUTDIR [bench args]}")
shift
R=$(cd "$(dirname "$0")" && pwd)
mkdir -p "$OUT"
cd /tmp && export TMPDIR=/tmp
T="rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/trace -o run -- python3 $R/bench.py --steps 50 --warmup 5 --cpu-rows 0 $*"
F="rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/fetch -o pmc -- python3 $R/bench.py --profile --steps 3 --warmup 1 $*"
W="rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/write -o pmc -- python3 $R/bench.py --profile --steps 3 --warmup 1 $*"
SQ1="SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_BUSY_CU_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS"
SQ2="SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_WAIT_INST_LDS SQ_LDS_BANK_CONFLICT SQ_LDS_DATA_FIFO_FULL SQ_LDS_CMD_FIFO_FULL SQ_WAIT_INST_ANY"
SQ3="SQ_INSTS_VALU_TRANS_F32 SQ_THREAD_CYCLES_VALU SQ_ACTIVE_INST_ANY SQ_INST_LEVEL_LDS SQ_LDS_ADDR_CONFLICT SQ_CYCLES SQ_ACTIVE_INST_MISC SQ_ACTIVE_INST_SCA"
S1="rocprofv3 --pmc $SQ1 --output-format csv -d $OUT/sq1 -o pmc -- python3 $R/bench.py --profile --steps 3 --warmup 1 $*"
S2="rocprofv3 --pmc $SQ2 --output-format csv -d $OUT/sq2 -o pmc -- python3 $R/bench.py --profile --steps 3 --warmup 1 $*"
S3="rocprofv3 --pmc $SQ3 --output-format csv -d $OUT/sq3 -o pmc -- python3 $R/bench.py --profile --steps 3 --warmup 1 $*"
# the commands as run, with the repository root written as $REPO
printf '%s\n' "$T" "$F" "$W" "$S1" "$S2" "$S3" | sed "s#$R#\$REPO#g" > "$OUT/commands.txt"
echo "== kernel trace"
timeout -k 10 240 $T > "$OUT/trace.log" 2>&1 || exit $?
echo "== FETCH_SIZE"
timeout -s KILL 150 $F > "$OUT/fetch.log" 2>&1 || exit $?
echo "== WRITE_SIZE"
timeout -s KILL 150 $W > "$OUT/write.log" 2>&1 || exit $?
echo "== SQ counters (three passes)"
timeout -s KILL 150 $S1 > "$OUT/sq1.log" 2>&1 || exit $?
timeout -s KILL 150 $S2 > "$OUT/sq2.log" 2>&1 || exit $?
timeout -s KILL 150 $S3 > "$OUT/sq3.log" 2>&1 || exit $?
cd "$R" && python3 bench.py --summarize "$OUT" "$@"
