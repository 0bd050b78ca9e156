#!/bin/bash
# rocprofv3 runs behind the committed summaries under profiles/: a kernel trace of
# the benchmark, then one counter pass each for FETCH_SIZE and WRITE_SIZE (with the
# 512 MiB calibration copy of bench.py --profile), then the summaries.
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
# the commands as run, with the repository root written as $REPO
printf '%s\n' "$T" "$F" "$W" | sed "s#$R#\$REPO#g" > "$OUT/commands.txt"
echo "== kernel trace"
timeout -k 10 240 $T > "$OUT/trace.log" 2>&1 || exit $?
echo "== FETCH_SIZE"
timeout -s KILL 150 $F > "$OUT/fetch.log" 2>&1 || exit $?
echo "== WRITE_SIZE"
timeout -s KILL 150 $W > "$OUT/write.log" 2>&1 || exit $?
cd "$R" && python3 bench.py --summarize "$OUT" "$@"
