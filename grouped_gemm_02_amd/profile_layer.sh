#!/bin/bash
# Profiles the layer with rocprofv3 on an MI355X and writes the summaries
# that are kept under profiles/ into <out_dir>/profiles. Usage (from the
# repository root):
#   bash grouped_gemm_02_amd/profile_layer.sh <out_dir>
# Kernel statistics for every workload (the bench defaults: 20 timed steps
# after 5 warm-up steps, so the averages compare with its event timings),
# then FETCH_SIZE and WRITE_SIZE counter passes (separate runs) for the
# default workload.
set -e
OUT=${1:-rocprof_out}
export TMPDIR=/tmp
PROF="$OUT/profiles"
mkdir -p "$OUT" "$PROF"
# workload:precision:weight-gradient reading:router step
for cpw in qwen3_30b:bf16:bf16:none ep8_share:fp8_block:bf16:none qwen3_235b:fp8_bwd:bf16:none \
           zipf:mxfp8:bf16:none ep8_share:fp8_block:fp8:none qwen3_235b:fp8_bwd:fp8:none zipf:mxfp8:fp8:none \
           qwen3_30b:bf16:bf16:skewed qwen3_30b:fp8_fp4:bf16:none; do
  IFS=: read -r c prec wg rt <<< "$cpw"
  tag=${c}_${prec}; [ "$wg" = fp8 ] && tag=${tag}_fp8_wgrad; [ "$rt" != none ] && tag=${tag}_router_${rt}
  echo "stats $tag"
  args="--config $c --precision $prec --wgrad $wg --router $rt --steps 20 --warmup 5 --no-cpu-baseline"
  timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d "$OUT/stats_$tag" -o run -- \
    python3 bench.py $args > "$OUT/stats_$tag.log" 2>&1
  python3 -m grouped_gemm_02_amd.profile_summary stats "$OUT/stats_$tag/run_kernel_stats.csv" \
    "$PROF/kernel_stats_${tag}.txt" --cmd "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT/stats_$tag -o run -- python3 bench.py $args"
done
echo "pmc fetch"
timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/pmc_fetch" -o pmc -- \
  python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > "$OUT/pmc_fetch.log" 2>&1
echo "pmc write"
timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/pmc_write" -o pmc -- \
  python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > "$OUT/pmc_write.log" 2>&1
python3 -m grouped_gemm_02_amd.profile_summary traffic "$OUT/pmc_fetch/pmc_counter_collection.csv" \
  "$OUT/pmc_write/pmc_counter_collection.csv" "$PROF/gemm_traffic_qwen3_30b_bf16.json" --workload qwen3_30b/bf16 \
  --cmd "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o pmc -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline ; rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o pmc -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline"
echo "profiles written"
