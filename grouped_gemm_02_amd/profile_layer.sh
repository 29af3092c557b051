#!/bin/bash
# Profiles the layer with rocprofv3 on an MI355X and writes the summaries
# that are kept under profiles/ into <out_dir>/profiles. Usage (from the
# repository root):
#   bash grouped_gemm_02_amd/profile_layer.sh <out_dir>
# Kernel statistics for every workload (20 timed steps after 5 warm-up
# steps), then counter passes, each its own run: FETCH_SIZE, WRITE_SIZE and
# the MFMA-busy pair for the EP=8 share (fp32-scale FP8), the MFMA-busy pair
# and FETCH_SIZE / WRITE_SIZE for the default 30B bf16 workload.
set -e
OUT=${1:-rocprof_out}
export TMPDIR=/tmp
PROF="$OUT/profiles"
mkdir -p "$OUT" "$PROF"
# workload:precision:weight-gradient reading:router step
for cpw in qwen3_30b:bf16:bf16:none ep8_share:fp8_block_f32:bf16:none qwen3_235b:fp8_bwd_f32:bf16:none \
           zipf:mxfp8:bf16:none ep8_share:fp8_block:bf16:none qwen3_235b:fp8_bwd:bf16:none \
           ep8_share:fp8_block:fp8:none qwen3_235b:fp8_bwd:fp8:none zipf:mxfp8:fp8:none \
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
# counter passes (each its own short run): pmc TAG NAME "COUNTERS" BENCH-ARGS...
pmc() {
  local tag=$1 name=$2 ctrs=$3; shift 3
  echo "pmc $tag $name"
  timeout -s KILL 120 rocprofv3 --pmc $ctrs --output-format csv -d "$OUT/pmc_${tag}_$name" -o pmc -- \
    python3 bench.py "$@" --steps 2 --warmup 1 --no-cpu-baseline > "$OUT/pmc_${tag}_$name.log" 2>&1
}
# FP8 (the EP=8 share with fp32 block scales): HBM traffic and MFMA busy
T8=ep8_share_fp8_block_f32
pmc $T8 fetch FETCH_SIZE --config ep8_share
pmc $T8 write WRITE_SIZE --config ep8_share
pmc $T8 mfma "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE" --config ep8_share
python3 -m grouped_gemm_02_amd.profile_summary traffic "$OUT/pmc_${T8}_fetch/pmc_counter_collection.csv" \
  "$OUT/pmc_${T8}_write/pmc_counter_collection.csv" "$PROF/gemm_traffic_$T8.json" --workload ep8_share/fp8_block_f32 \
  --cmd "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_${T8}_fetch -o pmc -- python3 bench.py --config ep8_share --steps 2 --warmup 1 --no-cpu-baseline ; rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_${T8}_write -o pmc -- python3 bench.py --config ep8_share --steps 2 --warmup 1 --no-cpu-baseline"
python3 -m grouped_gemm_02_amd.profile_summary mfma "$OUT/pmc_${T8}_mfma/pmc_counter_collection.csv" \
  "$PROF/mfma_busy_$T8.txt" --title "EP=8 share of the 30B layer, blockwise FP8 with fp32 scales" \
  --cmd "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $OUT/pmc_${T8}_mfma -o pmc -- python3 bench.py --config ep8_share --steps 2 --warmup 1 --no-cpu-baseline"
# the other FP8 workloads: MFMA busy
for t in zipf_mxfp8:zipf:"Qwen3-30B-A3B shape, Zipf(1.2) routing, MXFP8" \
         qwen3_235b_fp8_bwd_f32:qwen3_235b:"Qwen3-235B-A22B shape, bf16 forward, blockwise FP8 backward with fp32 scales"; do
  IFS=: read -r tag cfg title <<< "$t"
  pmc $tag mfma "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE" --config $cfg
  python3 -m grouped_gemm_02_amd.profile_summary mfma "$OUT/pmc_${tag}_mfma/pmc_counter_collection.csv" \
    "$PROF/mfma_busy_$tag.txt" --title "$title" \
    --cmd "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $OUT/pmc_${tag}_mfma -o pmc -- python3 bench.py --config $cfg --steps 2 --warmup 1 --no-cpu-baseline"
done
# bf16 (the 30B layer): MFMA busy
pmc qwen3_30b_bf16 mfma "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE" --config qwen3_30b
python3 -m grouped_gemm_02_amd.profile_summary mfma "$OUT/pmc_qwen3_30b_bf16_mfma/pmc_counter_collection.csv" \
  "$PROF/mfma_busy_qwen3_30b_bf16.txt" --title "Qwen3-30B-A3B-shaped layer, bf16" \
  --cmd "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $OUT/pmc_qwen3_30b_bf16_mfma -o pmc -- python3 bench.py --config qwen3_30b --steps 2 --warmup 1 --no-cpu-baseline"
echo "pmc fetch"
timeout -s KILL 120 rocprofv3 --pmc FETCH_SIZE --output-format csv -d "$OUT/pmc_fetch" -o pmc -- \
  python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > "$OUT/pmc_fetch.log" 2>&1
echo "pmc write"
timeout -s KILL 120 rocprofv3 --pmc WRITE_SIZE --output-format csv -d "$OUT/pmc_write" -o pmc -- \
  python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline > "$OUT/pmc_write.log" 2>&1
python3 -m grouped_gemm_02_amd.profile_summary traffic "$OUT/pmc_fetch/pmc_counter_collection.csv" \
  "$OUT/pmc_write/pmc_counter_collection.csv" "$PROF/gemm_traffic_qwen3_30b_bf16.json" --workload qwen3_30b/bf16 \
  --cmd "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT/pmc_fetch -o pmc -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline ; rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT/pmc_write -o pmc -- python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline"
# bf16 (the 30B layer): LDS bank conflicts
pmc qwen3_30b_bf16 lds "SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS" --config qwen3_30b
python3 -m grouped_gemm_02_amd.profile_summary lds "$OUT/pmc_qwen3_30b_bf16_lds/pmc_counter_collection.csv" \
  "$PROF/lds_bank_conflicts_qwen3_30b_bf16.txt" --title "Qwen3-30B-A3B-shaped layer, bf16" \
  --cmd "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS --output-format csv -d $OUT/pmc_qwen3_30b_bf16_lds -o pmc -- python3 bench.py --config qwen3_30b --steps 2 --warmup 1 --no-cpu-baseline"
echo "profiles written"
