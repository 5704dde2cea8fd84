#!/bin/bash
# Turns the rocprofv3 runs under a profile directory (kernel statistics ks_<w>/, counter runs
# pmc_<w>_<counter>/, the copy calibration pmc_copy_<counter>/, the mixed step's pmc_mixed_mfma/)
# into the summaries under profiles/. Usage: graph_replay_amd/make_profiles.sh <profile dir>
set -e
P=$1
KS='rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- python3 bench.py --workload'
PM='rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -d <out> -o run -- python3 bench.py --workload'
CAL='; calibration: the same with python3 bench.py --copy-probe'
stats() {   # workload, output name
  python -m graph_replay_amd.profiling stats $P/ks_$1/run_kernel_stats.csv "$KS $1 --no-cpu --steps 16 --warmup 2" > profiles/$2
  python -m graph_replay_amd.profiling kinds $P/ks_$1/run_kernel_trace.csv >> profiles/$2
}
stats bs1 decode_qwen3-0.6b_bs1_ctx1024_kernels.md
stats bs32 decode_qwen3-0.6b_bs32_kernels.md
stats bs256 decode_qwen3-0.6b_bs256_kernels.md
stats mixed mixed_qwen2.5-1.5b_544tok_kernels.md
stats moe moe_qwen3-30b-a3b_layer_kernels.md
for pair in "bs1:qwen3-0.6b_bs1" "bs32:qwen3-0.6b-bf16-bs32-ctx128-2048" "bs256:qwen3-0.6b-bf16-bs256" \
            "mixed:qwen2.5-1.5b-f16-mixed-512+32" "moe:qwen3-30b-a3b-moe-layer-bf16"; do
  w=${pair%%:*}; n=${pair#*:}
  python -m graph_replay_amd.profiling traffic $P/pmc_copy_FETCH_SIZE $P/pmc_copy_WRITE_SIZE $P/pmc_${w}_FETCH_SIZE \
    $P/pmc_${w}_WRITE_SIZE "$n" "$PM $w --no-cpu --steps 8 --warmup 2$CAL" > profiles/hbm_traffic_$n.json
done
python -m graph_replay_amd.profiling counters $P/pmc_mixed_mfma qwen2.5-1.5b-f16-mixed-512+32 \
  "rocprofv3 --pmc MfmaUtil MfmaFlopsF16 --output-format csv -d <out> -o run -- python3 bench.py --workload mixed --no-cpu" \
  > profiles/mfma_qwen2.5-1.5b_544tok_counters.md
