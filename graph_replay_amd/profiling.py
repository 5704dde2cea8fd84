"""Summaries of rocprofv3 output for profiles/ (measurement tooling, not the step itself).

    python -m graph_replay_amd.profiling stats <run>_kernel_stats.csv "<command>" > profiles/<name>.md
    python -m graph_replay_amd.profiling kinds <run>_kernel_trace.csv >> profiles/<name>.md
    python -m graph_replay_amd.profiling traffic <copy FETCH dir> <copy WRITE dir> <FETCH dir> <WRITE dir> \\
        <workload> "<command>" > profiles/hbm_traffic_<workload>.json
    python -m graph_replay_amd.profiling counters <pmc dir> <workload> "<command>" > profiles/<name>.md

`traffic` turns two `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs into HBM bytes per launch:
each counter (KiB per dispatch) is scaled by what it reads for a plain 1 GiB device copy
(`bench.py --copy-probe`), so the figure is in true bytes. Dispatches are named by the decode-step
kernel kind they belong to; the JSON carries a hash of the kernel sources, and bench.py reports the
traffic only while the sources still hash the same.
"""
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30


def source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(HERE, "csrc", "*"))):
        h.update(os.path.basename(p).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def stats(path: str, cmd: str) -> None:
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("# rocprofv3 kernel statistics\n")
    print("Command (run from /tmp with TMPDIR=/tmp on one MI355X):\n")
    print("```\n" + cmd + "\n```\n")
    print("| calls | avg (us) | min (us) | max (us) | total (ms) | % | kernel |")
    print("|---:|---:|---:|---:|---:|---:|---|")
    for r in rows[:25]:
        name = r["Name"].replace("|", "\\|")
        if len(name) > 110:
            name = name[:107] + "..."
        print(f"| {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
              f"{float(r['Percentage']):.2f} | `{name}` |")


def kinds(trace: str) -> None:
    """Markdown table of kernel durations per decode-step kind (batch-1 Qwen3-0.6B dispatches,
    told apart by kernel name and grid size) from a rocprofv3 kernel trace."""
    acc = {}
    for r in csv.DictReader(open(trace)):
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        k = _kind_bs1(r["Kernel_Name"], grid)
        if k:
            acc.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    print("\nPer decode-step kind (kernel trace of the same run; the two projections of the multi-kernel")
    print("step that share the `k_gemv<BF16, 1, 2, 2>` instantiation are told apart by grid size):\n")
    print("| kind | calls | avg (us) | median (us) |")
    print("|---|---:|---:|---:|")
    for k, v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        print(f"| {k} | {len(v)} | {sum(v) / len(v) / 1e3:.2f} | {v[len(v) // 2] / 1e3:.2f} |")


def _counter_rows(d: str):
    return list(csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))))


def _copy_factor(d: str) -> float:
    vals = [float(r["Counter_Value"]) * 1024 for r in _counter_rows(d) if "copyBuffer" in r["Kernel_Name"]]
    return COPY_BYTES / (sum(vals) / len(vals))


# Which decode-step kernel kind a (kernel, grid size) dispatch of the batch-1 Qwen3-0.6B step is.
def _kind_bs1(name: str, grid: int) -> str:
    if "k_persist_decode" in name:
        return "decode_step_persistent"
    if "k_attn_rows" in name:
        return "attn_decode"
    if "k_sample" in name:
        return "sample"
    if "k_gemv<gr::BF16, 1, 8, 2>" in name:
        return "lm_head"
    if "k_gemv<gr::BF16, 1, 1, 8>" in name:
        return "down_proj"
    if "k_gemv<gr::BF16, 1, 1, 4>" in name:
        return "o_proj"
    if "k_gemv<gr::BF16, 1, 2, 2>" in name:
        return "gate_up_silu" if grid == 196608 else "qkv_proj"
    return ""


# The kind of a dispatch of any other workload: the step's kernels by name, the projections by
# kernel and grid size (each projection of a step has its own grid).
_NAMED = (("k_persist_decode", "decode_step_persistent"), ("k_attn_prefill", "attn_prefill"),
          ("k_attn_rows", "attn_decode"), ("k_attn_flat", "attn_decode"), ("k_sample_filter", "sample_filter"), ("k_sample", "sample"),
          ("k_add_rmsnorm", "add_rmsnorm"), ("k_qkv_post", "qknorm_rope_kvwrite"), ("k_gemv_stream", "lm_head"),
          ("k_moe_align", "moe_align"), ("k_moe_sum", "moe_sum"))


def _kind(name: str, grid: int, workload: str) -> str:
    if "bs1" in workload:
        return _kind_bs1(name, grid)
    for key, kind in _NAMED:
        if key in name:
            return kind
    if "k_moe_gemm" in name:
        return "moe_gate_up" if ", true," in name else "moe_down"
    for key in ("k_gemv_mfma", "k_gemm_ring", "k_gemm", "k_gemv"):
        if key + "<" in name:
            return f"{key}[grid {grid}]"
    return ""


def traffic(cf: str, cw: str, f: str, w: str, workload: str, cmd: str) -> None:
    ff, wf = _copy_factor(cf), _copy_factor(cw)
    kinds = {}
    # per kind, the launch shape with the most dispatches (the timed bucket's; the graph captures of
    # the other buckets at init launch the same kinds on other grids)
    for d, fac, key in ((f, ff, "fetch_bytes"), (w, wf, "write_bytes")):
        acc = {}
        for r in _counter_rows(d):
            k = _kind(r["Kernel_Name"], int(r["Grid_Size"]), workload)
            if k:
                acc.setdefault(k, {}).setdefault(int(r["Grid_Size"]), []).append(
                    float(r["Counter_Value"]) * 1024 * fac)
        for k, grids in acc.items():
            grid, v = max(grids.items(), key=lambda gv: (len(gv[1]), gv[0]))
            kinds.setdefault(k, {})[key] = round(sum(v) / len(v))
            kinds[k]["dispatches"] = len(v)
            kinds[k]["grid"] = grid
            if len(grids) > 1:
                per = kinds[k].setdefault("by_grid", {})
                for gsz, vv in sorted(grids.items()):
                    per.setdefault(str(gsz), {})[key] = round(sum(vv) / len(vv))
                    per[str(gsz)]["dispatches"] = len(vv)
    print(json.dumps({"source_hash": source_hash(), "workload": workload, "command": cmd,
                      "fetch_factor": round(ff, 4), "write_factor": round(wf, 4), "kinds": kinds}, indent=1))


def counters(d: str, workload: str, cmd: str) -> None:
    """Markdown table of the mean of every counter per dispatch kind of one rocprofv3 --pmc run."""
    acc = {}
    for r in _counter_rows(d):
        k = _kind(r["Kernel_Name"], int(r["Grid_Size"]), workload) or r["Kernel_Name"][:60]
        acc.setdefault((k, r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    names = sorted({c for _, c in acc})
    print(f"# rocprofv3 counters per dispatch, {workload}\n")
    print("Command (run from /tmp with TMPDIR=/tmp on one MI355X):\n")
    print("```\n" + cmd + "\n```\n")
    print("| kind | dispatches | " + " | ".join(names) + " |")
    print("|---|---:|" + "---:|" * len(names))
    for k in sorted({k for k, _ in acc}):
        vals = [acc.get((k, c), []) for c in names]
        n = max(len(v) for v in vals)
        print(f"| {k} | {n} | " + " | ".join(f"{sum(v) / len(v):.4g}" if v else "" for v in vals) + " |")


if __name__ == "__main__":
    if sys.argv[1] == "counters":
        counters(sys.argv[2], sys.argv[3], sys.argv[4])
    elif sys.argv[1] == "stats":
        stats(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "kinds":
        kinds(sys.argv[2])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:8])
    else:
        raise SystemExit(__doc__)
