"""Decode-step throughput on one MI355X at the Qwen3-0.6B shape (bf16, random N(0, 0.02) weights).

One "step" is one whole decode step (every layer, LM head, sampling, device-side advance), replayed
as the bucket's hipGraph. The primary line is batch 1 with a 1,024-token context built by a real
prefill, run as one persistent kernel with the sampler inside (--no-persistent: the multi-kernel graph);
the same JSON line carries the batch-32 workload (contexts uniform in [128, 2048], shuffled paged
KV, Gumbel-max at T = 1) under "bs32". Inputs are resident in HBM before the timed region.

    python bench.py [--gpus 1] [--steps 256] [--warmup 8] [--no-bs32] [--no-mixed] [--no-moe]
                    [--no-cpu] [--no-persistent] [--workload both|bs1|bs32|mixed|moe]

The line also carries the Qwen2.5-1.5B-shape mixed step (prefill chunks + decode rows, 544 packed
tokens) under "mixed": the bucketed plan replayed as a hipGraph against the exact-size eager plan;
and under "moe" the Qwen3-30B-A3B expert layer (grouping + two grouped GEMMs + k-sum) at 32 and
512 tokens, replayed as a graph.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0      # MI355X HBM3E, vendor figure
PEAK_MFMA_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 matrix cores, vendor figure
METRIC = "decode tokens/s/GPU at Qwen3-0.6B shape, bs 1 & 32; % of HBM roofline"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kind_bytes(shape, rows: int, seq_lens_sum: int, weight_prefetch: bool = False) -> dict:
    """Algorithmic HBM bytes of ONE launch of each kernel kind in a decode step of `rows` rows. With the
    weight prefetch (at most 8 rows), the attention launch also reads the layer's O, gate|up and down
    weights from HBM into L2 (the GEMVs then find them there), so they count for that launch."""
    eb = shape.elem_bytes
    H, I, V, d = shape.hidden, shape.intermediate, shape.vocab, shape.head_dim
    nq, nkv = shape.q_heads, shape.kv_heads
    qkv = shape.qkv_out
    staged = (H * nq * d + 2 * I * H + H * I) * eb if (weight_prefetch and rows <= 8) else 0
    return {
        "qkv_proj": qkv * H * eb + rows * qkv * 4,
        "o_proj": H * nq * d * eb + rows * H * 4,
        "gate_up_silu": 2 * I * H * eb + rows * I * eb,
        "down_proj": H * I * eb + rows * H * 4,
        "lm_head": V * H * eb + rows * V * 4,
        "attn_decode": seq_lens_sum * 2 * nkv * d * eb + rows * nq * d * (4 + eb) + staged,
        "qknorm_rope_kvwrite": rows * (qkv * 4 + nq * d * 4 + 2 * nkv * d * eb),
        "sample": rows * V * 4,
        "add_rmsnorm": rows * H * (4 + 4 + 4 + eb),
        # the whole single-row step in one kernel: every weight, the KV read, the logits written
        "decode_step_persistent": step_bytes(shape, seq_lens_sum) + rows * V * 4,
    }


def step_bytes(shape, seq_lens_sum: int) -> int:
    """Weights + KV read by one decode step (the roofline numerator)."""
    weights = synth.num_params(shape) * shape.elem_bytes
    kv = seq_lens_sum * shape.layers * 2 * shape.kv_heads * shape.head_dim * shape.elem_bytes
    return weights + kv


def timed_replays(dec, steps: int):
    torch = dec.torch
    s = dec.stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(steps):
        dec.decode_continue()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


WARM_RUNS, TIMED_RUNS = 2, 5


def timed_runs(dec, steps: int, refeed) -> dict:
    """The measurement protocol of the pages' benchmark (median of 5 timed runs after 2 warm-up
    runs). Every run starts from the same state: refeed() sends the workload's batch again and runs
    the warm-up steps (untimed), then exactly `steps` graph replays continue on the device, bracketed
    by synchronisations and HIP events on the decoder's stream. 2 runs untimed, 5 timed; the median
    run is the result."""
    runs = []
    for r in range(WARM_RUNS + TIMED_RUNS):
        refeed()
        ms = timed_replays(dec, steps)
        if r >= WARM_RUNS:
            runs.append(ms)
    med = float(np.median(runs))
    return {"median_ms": med, "runs_ms_per_step": [round(r / steps, 4) for r in runs],
            "protocol": f"{WARM_RUNS} warm-up runs, then the median of {TIMED_RUNS} timed runs of {steps} replays, "
                        "each from the same state"}


def measured_traffic(workload: str, kind: str):
    """HBM bytes per launch of `kind` from the committed rocprofv3 counter runs (profiles/), or None
    when there is no such run or the kernels changed since it was taken."""
    from graph_replay_amd import profiling
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    k = t.get("kinds", {}).get(kind)
    if t.get("source_hash") != profiling.source_hash() or not k:
        return None
    return int(k.get("fetch_bytes", 0) + k.get("write_bytes", 0))


def roofline_from_profile(shape, dec, rows: int, seq_lens_sum: int, weight_prefetch: bool = False) -> dict:
    prof = dec.profile_decode()
    per = {}
    for name, ms in prof:
        t = per.setdefault(name, [0.0, 0])
        t[0] += ms
        t[1] += 1
    dom = max(per, key=lambda k: per[k][0])
    avg_ms = per[dom][0] / per[dom][1]
    nbytes = kind_bytes(shape, rows, seq_lens_sum, weight_prefetch)[dom]
    achieved = nbytes / (avg_ms * 1e-3) / 1e9
    table = {k: {"launches": v[1], "total_us": round(v[0] * 1e3, 1), "avg_us": round(v[0] * 1e3 / v[1], 2)}
             for k, v in sorted(per.items(), key=lambda kv: -kv[1][0])}
    return {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
            "bytes_per_launch": int(nbytes), "avg_launch_us": round(avg_ms * 1e3, 2),
            "profile_sum_us": round(sum(ms for _, ms in prof) * 1e3, 1), "kernels": table}


def phase_breakdown(st, layers: int) -> dict:
    """Mean microseconds per layer between the phase stamps of a profiled persistent step (block 0's
    view): each interval ends when that phase's input has arrived (or, for attention, when block 0's
    attention item is done)."""
    names = ["to_qkv_in", "to_attn_done", "to_merge_done", "to_o_in", "to_mlp_in", "to_down_in"]
    acc = {n: 0.0 for n in names}
    for l in range(layers):
        prev = st[0] if l == 0 else st[8 * (l - 1) + 6]
        for k, n in enumerate(names):
            cur = st[8 * l + k + 1]
            acc[n] += cur - prev
            prev = cur
    out = {n: round(v / layers, 2) for n, v in acc.items()}
    out["final_norm_in"] = round(st[8 * layers + 1] - st[8 * (layers - 1) + 6], 2)
    out["lm_head"] = round(st[8 * layers + 2] - st[8 * layers + 1], 2)
    out["total"] = round(st[8 * layers + 2], 2)
    return out


def run_bs1(shape, W, steps: int, warmup: int, ctx_len: int = 1024, weight_prefetch: bool = True,
            persistent: bool = False):
    import graph_replay_amd as g
    torch = __import__("torch")
    total = ctx_len + 1 + warmup + steps + 2            # positions used, profile step included
    table = synth.block_tables([total], -(-total // 16) + 2, 1002, shuffled=False)[0]
    nb = len(table) + 2
    dec = g.Decoder(shape, W, num_blocks=nb, max_blocks_per_seq=len(table), max_position=total + 16, max_batch=1,
                    buckets=[1], max_tokens=ctx_len, max_reqs=1, max_logit_rows=1, weight_prefetch=weight_prefetch,
                    persistent_decode=persistent)
    bt = np.asarray([table], np.int32)
    prompt = synth.tokens(ctx_len, shape.vocab, 1002)
    pos = np.arange(ctx_len, dtype=np.int32)
    slots = (bt[0][pos // 16] * 16 + pos % 16).astype(np.int32)
    log("prefill", ctx_len, "tokens")
    dec.mixed([0, ctx_len], [ctx_len], prompt, pos, slots, bt, [ctx_len - 1], num_prefill_reqs=1)
    torch.cuda.synchronize()
    first = int(dec.tokens[0].item())
    p = ctx_len

    def refeed():
        dec.decode([first], [p], [p + 1], [int(bt[0][p // 16] * 16 + p % 16)], bt)
        for _ in range(warmup - 1):
            dec.decode_continue()
        torch.cuda.synchronize()

    start_len = ctx_len + 1 + warmup                      # seq_len of the first timed replay
    log("timing", steps, "bs1 steps x", TIMED_RUNS, "runs")
    tr = timed_runs(dec, steps, refeed)
    ms = tr["median_ms"]
    seq_sum_mean = start_len + (steps - 1) / 2.0
    nbytes = step_bytes(shape, seq_sum_mean)
    ms_step = ms / steps
    roof = roofline_from_profile(shape, dec, 1, start_len + steps, weight_prefetch)
    if dec.kernels_per_decode(1) == 1 and roof["kernel"] == "decode_step_persistent":
        # the graph is this one kernel: its launch time is the timed replays' (HIP events on the
        # decoder's stream), at the timed steps' mean context; the eager profiled step's own events
        # also hold launch overhead, so they stay as a cross-check only
        nb = kind_bytes(shape, 1, seq_sum_mean, weight_prefetch)[roof["kernel"]]
        roof["eager_profile_avg_us"] = roof["avg_launch_us"]
        roof["avg_launch_us"] = round(ms_step * 1e3, 2)
        roof["bytes_per_launch"] = int(nb)
        roof["achieved"] = round(nb / (ms_step * 1e-3) / 1e9, 1)
        roof["frac"] = round(roof["achieved"] / PEAK_HBM_GBS, 4)
        roof["launch_time"] = "timed graph replays"
    roof["traffic"] = measured_traffic("qwen3-0.6b_bs1", roof["kernel"])
    if persistent:
        st = dec.phase_stamps()
        if st is not None:
            roof["phases_us"] = phase_breakdown(st, shape.layers)
    dec.device_status()
    out = {
        "tok_s": steps / (ms * 1e-3), "ms_per_step": ms_step, "bytes_per_step": int(nbytes),
        "step_hbm_GBps": nbytes / (ms_step * 1e-3) / 1e9, "kernels_per_step": dec.kernels_per_decode(1),
        "roofline": roof, "timing": {k: v for k, v in tr.items() if k != "median_ms"},
    }
    out["step_hbm_frac"] = out["step_hbm_GBps"] / PEAK_HBM_GBS
    dec.close()
    del dec
    torch.cuda.empty_cache()
    return out


def run_bs32(shape, W, steps: int, warmup: int, wl=None):
    """A many-row decode workload (batch 32 by default; the batch-256 workload with wl) over seeded
    N(0, 1) KV histories resident in HBM, Gumbel-max at the workload's temperature, shuffled tables."""
    import graph_replay_amd as g
    torch = __import__("torch")
    wl = wl or synth.workload_q3_bs32()
    ctx = wl.contexts
    B = len(ctx)
    need = [c + 1 + warmup + steps + 2 for c in ctx]
    nb = sum(-(-n // 16) for n in need) + 2
    tables = synth.block_tables(need, nb, 1003, shuffled=True)
    width = max(len(t) for t in tables)
    dec = g.Decoder(shape, W, num_blocks=nb, max_blocks_per_seq=width, max_position=max(need) + 16, max_batch=B,
                    buckets=wl.buckets)
    gen = torch.Generator(device=dec.device)
    gen.manual_seed(wl.input_seed)
    for l in range(shape.layers):                       # seeded N(0, 1) KV history, resident in HBM
        dec.k_pool[l].normal_(generator=gen)
        dec.v_pool[l].normal_(generator=gen)
    bt = np.full((B, width), -1, np.int32)
    for j, t in enumerate(tables):
        bt[j, :len(t)] = t
    pos = np.asarray(ctx, np.int32)
    slots = np.array([bt[j][pos[j] // 16] * 16 + pos[j] % 16 for j in range(B)], np.int32)
    toks = synth.tokens(B, shape.vocab, wl.input_seed)

    def refeed():
        dec.decode(toks, pos, pos + 1, slots, bt, temperature=np.full(B, wl.temperature, np.float32),
                   seed=wl.input_seed)
        for _ in range(warmup - 1):
            dec.decode_continue()
        torch.cuda.synchronize()

    log("timing", steps, f"bs{B} steps x", TIMED_RUNS, "runs")
    tr = timed_runs(dec, steps, refeed)
    ms = tr["median_ms"]
    start_sum = sum(c + 1 + warmup for c in ctx)
    seq_sum_mean = start_sum + B * (steps - 1) / 2.0
    nbytes = step_bytes(shape, seq_sum_mean)
    ms_step = ms / steps
    roof = roofline_from_profile(shape, dec, B, start_sum + B * steps)
    roof["traffic"] = measured_traffic(wl.name, roof["kernel"])
    out = {"workload": wl.name, "batch": B, "tok_s": B * steps / (ms * 1e-3), "ms_per_step": ms_step,
           "bytes_per_step": int(nbytes), "step_hbm_GBps": nbytes / (ms_step * 1e-3) / 1e9,
           "kernels_per_step": dec.kernels_per_decode(B), "roofline": roof,
           "timing": {k: v for k, v in tr.items() if k != "median_ms"}}
    out["step_hbm_frac"] = out["step_hbm_GBps"] / PEAK_HBM_GBS
    dec.close()
    return out


def mixed_flops(shape, prefill_lens, decode_ctx, n_logits: int) -> float:
    """Algorithmic FLOPs of one mixed step: linears over every packed token, the LM head over the
    sampled rows, causal attention of each prefill chunk and one query row per decode request."""
    H, I, d, nq, nkv = shape.hidden, shape.intermediate, shape.head_dim, shape.q_heads, shape.kv_heads
    lin = shape.layers * ((nq + 2 * nkv) * d * H + H * nq * d + 2 * I * H + H * I)
    T = sum(prefill_lens) + len(decode_ctx)
    att = sum(n * (n + 1) // 2 for n in prefill_lens) + sum(c + 1 for c in decode_ctx)
    return 2.0 * lin * T + 2.0 * shape.vocab * H * n_logits + 4.0 * d * nq * att * shape.layers


def run_mixed(steps: int = 20, warmup: int = 2) -> dict:
    """The Qwen2.5-1.5B-shape mixed step (prefill chunks 16/240/256 + 32 decode rows, 544 packed
    tokens, 35 sampled rows), median step time over `steps` steps: the bucketed plan replayed as a
    hipGraph (bucket 576) and the exact-size plan launched eagerly."""
    import graph_replay_amd as g
    torch = __import__("torch")
    wl = synth.workload_q25_mixed()
    shape = wl.shape
    log("mixed weights")
    W = synth.make_weights(shape, 0)
    P = len(wl.prefill_lens)
    need = [n + 1 for n in wl.prefill_lens] + [c + 1 for c in wl.decode_contexts]
    nb = sum(-(-n // 16) for n in need) + 2
    tables = synth.block_tables(need, nb, wl.input_seed, shuffled=True)
    width = max(len(t) for t in tables)
    bt = np.full((len(tables), width), -1, np.int32)
    for j, t in enumerate(tables):
        bt[j, :len(t)] = t
    toks, pos, slots, qsl, lens, lidx = [], [], [], [0], [], []
    for j, n in enumerate(wl.prefill_lens):
        toks += list(synth.tokens(n, shape.vocab, wl.input_seed + 10 + j))
        pos += list(range(n))
        slots += [int(bt[j][p // 16] * 16 + p % 16) for p in range(n)]
        qsl.append(qsl[-1] + n); lens.append(n); lidx.append(qsl[-1] - 1)
    dtok = synth.tokens(len(wl.decode_contexts), shape.vocab, wl.input_seed + 99)
    for i, c in enumerate(wl.decode_contexts):
        j = P + i
        toks.append(int(dtok[i])); pos.append(c); slots.append(int(bt[j][c // 16] * 16 + c % 16))
        qsl.append(qsl[-1] + 1); lens.append(c + 1); lidx.append(qsl[-1] - 1)
    T, R = qsl[-1], len(lens)
    out = {"workload": wl.name, "tokens": T, "sampled_rows": len(lidx)}
    for name, buckets in (("graph", [T + (-T) % 64]), ("eager", None)):
        dec = g.Decoder(shape, W, num_blocks=nb, max_blocks_per_seq=width, max_position=max(need) + 16, max_batch=1,
                        buckets=[1], max_tokens=T + (-T) % 64, max_reqs=R, max_logit_rows=R,
                        mixed_buckets=buckets)
        gen = torch.Generator(device=dec.device)
        gen.manual_seed(wl.input_seed)
        for l in range(shape.layers):                   # seeded N(0, 1) KV history, resident in HBM
            dec.k_pool[l].normal_(generator=gen)
            dec.v_pool[l].normal_(generator=gen)
        args = dict(query_start_loc=qsl, seq_lens=lens, tokens=toks, positions=pos, slots=slots, block_table=bt,
                    logits_indices=lidx, num_prefill_reqs=P)
        for _ in range(warmup):
            dec.mixed(**args)
        torch.cuda.synchronize()
        log("timing", steps, "mixed steps,", name)
        times = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(dec.stream)
            dec.mixed(**args)
            e1.record(dec.stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        out[f"{name}_bucket"] = dec.last_mixed_bucket()
        out[f"ms_per_step_{name}"] = round(float(np.median(times)), 4)
        dec.close()
        del dec
        torch.cuda.empty_cache()
    flops = mixed_flops(shape, wl.prefill_lens, wl.decode_contexts, len(lidx))
    ms = out["ms_per_step_graph"]
    out["value"] = round(T / (ms * 1e-3), 1)
    out["unit"] = "tokens/s"
    out["step_mfma"] = {"flops_per_step": flops, "achieved": round(flops / (ms * 1e-3) / 1e12, 1),
                        "peak": PEAK_MFMA_F16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(flops / (ms * 1e-3) / 1e12 / PEAK_MFMA_F16_TFLOPS, 4)}
    return out


def moe_layer_bytes(s, n: int, active: int) -> dict:
    """Algorithmic HBM bytes of one MoE layer call per kernel: every active expert's weights once,
    each token row once, the activation rows written then read (dtype), the weighted down rows
    written then read (fp32), the output written, and the grouping's small int32 arrays."""
    eb = 2
    D, I, k = s.hidden, s.inter, s.top_k
    total = n * k
    m_max = -(-(total + s.experts * 15) // 16) * 16
    return {
        "moe_align": total * 4 + (m_max + m_max // 16 + 1) * 4,
        "moe_gate_up": active * 2 * I * D * eb + n * D * eb + total * I * eb + m_max * 4,
        "moe_down": active * D * I * eb + total * I * eb + total * D * 4 + total * 4 + m_max * 4,
        "moe_sum": total * D * 4 + n * D * eb + total * 4,
    }


def run_moe(steps: int = 50) -> dict:
    """The Qwen3-30B-A3B expert layer (128 experts, 8 per token, hidden 2048, width 768, bf16) at a
    32-token decode batch and a 512-token chunk: moe_forward (4 kernels) captured as a graph over
    static buffers and replayed `steps` times; HBM bytes of the whole call over its time."""
    import graph_replay_amd as g
    torch = __import__("torch")
    from synth import moe as smoe
    s = smoe.QWEN3_30B_A3B_MOE
    log("moe weights")
    gu, dn = (t.cuda() for t in smoe.make_moe_weights(s, 0))
    out = {"workload": "qwen3-30b-a3b-moe-layer-bf16", "experts": s.experts, "top_k": s.top_k,
           "hidden": s.hidden, "inter": s.inter, "kernels_per_layer": 4}
    for n in (32, 512):
        x = smoe.token_rows(s, n, 3000 + n).cuda()
        ids, w = smoe.routing(s, n, 3000 + n)
        d_ids, d_w = torch.as_tensor(ids).cuda(), torch.as_tensor(w).cuda()
        y = torch.empty_like(x)
        ws = torch.empty(g.moe_workspace_bytes(x, gu, dn, d_w, d_ids, y), dtype=torch.uint8, device="cuda")
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for _ in range(3):
                g.moe_forward(x, gu, dn, d_w, d_ids, y, ws)
        stream.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            g.moe_forward(x, gu, dn, d_w, d_ids, y, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            graph.replay()
            e0.record(stream)
            for _ in range(steps):
                graph.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        active = int(np.unique(ids).size)
        kb = moe_layer_bytes(s, n, active)
        nbytes = sum(kb.values())
        flops = 2 * n * s.top_k * 3 * s.inter * s.hidden
        out[f"n{n}"] = {"tokens": n, "active_experts": active, "us_per_layer": round(us, 2),
                        "bytes_per_layer": int(nbytes),
                        "hbm": {"achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
                        "mfma": {"achieved": round(flops / (us * 1e-6) / 1e12, 1), "peak": PEAK_MFMA_F16_TFLOPS,
                                 "unit": "TFLOP/s"},
                        "kernel_bytes": kb}
        log(f"moe n={n}: {us:.1f} us per layer, {active} experts")
        del graph
    return out


def cpu_baseline(shape, W, budget_s: float = 20.0, ctx_len: int = 1024) -> dict:
    """The oracle (fp32 NumPy, unfused, per request) timed on this host on a bounded sample: decode
    steps of one request over a 1,024-key injected history (same shape as the GPU workload)."""
    import oracle
    from threadpoolctl import threadpool_info
    w32 = {"embed": W["embed"].float().numpy(), "final_norm": W["final_norm"].float().numpy(),
           "layers": [{k: (None if v is None else v.float().numpy()) for k, v in l.items()} for l in W["layers"]]}
    w32["lm_head"] = w32["embed"]
    cache = oracle.RequestCache(shape.layers)
    for l in range(shape.layers):
        k, v = synth.injected_kv(shape, 1002, 0, l, ctx_len)
        cache.set(l, k.float().numpy(), v.float().numpy())
    tok = int(synth.tokens(1, shape.vocab, 5)[0])
    times = []
    t_start = time.perf_counter()
    p = ctx_len
    while True:
        t0 = time.perf_counter()
        hid = oracle.forward_request(shape, w32, cache, [tok], [p])
        tok = int(oracle.sample(oracle.final_logits(w32, hid), 0.0)[0])
        times.append(time.perf_counter() - t0)
        p += 1
        if time.perf_counter() - t_start > budget_s or len(times) >= 64:
            break
    med = float(np.median(times[1:] if len(times) > 2 else times))
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    return {"value": round(1.0 / med, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} greedy decode steps of one request over a {ctx_len}-key injected history, "
                      f"Qwen3-0.6B shape fp32 NumPy; median step {med * 1e3:.1f} ms",
            "host_cpus": os.cpu_count()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--no-bs32", action="store_true")
    ap.add_argument("--workload", choices=["both", "bs1", "bs32", "bs256", "mixed", "moe"], default="both",
                    help="bs1: the primary line only; bs32 / bs256 / mixed / moe: that workload only (for profiling)")
    ap.add_argument("--no-bs256", action="store_true")
    ap.add_argument("--bs256-steps", type=int, default=32,
                    help="replays per timed run of the batch-256 workload (each run holds 256 rows x steps keys more)")
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--no-mixed", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy a 1 GiB device buffer 4 times (calibrates the HBM byte counters)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-weight-prefetch", action="store_true",
                    help="batch-1 step without the L2 weight prefetch in the attention launches")
    ap.add_argument("--no-persistent", action="store_true",
                    help="batch-1 step as the multi-kernel graph instead of one persistent kernel")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the decode step shards by request, with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    warmup = max(1, args.warmup)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X (no GPU visible)", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")     # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 1 << 30, "copies": 4}), flush=True)
        return
    import graph_replay_amd as g
    g.load()
    shape = synth.QWEN3_0_6B
    log("weights")
    W = synth.make_weights(shape, 0)
    if args.workload == "bs32":
        r32 = run_bs32(shape, W, args.steps, warmup)
        print(json.dumps({"metric": METRIC, "workload": r32["workload"], "value": round(r32["tok_s"], 1),
                          "unit": "tokens/s", "ms_per_step": round(r32["ms_per_step"], 4),
                          "kernels_per_step": r32["kernels_per_step"], "roofline": r32["roofline"]}), flush=True)
        return
    if args.workload == "bs256":
        r = run_bs32(shape, W, min(args.steps, args.bs256_steps), warmup, synth.workload_q3_bs256())
        print(json.dumps({"metric": METRIC, "workload": r["workload"], "value": round(r["tok_s"], 1),
                          "unit": "tokens/s", "ms_per_step": round(r["ms_per_step"], 4),
                          "kernels_per_step": r["kernels_per_step"], "roofline": r["roofline"]}), flush=True)
        return
    if args.workload == "mixed":
        print(json.dumps({"metric": METRIC, **run_mixed()}), flush=True)
        return
    if args.workload == "moe":
        print(json.dumps({"metric": METRIC, "moe": run_moe()}), flush=True)
        return
    r1 = run_bs1(shape, W, args.steps, warmup, weight_prefetch=not args.no_weight_prefetch,
                 persistent=not args.no_persistent)
    r32 = None if (args.no_bs32 or args.workload == "bs1") else run_bs32(shape, W, args.steps, warmup)
    r256 = None if (args.no_bs256 or args.workload == "bs1") else run_bs32(
        shape, W, min(args.steps, args.bs256_steps), warmup, synth.workload_q3_bs256())
    rmix = None if (args.no_mixed or args.workload == "bs1") else run_mixed()
    rmoe = None if (args.no_moe or args.workload == "bs1") else run_moe()
    cpu = None if args.no_cpu else cpu_baseline(shape, W)
    line = {
        "metric": METRIC, "value": round(r1["tok_s"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": warmup, "ms_per_step": round(r1["ms_per_step"], 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3-0.6b-bf16-decode-bs1-ctx1024", "batch": 1, "context": 1024,
                   "decode_steps": args.steps,
                   "graph": "one hipGraph replay per step" + ("" if args.no_persistent else
                                                               " (one persistent kernel, sampling inside)"),
                   "kernels_per_step": r1["kernels_per_step"], "weight_prefetch": not args.no_weight_prefetch,
                   "persistent_decode": not args.no_persistent},
        "step_hbm": {"bytes_per_step": r1["bytes_per_step"], "achieved": round(r1["step_hbm_GBps"], 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(r1["step_hbm_frac"], 4)},
        "roofline": r1["roofline"],
        "timing": r1["timing"],
        "cpu_baseline": cpu,
    }
    for key, r in (("bs32", r32), ("bs256", r256)):
        if r is not None:
            line[key] = {"workload": r["workload"], "value": round(r["tok_s"], 1), "unit": "tokens/s",
                         "ms_per_step": round(r["ms_per_step"], 4), "kernels_per_step": r["kernels_per_step"],
                         "step_hbm": {"bytes_per_step": r["bytes_per_step"], "achieved": round(r["step_hbm_GBps"], 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(r["step_hbm_frac"], 4)},
                         "roofline": r["roofline"], "timing": r["timing"]}
    if rmix is not None:
        line["mixed"] = rmix
    if rmoe is not None:
        line["moe"] = rmoe
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
