"""Benchmark: one Cross-Decoder group step (full attention + importance, token
top-k with the forced window, N KV-reusing sparse layers) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints ONE JSON line.  With no --workload the line is the headline measurement,
decode at 1M context (batch 1, 32 query / 4 KV heads, head dim 128, 8 sparse
layers, top-1024 + recent 128): `value` is query tokens per second of the
whole step with inputs resident in HBM; `roofline` rates the dominant kernel
(the full layer's split-context stream) by its algorithmic bytes (K + V + Q + O
+ 4 bytes of importance per key row) over its own average duration, timed with
HIP events on the stream it runs on, against the datasheet peak and against
the streaming-read ceiling measured on the same device; `cpu_baseline` is the
float64 CPU oracle on a bounded sample of the same workload.  The same line
carries every other workload (`workloads`: step times, tokens/s, phases and
roofline of each; cold-cache and HIP-graph timings where the protocol asks for
them) and the prefill early-exit timing (`early_exit`).  --workload NAME prints
one such line for that workload alone (and its variants: --select-block,
--swa-branch, --graph; the KV Bridging workloads bridge_prompt_128k /
bridge_append_b16; prefill_early_exit).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "query tokens/s, full+sparse Cross-Decoder attn at 1M ctx; HBM TB/s vs peak"
HEADLINE = "decode_1m_b1_heavy"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "full_decode_split_decode_1m_pmc.md")
KERNEL_SOURCES = [os.path.join(ROOT, "kv_reuse_amd", "csrc", f)
                  for f in ("full_decode.hip", "hs2_internal.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the full-layer kernel from the committed rocprofv3
    counter summary, if it was taken on this workload and this kernel source."""
    try:
        txt = open(TRAFFIC_SUMMARY, encoding="utf-8").read()
    except OSError:
        return None
    m = re.search(r"traffic_record: workload=(\S+) source=(\S+) fetch_bytes=(\d+) "
                  r"write_bytes=(\d+)", txt)
    if not m or m.group(1) != workload or m.group(2) != kernel_source_hash():
        return None
    return int(m.group(3)) + int(m.group(4))


def algorithmic_full_layer_bytes(w) -> int:
    """K + V once, Q in, O out, and 4 bytes of importance per (row, key)."""
    rows = w.batch * w.n_q_tokens * w.n_kv_heads
    kv = 2 * w.batch * w.n_kv_heads * w.ctx_len * w.head_dim * 2
    qo = 2 * w.batch * w.n_q_tokens * w.n_q_heads * w.head_dim * 2
    return kv + qo + 4 * rows * w.ctx_len


def algorithmic_full_layer_flops(w) -> int:
    """Causal attention: every query head attends to keys 0..P_t, 2*D flops for
    the logit and 2*D for the value sum per key."""
    pos = w.ctx_len - w.n_q_tokens + np.arange(w.n_q_tokens, dtype=np.int64)
    return int(w.batch * w.n_q_heads * 4 * w.head_dim * int((pos + 1).sum()))


def host_info() -> dict:
    """The host the CPU baseline runs on: usable cores, CPU model, BLAS threads."""
    from threadpoolctl import threadpool_info
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return {"cores": len(os.sched_getaffinity(0)), "cpu_model": model, "blas_threads": int(blas)}


def cpu_baseline(w, x, budget_s: float = 20.0, block: int = 0):
    """Time the CPU oracle (as it stands) on whole (batch, query token, KV head)
    rows of the same inputs until the budget is used; scale to query tokens per
    second."""
    import oracle.hs2_oracle as orc
    rows = [(b, t, g) for t in range(w.n_q_tokens) for b in range(w.batch)
            for g in range(w.n_kv_heads)]
    if w.n_q_tokens > 1:
        # a spread of query tokens across the chunk (all KV heads of each)
        stride = max(1, w.n_q_tokens // 64)
        rows = [(b, t, g) for t in range(0, w.n_q_tokens, stride) for b in range(w.batch)
                for g in range(w.n_kv_heads)]
    done = 0
    t0 = time.perf_counter()
    for r in rows:
        orc.cross_decoder_step(x["q_full"], x["k"], x["v"], x["q_sparse"], top_k=w.top_k,
                               window=w.window, scale=w.scale, rows=[r], keep_scores=False,
                               block=block)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    tokens = done / w.n_kv_heads          # one query token spans all KV heads of its batch row
    info = host_info()
    # the oracle's dense products run on the BLAS threads, the rest on one
    used = min(info["cores"], info["blas_threads"])
    return {"value": tokens / dt, "unit": "query tokens/s", "cores": used,
            "kind": "oracle", "host_cores": info["cores"], "blas_threads": info["blas_threads"],
            "cpu_model": info["cpu_model"],
            "sample": f"{done} (batch, query token, KV head) rows of {w.name}: full float64 "
                      f"attention over all {w.ctx_len} keys, group-max importance, full sort, "
                      f"{w.n_sparse_layers} sparse layers; {dt:.2f} s on {info['blas_threads']} "
                      f"BLAS threads of {info['cores']} usable cores"}


# KV Bridging workloads (the projection of Self-Decoder hidden states into the
# cache): (batch, new tokens per batch entry, d_model, KV heads, cache capacity)
BRIDGE_WORKLOADS = {
    "bridge_prompt_128k": (1, 131072, 4096, 4, 131072),   # a whole 128K prompt
    "bridge_append_b16": (16, 1, 4096, 4, 32768),         # decode-time append, batch 16
}


def bench_bridge(args, name):
    """Time hs2_kv_bridge alone; one JSON line like the main benchmark's."""
    import torch
    from kv_reuse_amd import hs2
    from kv_reuse_amd import workloads as wl

    B, n, dm, Hkv, cap = BRIDGE_WORKLOADS[name]
    D = 128
    log(f"[bench] generating {name}")
    hidden, w_kv = wl.bridge_inputs_device(B, n, dm, Hkv)
    k = torch.empty((B, Hkv, cap, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    pos0 = cap - n
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        hs2.kv_bridge(hidden, w_kv, k, v, pos0)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        hs2.kv_bridge(hidden, w_kv, k, v, pos0)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / args.steps
    M = B * n
    if M > 64:
        flops = 2 * M * dm * 2 * Hkv * D
        ach = flops / (ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": None, "kernel": "bridge_gemm_kernel", "algorithmic_flops": flops,
                    "kernel_ms": round(ms, 5)}
    else:
        nbytes = 2 * Hkv * D * dm * 2 + M * dm * 2 + 2 * M * Hkv * D * 2
        ach = nbytes / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                    "kernel": "bridge_small_kernel", "algorithmic_bytes": nbytes,
                    "kernel_ms": round(ms, 5)}
    rec = {"metric": "tokens/s projected into the Cross-Decoder KV cache (KV Bridging)",
           "value": round(M / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": name, "batch": B, "n_tokens": n, "d_model": dm,
                      "n_kv_heads": Hkv, "head_dim": D, "kv_capacity": cap},
           "roofline": roofline, "wall_s_timed": round(wall, 4), "cpu_baseline": None}
    if not args.no_cpu_baseline:
        import oracle.hs2_oracle as orc
        nt = min(M, 2048)
        hb = hidden.reshape(M, dm)[:nt].view(torch.int16).cpu().numpy().view(np.uint16)
        wb = w_kv.view(torch.int16).cpu().numpy().view(np.uint16)
        reps = 0
        t1 = time.perf_counter()
        while reps == 0 or time.perf_counter() - t1 < 2.0:
            orc.kv_bridge(hb.reshape(1, nt, dm), wb)
            reps += 1
        dt = time.perf_counter() - t1
        info = host_info()
        # numpy's einsum contracts in its own single-threaded loops
        rec["cpu_baseline"] = {"value": round(reps * nt / dt, 3), "unit": "tokens/s",
                               "cores": 1, "kind": "oracle", "host_cores": info["cores"],
                               "cpu_model": info["cpu_model"],
                               "sample": f"{reps} x {nt} tokens of {name}: float64 projection "
                                         f"into K and V of {Hkv} heads; {dt:.2f} s"}
    print(json.dumps(rec), flush=True)


# ---------------------------------------------------------------- timing helpers

def timed_steps(step, steps: int, warmup: int):
    """Warm up, then time `steps` steps back to back between two events on the
    current stream (bracketed by synchronisations), then each step on its own
    for the median and the minimum.  Returns (mean ms, median ms, min ms, wall s)."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean = e0.elapsed_time(e1) / steps
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in per:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in per)
    return mean, each[len(each) // 2], each[0], wall


def cold_steps(step, steps: int, scratch):
    """Median ms of a step whose inputs are not in any cache: a 1 GiB scratch
    buffer is written before each step (outside the timed events)."""
    import torch
    stream = torch.cuda.current_stream()
    per = []
    for i in range(steps):
        scratch.fill_(i & 0xFF)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        step()
        b.record(stream)
        per.append((a, b))
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in per)
    return each[len(each) // 2]


def graph_steps(step, iters: int, warmup: int = 3):
    """The step captured once in a HIP graph; ms per replay over `iters` replays."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def stream_ceiling(nbytes: int = 2 << 30, iters: int = 10) -> dict:
    """The device's measured streaming-read bandwidth (non-temporal 16-byte loads
    over a buffer larger than every cache)."""
    import torch
    from kv_reuse_amd import hs2
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    hs2.stream_read_ms(buf, 2)
    ms = hs2.stream_read_ms(buf, iters)
    del buf
    return {"gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes, "passes": iters,
            "kind": "non-temporal streaming read (hs2_stream_read_ms)"}


def roofline_of(w, kernel_ms: float, stream_gbs=None) -> dict:
    if w.n_q_tokens == 1:
        algo = algorithmic_full_layer_bytes(w)
        achieved = algo / (kernel_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
             "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
             "traffic": measured_traffic(w.name), "kernel": "full_decode_split_kernel",
             "algorithmic_bytes": algo, "kernel_ms": round(kernel_ms, 5)}
        if stream_gbs:
            r["measured_stream_gbs"] = stream_gbs
            r["frac_of_measured_stream"] = round(achieved / stream_gbs, 4)
        return r
    flops = algorithmic_full_layer_flops(w)
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    return {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None, "kernel": "full_prefill_kernel", "algorithmic_flops": flops,
            "kernel_ms": round(kernel_ms, 5)}


def measure_workload(w, args, *, select_block=0, swa=False, graph=False, graph_iters=0,
                     cold=False, keep_inputs=False, stream_gbs=None):
    """One workload's step: timings, per-phase times and roofline (a dict), and
    its host inputs when keep_inputs (for the CPU baseline)."""
    import dataclasses
    import torch
    from kv_reuse_amd import hs2
    from kv_reuse_amd import workloads as wl

    log(f"[bench] {w.name}: generating")
    x = wl.generate(w)
    s = hs2.shape_of(w)
    if select_block:
        s = dataclasses.replace(s, select_block=select_block)
    B, T, Hq, Hkv, D, L = (w.batch, w.n_q_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim,
                           w.n_sparse_layers)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, qs = dev(x["q_full"]), dev(x["k"]), dev(x["v"]), dev(x["q_sparse"])
    out = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    outs = torch.empty((L, B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, T, Hkv, s.cap), dtype=torch.int32, device="cuda")
    nsel = torch.empty((B, T, Hkv), dtype=torch.int32, device="cuda")
    ws = hs2.alloc_workspace(s, L)
    torch.cuda.synchronize()
    if swa:
        Lc = hs2.local_rows(s)
        kl_b, vl_b = wl.swa_local_cache(L, B, Hkv, Lc)
        k_loc, v_loc = dev(kl_b), dev(vl_b)

        def step():
            hs2.cross_decoder_step(s, q, None, k, v, out, None, idx, nsel, ws=ws)
            hs2.sparse_attn_swa(s, qs, k, v, idx, nsel, k_loc, v_loc, outs, ws=ws)
    else:
        def step():
            hs2.cross_decoder_step(s, q, qs, k, v, out, outs, idx, nsel, ws=ws)

    log(f"[bench] {w.name}: timing {args.steps} steps")
    if graph:
        gms = graph_steps(step, max(args.steps, 3))
        mean = med = mn = gms
        wall = None
    else:
        mean, med, mn, wall = timed_steps(step, args.steps, args.warmup)
    rec = {"ms_per_step": round(mean, 5), "ms_per_step_median": round(med, 5),
           "ms_per_step_min": round(mn, 5), "tokens_per_s": round(B * T / (mean * 1e-3), 2)}
    if wall is not None:
        rec["wall_s_timed"] = round(wall, 4)
    if graph_iters:
        rec["graph_ms_per_step"] = round(graph_steps(step, graph_iters), 5)
        rec["graph_replays"] = graph_iters
    if cold:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        rec["cold_ms_per_step_median"] = round(cold_steps(step, max(args.steps, 5), scratch), 5)
        del scratch
    phases = hs2.cross_decoder_step_timed(s, q, qs, k, v, out, outs, idx, nsel, ws,
                                          max(args.steps, 10))
    full_ms = phases[0] + phases[1]
    rec["phases_ms"] = {"full_split": round(phases[0], 5), "full_combine": round(phases[1], 5),
                        "select": round(phases[2], 5), "sparse": round(phases[3], 5)}
    rec["after_full_frac"] = round((phases[2] + phases[3]) / full_ms, 4) if full_ms > 0 else None
    rec["sparse_frac"] = round(phases[3] / full_ms, 4) if full_ms > 0 else None
    rec["roofline"] = roofline_of(w, phases[0], stream_gbs)
    # a diagnostic of the selection's output (not a pass criterion): the share
    # of the planted needles among older keys that the last step kept
    torch.cuda.synchronize()
    rec["needle_recall"] = wl.needle_recall(w, x["needles"], idx.cpu().numpy(), nsel.cpu().numpy())
    del q, k, v, qs, out, outs, idx, nsel, ws
    torch.cuda.empty_cache()
    return rec, (x if keep_inputs else None)


def config_of(w, select_block=0, swa=False, graph=False):
    return {"workload": w.name, "batch": w.batch, "n_q_tokens": w.n_q_tokens,
            "ctx_len": w.ctx_len, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
            "head_dim": w.head_dim, "top_k": w.top_k, "window": w.window,
            "n_sparse_layers": w.n_sparse_layers,
            "selection": f"block_{select_block}" if select_block else "token",
            "sparse_layers": "separate_window_branch" if swa else "shared",
            "launch": "hip_graph" if graph else "stream"}


def early_exit(steps: int = 5, warmup: int = 2, n_groups: int = 4, n_sparse: int = 5) -> dict:
    """Prefill of a 4096-token chunk at the end of a 128K context, attention
    layers only: the early exit (the Self-Decoder's full layer + KV Bridging
    into every Cross-Decoder group's cache) against the full prefill (the same
    plus every group's full layer, selection and sparse layers)."""
    import torch
    from kv_reuse_amd import prefill_pipeline as pp

    log("[bench] prefill early exit: building")
    t = pp.synthetic(n_groups=n_groups, n_sparse=n_sparse)
    p = pp.PrefillPipeline(t)
    torch.cuda.synchronize()
    res = {}
    for name, fn in (("self_decoder_full_layer", p.self_decoder), ("kv_bridging", p.bridge),
                     ("cross_decoder", p.cross_decoder), ("early_exit", p.early_exit),
                     ("full_prefill", p.full)):
        mean, med, _, _ = timed_steps(fn, steps, warmup)
        res[name + "_ms"] = round(mean, 4)
    del p, t
    torch.cuda.empty_cache()
    res.update({
        "chunk_tokens": 4096, "ctx_len": 131072, "n_q_heads": 32, "n_kv_heads": 4, "d_model": 4096,
        "cross_decoder_groups": n_groups, "sparse_layers_per_group": n_sparse,
        "early_exit_over_full": round(res["early_exit_ms"] / res["full_prefill_ms"], 4),
        "early_exit_tokens_per_s": round(4096 / (res["early_exit_ms"] * 1e-3), 1),
        "full_prefill_tokens_per_s": round(4096 / (res["full_prefill_ms"] * 1e-3), 1),
        "note": "attention layers only (no MLP/MoE, no sliding-window layers of the "
                "Self-Decoder); the pages' whole-model analytic estimate (prefill FLOPs "
                "about 1/5 of the previous design at 1M tokens) is context, not a target"})
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help="one workload alone (default: the headline line with every workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="the headline workload only (no other workloads, stream ceiling or "
                         "early exit): for profiling runs")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays")
    ap.add_argument("--swa-branch", action="store_true",
                    help="time the previous generation's sparse layers instead: a separate "
                         "sliding-window branch over each layer's own local cache plus the "
                         "selected older tokens")
    ap.add_argument("--select-block", type=int, default=0,
                    help="time the block-level selection variant with this block size "
                         "(0: the token-level selection of the method)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB three times (the "
                         "reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU form in this build "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    from kv_reuse_amd import workloads as wl
    import kv_reuse_amd.hs2  # noqa: F401  (fails loudly when the library is missing)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.workload in BRIDGE_WORKLOADS:
        bench_bridge(args, args.workload)
        return
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {n} bytes read + {n} bytes written, 3 launches")
        del src, dst
    if args.workload == "prefill_early_exit":
        ee = early_exit()
        rec = {"metric": "query tokens/s of a 4096-token prefill chunk over 128K, early exit "
                         "vs full Cross-Decoder prefill (attention layers)",
               "value": ee["early_exit_tokens_per_s"], "unit": "query tokens/s", "n_gpus": 1,
               "steps": 5, "warmup": 2, "ms_per_step": ee["early_exit_ms"],
               "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
               "dtype": "bf16", "data": "synthetic",
               "config": {"workload": "prefill_early_exit"}, "early_exit": ee,
               "roofline": None, "cpu_baseline": None}
        print(json.dumps(rec), flush=True)
        return

    name = args.workload or HEADLINE
    w = wl.WORKLOADS[name]
    headline = args.workload is None
    extras = headline and not args.no_extras and not (args.graph or args.swa_branch
                                                      or args.select_block)
    stream = stream_ceiling() if extras else None
    stream_gbs = stream["gbs"] if stream else None
    rec_w, x = measure_workload(w, args, select_block=args.select_block, swa=args.swa_branch,
                                graph=args.graph, keep_inputs=not args.no_cpu_baseline,
                                stream_gbs=stream_gbs)
    rec = {
        "metric": METRIC if name == HEADLINE else
        f"query tokens/s, full+sparse Cross-Decoder attn, {name}",
        "value": rec_w["tokens_per_s"],
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec_w["ms_per_step"],
        "ms_per_step_median": rec_w["ms_per_step_median"],
        "ms_per_step_min": rec_w["ms_per_step_min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config_of(w, args.select_block, args.swa_branch, args.graph),
        "roofline": rec_w["roofline"],
        "phases_ms": rec_w["phases_ms"],
        "after_full_frac": rec_w["after_full_frac"],
        "sparse_frac": rec_w["sparse_frac"],
        "needle_recall": rec_w["needle_recall"],
        "wall_s_timed": rec_w.get("wall_s_timed"),
    }
    if stream:
        rec["stream_read"] = stream
    if not args.no_cpu_baseline and not args.swa_branch:
        log("[bench] cpu baseline (oracle)")
        rec["cpu_baseline"] = cpu_baseline(w, x, budget_s=20.0, block=args.select_block)
    else:
        rec["cpu_baseline"] = None
    del x
    if extras:
        workloads = {name: {k2: v2 for k2, v2 in rec_w.items()}}
        for other in ("decode_2k_b4", "decode_32k_b16", "decode_256k_b4_drift",
                      "prefill_4k_over_128k"):
            wo = wl.WORKLOADS[other]
            opts = {}
            if other == "decode_2k_b4":
                opts = {"graph_iters": 1000, "cold": True}
            elif other == "prefill_4k_over_128k":
                opts = {"cold": True}
            r, xo = measure_workload(wo, args, keep_inputs=not args.no_cpu_baseline,
                                     stream_gbs=stream_gbs, **opts)
            if xo is not None:
                log(f"[bench] {other}: cpu baseline (oracle)")
                r["cpu_baseline"] = cpu_baseline(wo, xo, budget_s=5.0)
            workloads[other] = r
            del xo
        rec["workloads"] = workloads
        rec["early_exit"] = early_exit()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
