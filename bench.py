"""Benchmark: one Cross-Decoder group step (full attention + importance, token
top-k with the forced window, N KV-reusing sparse layers) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Prints ONE JSON line.  The default workload is decode at 1M context (batch 1,
32 query / 4 KV heads, head dim 128, 8 sparse layers, top-1024 + recent 128).
`value` is query tokens per second of the whole step with inputs resident in
HBM; `roofline` rates the dominant kernel (the full layer's split-context
stream) by its algorithmic bytes (K + V + Q + O + 4 bytes of importance per key
row) over its own average duration, timed with HIP events on the stream it runs
on; `cpu_baseline` is the float64 CPU oracle on a bounded sample of the same
workload.
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


def cpu_baseline(w, x, budget_s: float = 20.0, block: int = 0):
    """Time the CPU oracle (as it stands) on whole (batch, query token, KV head)
    rows of the same inputs until the budget is used; scale to query tokens per
    second."""
    from threadpoolctl import threadpool_info
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
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    return {"value": tokens / dt, "unit": "query tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{done} (batch, query token, KV head) rows of {w.name}: full float64 "
                      f"attention over all {w.ctx_len} keys, group-max importance, full sort, "
                      f"{w.n_sparse_layers} sparse layers; {dt:.2f} s"}


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
        # numpy's einsum contracts in its own single-threaded loops
        rec["cpu_baseline"] = {"value": round(reps * nt / dt, 3), "unit": "tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"{reps} x {nt} tokens of {name}: float64 projection "
                                         f"into K and V of {Hkv} heads; {dt:.2f} s"}
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_1m_b1_heavy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays (for the small, "
                         "launch-bound workloads)")
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
    from kv_reuse_amd import hs2
    from kv_reuse_amd import workloads as wl

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
    w = wl.WORKLOADS[args.workload]
    log(f"[bench] generating {w.name}")
    x = wl.generate(w)
    s = hs2.shape_of(w)
    if args.select_block:
        import dataclasses
        s = dataclasses.replace(s, select_block=args.select_block)
    B, T, Hq, Hkv, D, S, L = (w.batch, w.n_q_tokens, w.n_q_heads, w.n_kv_heads, w.head_dim,
                              w.ctx_len, w.n_sparse_layers)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, qs = dev(x["q_full"]), dev(x["k"]), dev(x["v"]), dev(x["q_sparse"])
    out = torch.empty((B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    outs = torch.empty((L, B, T, Hq, D), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((B, T, Hkv, s.cap), dtype=torch.int32, device="cuda")
    nsel = torch.empty((B, T, Hkv), dtype=torch.int32, device="cuda")
    ws = hs2.alloc_workspace(s, L)
    torch.cuda.synchronize()

    if args.swa_branch:
        Lc = hs2.local_rows(s)
        kl_b, vl_b = wl.swa_local_cache(L, B, Hkv, Lc)
        k_loc, v_loc = dev(kl_b), dev(vl_b)

        def step():
            hs2.cross_decoder_step(s, q, None, k, v, out, None, idx, nsel, ws=ws)
            hs2.sparse_attn_swa(s, qs, k, v, idx, nsel, k_loc, v_loc, outs, ws=ws)
    else:
        def step():
            hs2.cross_decoder_step(s, q, qs, k, v, out, outs, idx, nsel, ws=ws)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.graph:
        # the library only enqueues kernels: the whole step captures into one graph
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

        def step():
            graph.replay()

        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    # each step on its own, for the median and the minimum
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in per:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    each = sorted(a.elapsed_time(b) for a, b in per)
    tokens_per_s = B * T / (ms_step / 1e3)

    log("[bench] per-phase timing")
    phases = hs2.cross_decoder_step_timed(s, q, qs, k, v, out, outs, idx, nsel, ws,
                                          max(args.steps, 10))
    full_ms = phases[0]
    if w.n_q_tokens == 1:
        algo = algorithmic_full_layer_bytes(w)
        achieved = algo / (full_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": measured_traffic(w.name), "kernel": "full_decode_split_kernel",
                    "algorithmic_bytes": algo, "kernel_ms": round(full_ms, 5)}
    else:
        flops = algorithmic_full_layer_flops(w)
        achieved = flops / (full_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 1),
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                    "kernel": "full_prefill_kernel", "algorithmic_flops": flops,
                    "kernel_ms": round(full_ms, 5)}

    rec = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_median": round(each[len(each) // 2], 5),
        "ms_per_step_min": round(each[0], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_q_tokens": T, "ctx_len": S,
                   "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": D, "top_k": w.top_k,
                   "window": w.window, "n_sparse_layers": L,
                   "selection": (f"block_{args.select_block}" if args.select_block
                                 else "token"),
                   "sparse_layers": "separate_window_branch" if args.swa_branch else "shared",
                   "launch": "hip_graph" if args.graph else "stream"},
        "roofline": roofline,
        "phases_ms": {"full_split": round(phases[0], 5), "full_combine": round(phases[1], 5),
                      "select": round(phases[2], 5), "sparse": round(phases[3], 5)},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline and not args.swa_branch:
        log("[bench] cpu baseline (oracle)")
        rec["cpu_baseline"] = cpu_baseline(w, x, block=args.select_block)
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
