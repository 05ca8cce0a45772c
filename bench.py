"""Benchmark of the fused attention-KL hot path on one MI355X.

One step = the whole path on one batch of the 64K causal workload (32 heads,
N_Q = N_K = 65536, head_dim 128, bf16, student near teacher, seed 2):
forward (KL, LSE1, LSE2) + backward Setting 1 (dQ2, dK2) + backward Setting 2
(dQ1, dK1), each through the C ABI on the current stream, inputs resident in
HBM before the timed region starts.

value = algorithmic TFLOP per step / seconds per step, where the algorithmic
work counts only unmasked (query, key) pairs: 4 d flop each in the forward and
8 d in each backward setting (recomputation once; the separate path's second
recomputation is not counted).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "fwd/bwd TFLOP/s + ms, 32 heads d=128 bf16 causal N=64K; % MFMA peak"


def upload(w: W.Workload, threads: int):
    """Seeded inputs of workload w, generated per head on the host, into HBM."""
    import torch
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = [torch.empty(w.heads, n, w.head_dim, dtype=tdt, device="cuda") for n in (w.n_q, w.n_k, w.n_q, w.n_k)]

    def one(h):
        return h, [torch.from_numpy(a).to(tdt) for a in W.head_inputs(w, h)]

    with ThreadPoolExecutor(threads) as ex:
        for h, parts in ex.map(one, range(w.heads)):
            for t, a in zip(out, parts):
                t[h].copy_(a, non_blocking=False)
    torch.cuda.synchronize()
    return out


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "streaming_kl_divergence_amd", "csrc"))):
        h.update(open(os.path.join(ROOT, "streaming_kl_divergence_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel sources changed since it was taken."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    e = d.get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def cpu_baseline():
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    head 0 of the 64K causal workload restricted to its first 16384 queries and
    keys (causal rows 0..16383 see only keys 0..16383, so this is the top-left
    block of the real problem), forward + Setting 1 + Setting 2 backward."""
    import oracle
    w = W.WORKLOADS["causal64k"]
    n = 16384
    sub = w.replace(n_q=n, n_k=n, heads=1)
    q1, k1, q2, k2 = W.head_inputs(sub, 0)   # prefix rows of head 0's draws
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.forward_head(q1, k1, q2, k2, w.scale, True)
    oracle.backward_head(1, q1, k1, q2, k2, w.scale, True)
    oracle.backward_head(2, q1, k1, q2, k2, w.scale, True)
    dt = time.perf_counter() - t0
    flop = 20 * w.head_dim * sub.elements()
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"head 0 of causal64k, first {n} queries x {n} keys (causal), fwd + bwd Setting 1 + "
                      f"Setting 2, fp64 numpy/BLAS; {dt:.1f} s for {flop / 1e12:.3f} TFLOP"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="causal64k")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(heads would shard across GPUs with no exchange; see DESIGN.md).", file=sys.stderr)
        sys.exit(1)

    import torch
    import streaming_kl_divergence_amd as skl

    w = W.WORKLOADS[args.workload]
    threads = min(16, os.cpu_count() or 1)
    t_up = time.perf_counter()
    q1, k1, q2, k2 = upload(w, threads)
    t_up = time.perf_counter() - t_up
    scale, causal = w.scale, w.causal
    E = w.elements()
    d = w.head_dim
    flop_fwd = 4 * d * E
    flop_bwd = 8 * d * E
    flop_step = flop_fwd + 2 * flop_bwd
    stream = torch.cuda.current_stream()
    path = skl.bwd_select(w.n_q, w.n_k, w.heads, d, causal)
    # every call below launches one kernel, so the events around it time that kernel
    if path == "separate":
        calls = [("fwd_kernel", 4), ("bwd_kv_kernel set1", 6), ("bwd_q_kernel set1", 6),
                 ("bwd_kv_kernel set2", 6), ("bwd_q_kernel set2", 6)]
    else:
        calls = [("fwd_kernel", 4), ("bwd_kv_kernel fused set1", 8), ("bwd_kv_kernel fused set2", 8)]
    dq = torch.empty(w.heads, w.n_q, d, device="cuda", dtype=torch.float32)
    dk = torch.empty(w.heads, w.n_k, d, device="cuda", dtype=torch.float32)

    def step(ev=None):
        i = 0

        def mark():
            nonlocal i
            if ev:
                ev[i].record(stream)
            i += 1
        mark()
        kl, l1, l2 = skl.fwd(q1, k1, q2, k2, scale, causal)
        mark()
        for setting in (1, 2):
            kw = dict(kl=kl) if setting == 2 else {}
            if path == "separate":
                skl.bwd(setting, q1, k1, q2, k2, scale, causal, l1, l2, path="dk_only", dk=dk, **kw)
                mark()
                skl.bwd(setting, q1, k1, q2, k2, scale, causal, l1, l2, path="dq_only", dq=dq, **kw)
                mark()
            else:
                skl.bwd(setting, q1, k1, q2, k2, scale, causal, l1, l2, path=path, dq=dq, dk=dk, **kw)
                mark()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    n_ev = len(calls) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(len(calls))] for e in evs])  # [steps, calls]
    step_ms = np.array([e[0].elapsed_time(e[-1]) for e in evs])
    ms = float(np.mean(step_ms))
    value = flop_step / (ms * 1e-3) / 1e12

    mean_call = per_call.mean(0)
    parts = {}
    for (name, k), t in zip(calls, mean_call):
        parts[name] = {"ms": round(float(t), 3), "tflops": round(k * d * E / (t * 1e-3) / 1e12, 1),
                       "work": f"{k}*d flop per unmasked pair"}
    fwd_ms_ = float(mean_call[0])
    bwd1_ms = float(mean_call[1:1 + (len(calls) - 1) // 2].sum())
    bwd2_ms = float(mean_call[1 + (len(calls) - 1) // 2:].sum())
    parts["fwd_ms"] = round(fwd_ms_, 3)
    parts["bwd_set1_ms"] = round(bwd1_ms, 3)
    parts["bwd_set2_ms"] = round(bwd2_ms, 3)
    parts["fwd_tflops"] = round(flop_fwd / (fwd_ms_ * 1e-3) / 1e12, 1)
    parts["bwd_set1_tflops"] = round(flop_bwd / (bwd1_ms * 1e-3) / 1e12, 1)
    parts["bwd_set2_tflops"] = round(flop_bwd / (bwd2_ms * 1e-3) / 1e12, 1)
    parts["pct_mfma_peak_step"] = round(100 * value / PEAK_BF16_TFLOPS, 2)
    parts["wall_s_timed"] = round(wall, 3)
    parts["upload_s"] = round(t_up, 1)

    # dominant kernel: the single launch with the largest mean duration
    j = int(np.argmax(mean_call))
    kname, kflop = calls[j]
    achieved = kflop * d * E / (mean_call[j] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(float(achieved), 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(float(achieved) / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(kname),
                "avg_launch_ms": round(float(mean_call[j]), 3),
                "work_per_launch": f"{kflop}*d flop x {E} unmasked pairs = {kflop * d * E / 1e12:.3f} TFLOP"}
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.heads} heads, N_Q=N_K={w.n_q}, head_dim={d}, bf16, causal, "
                               "correlated student; step = fwd + bwd Setting 1 + bwd Setting 2",
                   "heads": w.heads, "n_q": w.n_q, "n_k": w.n_k, "head_dim": d, "causal": causal,
                   "bwd_path": path},
        "parts": parts,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
