"""Benchmark of the fused attention-KL hot path on one MI355X.

One step = the whole path on one batch of the 64K causal workload (32 heads,
N_Q = N_K = 65536, head_dim 128, bf16, student near teacher, seed 2):
forward (KL, LSE1, LSE2) + backward Setting 1 (dQ2, dK2) + backward Setting 2
(dQ1, dK1), each through the C ABI on the current stream, inputs resident in
HBM before the timed region starts.  The two settings' gradients come from
one recomputation (streamkl_bwd_both: its dK kernel, then its dQ kernel);
--bwd-path separate times the two single-setting passes instead.

value = algorithmic TFLOP per step / seconds per step, where the algorithmic
work counts only unmasked (query, key) pairs: 4 d flop each in the forward and
8 d in each backward setting (the scores recomputed once, 4 d, and the dQ and
dK products, 4 d).  The both-settings kernels execute exactly this work (8 d
per pair each); the single-setting path executes 12 d per setting, its second
recomputation not counted.

The roofline object rates the dominant kernel against the published bf16
MFMA peak.  The measured ceilings on the same GPU (an MFMA loop with realistic
operands under the board power limit, the HBM read rate, fp32 atomics) come from
--calibrate and --power.  --gemm-ref adds a 16384^3 bf16 GEMM through torch.mm
(hipBLASLt) as platform context (parts.gemm_bf16_16384_tflops).

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--gemm-ref] [--no-decode] [--no-ceiling]
      the one-line benchmark of the 64K causal step (the default); parts.decode512k
      carries the 512K-key split-K decode's HBM read rate, timed in the same run;
      parts.mfma_ceiling the matrix cores' sustained rate on this GPU with the
      step kernels' operand pattern, and each kernel's executed rate as a
      fraction of it (a figure that does not depend on which board ran).
  python bench.py --configs
      one JSON line per workload (tiny fp32, 8K causal, 64K causal with both
      backward paths and the both-settings backward, 512K decode split-K vs
      single pass, 128K non-causal, 512 x 128K fused vs separate): median and
      min of timed runs per call.
  python bench.py --sweep crossover|splitk|context
      the ablations: fused vs separate backward over N_Q at N_K = 128K; split-K
      vs one pass (and several split counts) over small N_Q; and latency,
      TFLOP/s and device memory over context length 4K..512K.  One JSON line
      per point.
  python bench.py --copy-calibration ...
      also runs one plain 1 GiB device copy first, so that a rocprofv3 --pmc
      run sees FETCH_SIZE / WRITE_SIZE of a copy of known size.
  python bench.py --calibrate
      the calibration probes (libstreamkl_probes.so): bf16 MFMA loops at 1-3
      waves per SIMD with constant and realistic operands (with board watts),
      the v_exp_f32 issue rate and whether it overlaps FMAs, plain 8 GiB HBM
      reads (default and non-temporal) and fp32 atomic adds: the measured
      ceilings beside the published peaks.
  python -m streaming_kl_divergence_amd.build --rev REV
  python bench.py --ab LIB_A,LIB_B [--workload NAME] [--ab-calls fwd,dk_both,...]
      two builds of the library (the second, say, from an earlier revision)
      timed against each other in one process on the same inputs, launches
      alternating; medians, ratios and whether the outputs are bitwise equal.
  python bench.py --power
      board power (the GPU's hwmon sensor) while each kernel of the 64K
      causal step runs back to back, beside idle power and MFMA probes with
      realistic operands: ms, watts and joules per call.
  python bench.py --workload decode512k
      the decode line instead: the split-K forward for one query per head,
      rated in GB/s against the HBM peak.
  python bench.py --pmc-summary FETCH_DIR WRITE_DIR [--workload NAME]
      reads two rocprofv3 --pmc outputs (FETCH_SIZE, then WRITE_SIZE, both of a
      --copy-calibration run), scales each counter by what it reads for the
      1 GiB copy, and writes profiles/traffic.json (profiles/traffic_NAME.json
      for another workload: HBM bytes per launch per kernel, tagged with a hash
      of the device sources).
  python bench.py --sq-summary DIR [DIR ...]
      reads rocprofv3 --pmc outputs holding SQ counters and GRBM_GUI_ACTIVE
      and prints, per kernel, how busy the matrix cores, the vector ALU and
      the LDS were and the shader clock the kernel ran at (markdown table).
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
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 (matrix and vector)


def peak_tflops(dtype: str) -> float:
    """Published MI355X peak of the arithmetic a workload's inputs run on."""
    return PEAK_FP32_TFLOPS if dtype == "fp32" else PEAK_BF16_TFLOPS
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


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the attention-KL library's device code (its .hip sources and
    the headers beside them, comments and layout ignored).  Host-only files
    such as the C ABI's argument checks, and the calibration probes (a library
    of their own), do not change what a kernel moves."""
    from streaming_kl_divergence_amd.build import SOURCES
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "streaming_kl_divergence_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if (f.endswith(".hip") and f in SOURCES) or f.endswith(".hpp"):
            with open(os.path.join(csrc, f)) as fh:
                h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def traffic_path(workload: str = "causal64k") -> str:
    """The committed counter summary of a workload's bench run."""
    name = "traffic.json" if workload == "causal64k" else f"traffic_{workload}.json"
    return os.path.join(ROOT, "profiles", name)


def measured_traffic(kernel: str, workload: str = "causal64k"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel sources changed since it was taken."""
    p = traffic_path(workload)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


_KERNELS = "fwd_kernel|bwd_kv_kernel|bwd_q_kernel|bwd_kv_both_kernel|bwd_q_both_kernel|splitk_combine_kernel"


def kernel_label(symbol: str):
    """Benchmark label of a library kernel symbol, mangled or demangled (None
    for other kernels)."""
    import re
    m = re.match(r"_ZN3skl(\d+)(" + _KERNELS + r")(.*)$", symbol)
    if m:
        name, targs = m.group(2), m.group(3)
        st = re.search(r"Li\d+ELi(\d)ELb(\d)", targs)
        setting, flag = (st.group(1), st.group(2)) if st else ("?", "0")
    else:
        m = re.match(r"(?:void )?skl::(" + _KERNELS + r")(?:<([^>]*)>)?\(", symbol)
        if not m:
            return None
        name = m.group(1)
        targs = [a.strip() for a in (m.group(2) or "").split(",")]
        # single-setting kernels: <T, D, SETTING, FUSED or SPLIT, HAS_G>
        setting, flag = (targs[2], "1" if targs[3] == "true" else "0") if len(targs) >= 4 else ("?", "0")
    if name in ("fwd_kernel", "splitk_combine_kernel", "bwd_kv_both_kernel", "bwd_q_both_kernel"):
        return name
    fused = name == "bwd_kv_kernel" and flag == "1"
    return f"{name}{' fused' if fused else ''} set{setting}"


COPY_BYTES = 1 << 30


def pmc_summary(fetch_dir: str, write_dir: str, workload: str = "causal64k"):
    """HBM bytes per launch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by the ratio of the 1 GiB copy's true bytes to what the
    counter reads for it."""
    import csv
    import glob

    def per_kernel(d, counter):
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = {}
        with open(f[0]) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")))
                vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"]) * 1024.0
        out = {}
        for (name, _), v in vals.items():
            out.setdefault(name, []).append(v)
        return out

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy = [k for k in fetch if "copyBuffer" in k or "copy" in k.lower()]
    if not copy:
        raise SystemExit("no copy kernel in the counter run (use --copy-calibration)")
    ck = max(copy, key=lambda k: max(fetch[k]))
    f_factor = COPY_BYTES / max(fetch[ck])
    w_factor = COPY_BYTES / max(write[ck])
    h = kernel_source_hash()
    table = {"_calibration": {"copy_kernel": ck, "copy_bytes": COPY_BYTES, "fetch_factor": round(f_factor, 4),
                              "write_factor": round(w_factor, 4)}}
    for name, v in fetch.items():
        label = kernel_label(name)
        if label is None:
            continue
        fb = f_factor * float(np.mean(v))
        wb = w_factor * float(np.mean(write.get(name, [0.0])))
        table[label] = {"symbol": name, "dispatches": len(v), "fetch_bytes": round(fb), "write_bytes": round(wb),
                        "bytes_per_launch": round(fb + wb), "source_hash": h}
    path = traffic_path(workload)
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(json.dumps(table, indent=1, sort_keys=True))


SIMDS, CUS, XCDS = 1024, 256, 8


def sq_summary(dirs):
    """Pipe utilisation per kernel from SQ counters (one or more --pmc runs of
    the same program; the last dispatch of each kernel is used).  Cycles are
    shader-clock cycles: GRBM_GUI_ACTIVE summed over the XCDs, divided by
    their number, is the kernel's length in cycles; the clock is that over
    the dispatch's duration."""
    import csv
    import glob
    per = {}
    for d in dirs:
        f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not f:
            raise SystemExit(f"no counter_collection.csv under {d}")
        disp = {}
        with open(f[0]) as fh:
            for r in csv.DictReader(fh):
                label = kernel_label(r["Kernel_Name"])
                if label is None:
                    continue
                e = disp.setdefault(int(r["Dispatch_Id"]), {"label": label, "c": {}})
                e["c"][r["Counter_Name"]] = e["c"].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                e["ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for i in sorted(disp):
            e = disp[i]
            dst = per.setdefault(e["label"], {"c": {}, "ns": {}})
            dst["c"].update(e["c"])
            dst["ns"][d] = e["ns"]
    rows = ["| kernel | clock GHz | MFMA busy | VALU busy | MFMA+VALU co-issue | LDS busy | VALU instr / MFMA |",
            "|---|---|---|---|---|---|---|"]
    for label, e in per.items():
        c = e["c"]
        if "GRBM_GUI_ACTIVE" not in c:
            continue
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS

        def frac(name, scale=1.0, units=SIMDS):
            return f"{100 * c[name] * scale / units / cyc:.0f}%" if name in c else "-"

        ghz = cyc / (float(np.mean(list(e["ns"].values()))))
        ratio = f"{c['SQ_INSTS_VALU'] / c['SQ_INSTS_MFMA']:.2f}" if "SQ_INSTS_VALU" in c and c.get("SQ_INSTS_MFMA") else "-"
        rows.append(f"| {label} | {ghz:.2f} | {frac('SQ_VALU_MFMA_BUSY_CYCLES')} | "
                    f"{frac('SQ_ACTIVE_INST_VALU', 4.0)} | {frac('SQ_VALU_MFMA_COEXEC_CYCLES')} | "
                    f"{frac('SQ_LDS_IDX_ACTIVE', 1.0, CUS)} | {ratio} |")
    print("\n".join(rows))


def _timed(fn, stream, warmup: int, reps: int):
    """fn() enqueues work on stream; returns per-run ms from HIP events."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def _timed_batches(fn, stream, warmup: int, reps: int, rounds: int = 5):
    """fn() enqueues work on stream; `rounds` batches of `reps` back-to-back
    calls, each batch between two HIP events; the median over the batches of
    ms per call.  For short calls whose throughput is the figure: the host
    enqueues ahead of the GPU, so no host time falls between two calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(rounds):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b) / reps)
    return float(np.median(out))


def configs_mode():
    """One JSON line per workload: median / min ms of each call, algorithmic
    TFLOP/s (MFMA-bound calls) or GB/s (the HBM-bound decode)."""
    import torch
    import streaming_kl_divergence_amd as skl
    stream = torch.cuda.current_stream()
    threads = min(16, os.cpu_count() or 1)

    def line(w, rows, extra=None):
        out = {"workload": w.name, "heads": w.heads, "n_q": w.n_q, "n_k": w.n_k, "head_dim": w.head_dim,
               "dtype": w.dtype, "causal": w.causal, "elements": w.elements(), "calls": rows}
        if extra:
            out.update(extra)
        print(json.dumps(out), flush=True)

    cur = {"peak": PEAK_BF16_TFLOPS}   # the peak of the workload being timed

    def entry(ms, flop=None, hbm=None):
        e = {"median_ms": round(float(np.median(ms)), 4), "min_ms": round(float(ms.min()), 4), "runs": len(ms)}
        if flop:
            peak = cur["peak"]
            tf = flop / (np.median(ms) * 1e-3) / 1e12
            e.update({"tflops": round(float(tf), 1), "pct_peak": round(100 * float(tf) / peak, 1)})
        if hbm:
            gbs = hbm / (np.median(ms) * 1e-3) / 1e9
            e.update({"gbs": round(float(gbs), 1), "pct_hbm": round(100 * float(gbs) / PEAK_HBM_GBS, 1)})
        return e

    def run(name, settings, paths=("auto",), reps=10, both=False, splitk=False):
        w = W.WORKLOADS[name]
        cur["peak"] = peak_tflops(w.dtype)
        q1, k1, q2, k2 = upload(w, threads)
        d, E = w.head_dim, w.elements()
        kl, l1, l2 = skl.fwd(q1, k1, q2, k2, w.scale, w.causal)
        rows = {"fwd": entry(_timed(lambda: skl.fwd(q1, k1, q2, k2, w.scale, w.causal), stream, 3, reps),
                             4 * d * E)}
        if splitk:
            # few query blocks: the split-K forward fills the chip
            auto = skl.splitk_auto(w.n_q, w.n_k, w.heads, d)
            rows[f"fwd splitk (auto {auto})"] = entry(
                _timed(lambda: skl.fwd_splitk(q1, k1, q2, k2, w.scale, w.causal), stream, 3, reps), 4 * d * E)
        dq = torch.empty(w.heads, w.n_q, d, device="cuda", dtype=torch.float32)
        dk = torch.empty(w.heads, w.n_k, d, device="cuda", dtype=torch.float32)
        for st in settings:
            kw = dict(kl=kl) if st == 2 else {}
            for path in paths:
                chosen = skl.bwd_select(w.n_q, w.n_k, w.heads, d, w.causal) if path == "auto" else path
                ms = _timed(lambda: skl.bwd(st, q1, k1, q2, k2, w.scale, w.causal, l1, l2, path=path,
                                            dq=dq, dk=dk, **kw), stream, 3, reps)
                rows[f"bwd set{st} {path}" + (f" ({chosen})" if path == "auto" else "")] = entry(ms, 8 * d * E)
        if both:
            outs = [torch.empty(w.heads, n, d, device="cuda", dtype=torch.float32) for n in (w.n_q, w.n_k, w.n_q, w.n_k)]
            ms = _timed(lambda: skl.bwd_both(q1, k1, q2, k2, w.scale, w.causal, l1, l2, kl, dq1=outs[0], dk1=outs[1],
                                             dq2=outs[2], dk2=outs[3]), stream, 3, reps)
            rows["bwd both settings"] = entry(ms, 16 * d * E)
            del outs
        line(w, rows)
        del q1, k1, q2, k2, dq, dk
        torch.cuda.empty_cache()

    run("tiny", (1, 2), both=True)
    run("causal8k", (1,))
    run("causal64k", (1, 2), paths=("auto", "fused", "separate"), reps=5, both=True)
    # decode: the same fused key loop with one split vs split-K
    w = W.WORKLOADS["decode512k"]
    q1, k1, q2, k2 = upload(w, threads)
    hbm = 2 * w.heads * w.n_k * w.head_dim * 2 + 2 * w.heads * w.n_q * w.head_dim * 2 + 3 * w.heads * w.n_q * 4
    auto = skl.splitk_auto(w.n_q, w.n_k, w.heads, w.head_dim)
    rows = {"single pass": entry(_timed(lambda: skl.fwd(q1, k1, q2, k2, w.scale, w.causal), stream, 3, 10),
                                 hbm=hbm)}
    for s_ in (1, auto):
        rows[f"splitk {s_}{' (auto)' if s_ == auto else ''}"] = entry(
            _timed(lambda: skl.fwd_splitk(q1, k1, q2, k2, w.scale, w.causal, num_splits=s_), stream, 3, 10),
            hbm=hbm)
    line(w, rows, {"hbm_bytes": hbm})
    del q1, k1, q2, k2
    torch.cuda.empty_cache()
    run("noncausal128k", (2,), reps=3)
    run("smallq128k", (2,), paths=("auto", "fused", "separate"), splitk=True)


def _rand_inputs(heads, n_q, n_k, d, seed=0, corr=True):
    """Sweep inputs drawn on the device (timing only; parity is covered by the tests)."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    q1 = torch.randn(heads, n_q, d, device="cuda", generator=g, dtype=torch.bfloat16)
    k1 = torch.randn(heads, n_k, d, device="cuda", generator=g, dtype=torch.bfloat16)
    q2 = torch.randn(heads, n_q, d, device="cuda", generator=g, dtype=torch.bfloat16)
    k2 = torch.randn(heads, n_k, d, device="cuda", generator=g, dtype=torch.bfloat16)
    if corr:
        q2 = (q1.float() + 0.3 * q2.float()).to(torch.bfloat16)
        k2 = (k1.float() + 0.3 * k2.float()).to(torch.bfloat16)
    return q1, k1, q2, k2


def sweep_mode(which: str):
    import torch
    import streaming_kl_divergence_amd as skl
    stream = torch.cuda.current_stream()
    H, d = 32, 128
    scale = d ** -0.5

    def emit(**kw):
        print(json.dumps({"sweep": which, **kw}), flush=True)

    def pairs(n_q, n_k, causal):
        if not causal:
            return H * n_q * n_k
        off = n_k - n_q
        return H * sum(min(n_k, i + off + 1) for i in range(n_q)) if n_q < 4096 else \
            H * (n_q * (n_q + 1) // 2 + n_q * off)

    if which == "crossover":
        # fused (one recompute, fp32 atomics into dQ) vs separate (dK and dQ
        # kernels, two recomputes), N_K = 128K, non-causal, both settings
        n_k = 131072
        for n_q in (64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384):
            q1, k1, q2, k2 = _rand_inputs(H, n_q, n_k, d)
            kl, l1, l2 = skl.fwd(q1, k1, q2, k2, scale, False)
            dq = torch.empty(H, n_q, d, device="cuda")
            dk = torch.empty(H, n_k, d, device="cuda")
            E = H * n_q * n_k
            row = {"n_q": n_q, "n_k": n_k, "heads": H, "dq_mib": H * n_q * d * 4 / 2 ** 20,
                   "selector": skl.bwd_select(n_q, n_k, H, d, False)}
            for st in (1, 2):
                kw = dict(kl=kl) if st == 2 else {}
                for path in ("fused", "separate"):
                    ms = np.median(_timed(lambda: skl.bwd(st, q1, k1, q2, k2, scale, False, l1, l2, path=path,
                                                          dq=dq, dk=dk, **kw), stream, 2, 5))
                    row[f"set{st}_{path}_ms"] = round(float(ms), 4)
                    row[f"set{st}_{path}_tflops"] = round(8 * d * E / (ms * 1e-3) / 1e12, 1)
                row[f"set{st}_fused_over_separate"] = round(row[f"set{st}_separate_ms"] / row[f"set{st}_fused_ms"], 3)
            emit(**row)
            del q1, k1, q2, k2, dq, dk
            torch.cuda.empty_cache()
    elif which == "splitk":
        # forward with few queries: one pass vs split-K (automatic and fixed counts)
        n_k = 524288
        q1, k1, q2, k2 = _rand_inputs(H, 256, n_k, d, corr=False)
        for n_q in (1, 4, 16, 64, 256):
            a = [t[:, :n_q].contiguous() if i % 2 == 0 else t for i, t in enumerate((q1, k1, q2, k2))]
            hbm = 2 * H * n_k * d * 2
            auto = skl.splitk_auto(n_q, n_k, H, d)
            row = {"n_q": n_q, "n_k": n_k, "heads": H, "auto_splits": auto}
            ms = np.median(_timed(lambda: skl.fwd(*a, scale, False), stream, 2, 5))
            row["one_pass_ms"] = round(float(ms), 4)
            for sp in sorted({1, 8, 32, 64, 128, 256, auto}):
                ms = np.median(_timed(lambda: skl.fwd_splitk(*a, scale, False, num_splits=sp), stream, 2, 5))
                row[f"splits_{sp}_ms"] = round(float(ms), 4)
            row["auto_gbs"] = round(hbm / (row[f"splits_{auto}_ms"] * 1e-3) / 1e9, 1)
            row["speedup_auto_over_one_pass"] = round(row["one_pass_ms"] / row[f"splits_{auto}_ms"], 2)
            emit(**row)
    elif which == "context":
        # latency, algorithmic TFLOP/s and the library's extra device memory
        # (saved state only: KL, LSE1, LSE2) over context length
        for causal in (True, False):
            for n in (4096, 16384, 65536, 131072, 262144, 524288):
                if not causal and n > 262144:
                    continue
                q1, k1, q2, k2 = _rand_inputs(H, n, n, d)
                E = pairs(n, n, causal)
                torch.cuda.synchronize()
                base = torch.cuda.memory_allocated()
                torch.cuda.reset_peak_memory_stats()
                kl, l1, l2 = skl.fwd(q1, k1, q2, k2, scale, causal)
                torch.cuda.synchronize()
                state = torch.cuda.max_memory_allocated() - base
                reps = 3 if n <= 65536 else 1
                row = {"n": n, "causal": causal, "heads": H, "pairs": E, "saved_state_bytes": int(state),
                       "materialised_p_bytes": 2 * E * 2}
                ms = np.median(_timed(lambda: skl.fwd(q1, k1, q2, k2, scale, causal), stream, 1, reps))
                row["fwd_ms"] = round(float(ms), 3)
                row["fwd_tflops"] = round(4 * d * E / (ms * 1e-3) / 1e12, 1)
                dq = torch.empty(H, n, d, device="cuda")
                dk = torch.empty(H, n, d, device="cuda")
                for st in (1, 2):
                    kw = dict(kl=kl) if st == 2 else {}
                    ms = np.median(_timed(lambda: skl.bwd(st, q1, k1, q2, k2, scale, causal, l1, l2, dq=dq, dk=dk,
                                                          **kw), stream, 1, reps))
                    row[f"bwd_set{st}_ms"] = round(float(ms), 3)
                    row[f"bwd_set{st}_tflops"] = round(8 * d * E / (ms * 1e-3) / 1e12, 1)
                # both settings from one recomputation (bf16 kernels)
                dq2 = torch.empty(H, n, d, device="cuda")
                dk2 = torch.empty(H, n, d, device="cuda")
                ms = np.median(_timed(lambda: skl.bwd_both(q1, k1, q2, k2, scale, causal, l1, l2, kl, dq1=dq, dk1=dk,
                                                           dq2=dq2, dk2=dk2), stream, 1, reps))
                row["bwd_both_ms"] = round(float(ms), 3)
                row["bwd_both_tflops"] = round(16 * d * E / (ms * 1e-3) / 1e12, 1)
                del dq2, dk2
                emit(**row)
                del q1, k1, q2, k2, dq, dk, kl, l1, l2
                torch.cuda.empty_cache()
    else:
        raise SystemExit(f"unknown sweep {which!r}")


class PowerSampler:
    """Board power from the GPU's hwmon sensor (power1_input, microwatts),
    sampled every 0.1 s in a thread while work runs; median over a window."""

    def __init__(self):
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input"))
        self.path = paths[0] if paths else None
        self.samples = []
        self._stop = False
        self._th = threading.Thread(target=self._run, daemon=True) if self.path else None
        if self._th:
            self._th.start()

    def _run(self):
        while not self._stop:
            try:
                with open(self.path) as f:
                    self.samples.append((time.time(), int(f.read().strip()) / 1e6))
            except (OSError, ValueError):
                pass
            time.sleep(0.1)

    def median(self, t0: float, t1: float):
        v = [w for t, w in self.samples if t0 <= t <= t1]
        return round(float(np.median(v)), 1) if v else None

    def stop(self):
        self._stop = True
        if self._th:
            self._th.join()


def _loop_for(fn, seconds: float):
    """Run fn() back to back for about `seconds`; (ms per call, window start, window end)."""
    import torch
    fn()
    torch.cuda.synchronize()
    t0 = time.time()
    n = 0
    while time.time() - t0 < seconds:
        fn()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    t1 = time.time()
    return (t1 - t0) / n * 1e3, t0 + 0.5, t1


def power_mode(seconds: float = 5.0):
    """Board power while each kernel of the 64K causal step runs back to back
    (forward, the both-settings dK and dQ kernels, and Setting 1's two
    kernels), beside idle power and the calibration probes' (pure MFMA with
    realistic operands from registers and from LDS, an exp + FMA vector mix).
    One JSON line per phase: ms per call, median watts, joules per call."""
    import torch
    import streaming_kl_divergence_amd as skl
    from streaming_kl_divergence_amd import _lib
    ps = PowerSampler()
    if ps.path is None:
        print(json.dumps({"power": "no hwmon power sensor readable"}), flush=True)
        return
    time.sleep(1.5)
    t = time.time()
    idle = ps.median(t - 1.2, t)
    print(json.dumps({"phase": "idle", "watts": idle}), flush=True)
    w = W.WORKLOADS["causal64k"]
    q1, k1, q2, k2 = upload(w, min(16, os.cpu_count() or 1))
    kl, l1, l2 = skl.fwd(q1, k1, q2, k2, w.scale, True)
    g = [torch.empty(w.heads, w.n_q, w.head_dim, device="cuda") for _ in range(4)]
    E = w.elements()
    d = w.head_dim
    phases = [
        ("fwd_kernel", 4, lambda: skl.fwd(q1, k1, q2, k2, w.scale, True)),
        ("bwd_kv_both_kernel", 8, lambda: skl.bwd_both(q1, k1, q2, k2, w.scale, True, l1, l2, kl, path="dk_only",
                                                       dk1=g[1], dk2=g[3])),
        ("bwd_q_both_kernel", 8, lambda: skl.bwd_both(q1, k1, q2, k2, w.scale, True, l1, l2, kl, path="dq_only",
                                                      dq1=g[0], dq2=g[2])),
        ("bwd_kv_kernel set1", 6, lambda: skl.bwd(1, q1, k1, q2, k2, w.scale, True, l1, l2, path="dk_only", dk=g[1])),
        ("bwd_q_kernel set1", 6, lambda: skl.bwd(1, q1, k1, q2, k2, w.scale, True, l1, l2, path="dq_only", dq=g[0])),
    ]
    for name, k, fn in phases:
        ms, a, b = _loop_for(fn, seconds)
        watts = ps.median(a, b)
        print(json.dumps({"phase": name, "ms": round(ms, 3), "executed_tflops": round(k * d * E / (ms * 1e-3) / 1e12, 1),
                          "watts": watts, "joules_per_call": round(watts * ms * 1e-3, 2) if watts else None,
                          "dynamic_joules_per_call": round((watts - idle) * ms * 1e-3, 2) if watts and idle else None}),
              flush=True)
        time.sleep(1.0)
    del q1, k1, q2, k2, g
    torch.cuda.empty_cache()
    P = _lib.probes()
    T = P.streamkl_probe_threads()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = torch.cuda.current_stream().cuda_stream
    src = torch.randn(3 * cus * T * 128, device="cuda").to(torch.bfloat16)   # 256 bytes per thread
    sink = torch.empty(3 * cus * T, device="cuda")
    # one workgroup per CU per wave-per-SIMD, all resident at once; ~10 ms calls
    for name, lds, wps in (("mfma_data_regs", 0, 1), ("mfma_data_regs", 0, 2), ("mfma_data_regs", 0, 3),
                           ("mfma_data_lds", 1, 1), ("mfma_data_lds", 1, 2)):
        wg, iters = wps * cus, 75000 // wps
        ms, a, b = _loop_for(lambda: P.streamkl_probe_mfma_data(src.data_ptr(), src.numel() * 2, lds, wps, wg, iters,
                                                                sink.data_ptr(), sink.numel(), s), seconds)
        tf = wg * 4 * iters * 8 * 32768 / (ms * 1e-3) / 1e12
        watts = ps.median(a, b)
        print(json.dumps({"phase": f"{name} {wps} wave(s)/SIMD", "ms": round(ms, 3), "executed_tflops": round(tf, 1),
                          "watts": watts,
                          "dynamic_pj_per_flop": round((watts - idle) / tf, 3) if watts and idle else None}),
              flush=True)
        time.sleep(1.0)
    ps.stop()


def ab_mode(libs: list[str], workload: str, calls: list[str] | None = None, rounds: int = 8, per: int = 5):
    """Two or more builds of libstreamkl.so (for instance one built with
    `python -m streaming_kl_divergence_amd.build --rev REV`) timed against each
    other in one process on the same inputs: for every call, `rounds` rounds in
    which each build runs one untimed and `per` timed launches (HIP events on
    the launching stream), the order of the builds alternating between rounds;
    the median per build, its ratio to the first build, and whether the outputs
    are bitwise equal (else their largest relative difference).  One JSON line
    per call.  Box-to-box differences cancel; on one box two builds of the same
    code have differed by up to a few percent, so a smaller difference is not a
    result."""
    import ctypes
    import torch
    from streaming_kl_divergence_amd import _lib
    w = W.WORKLOADS[workload]
    default = {"causal64k": ["fwd", "dk_both", "dq_both"], "decode512k": ["splitk"], "smallq128k": ["splitk", "dq2"]}
    calls = calls or default.get(workload, ["fwd"])
    loaded = []
    for path in libs:
        l = ctypes.CDLL(os.path.abspath(path), mode=ctypes.RTLD_LOCAL)
        for name, (res, args) in _lib._SIGS.items():
            f = getattr(l, name, None)
            if f is not None:
                f.restype, f.argtypes = res, args
        loaded.append(l)
    q1, k1, q2, k2 = upload(w, min(16, os.cpu_count() or 1))
    H, NQ, NK, d = w.heads, w.n_q, w.n_k, w.head_dim
    dt = _lib.BF16 if w.dtype == "bf16" else _lib.FP32
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    base = (q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), NQ, NK, H, d, int(w.causal), w.scale, dt)
    f32 = dict(device="cuda", dtype=torch.float32)
    state = [torch.empty(H, NQ, **f32) for _ in range(3)]            # KL, LSE1, LSE2 from the first build
    if loaded[0].streamkl_fwd(*base, *(t.data_ptr() for t in state), s) != 0:
        raise RuntimeError("forward failed")
    kl, l1, l2 = (t.data_ptr() for t in state)
    need = loaded[0].streamkl_workspace_bytes(0, NQ, NK, H, d, 0, 0)
    ws = torch.empty(max(16, need), device="cuda", dtype=torch.uint8)

    def outputs(call):
        if call in ("fwd", "splitk"):
            return [torch.empty(H, NQ, **f32) for _ in range(3)]
        n = NK if call.startswith("dk") else NQ
        return [torch.empty(H, n, d, **f32) for _ in range(2 if call.endswith("both") else 1)]

    def launcher(lib, call, out):
        p = [t.data_ptr() for t in out]
        if call == "fwd":
            return lambda: lib.streamkl_fwd(*base, *p, s)
        if call == "splitk":
            return lambda: lib.streamkl_fwd_splitk(*base, 0, *p, ws.data_ptr(), ws.numel(), s)
        path = _lib.BWD_DK_ONLY if call.startswith("dk") else _lib.BWD_DQ_ONLY
        if call == "dk_both":
            return lambda: lib.streamkl_bwd_both(*base, l1, l2, kl, None, None, p[0], None, p[1], path, s)
        if call == "dq_both":
            return lambda: lib.streamkl_bwd_both(*base, l1, l2, kl, None, p[0], None, p[1], None, path, s)
        g = p[0]
        if call in ("dk1", "dq1"):                        # Setting 1: gradients of Q2, K2
            dq, dk = (g, None) if call == "dq1" else (None, g)
            return lambda: lib.streamkl_bwd_set1(*base, l1, l2, None, dq, dk, path, None, 0, s)
        if call in ("dk2", "dq2"):                        # Setting 2: gradients of Q1, K1
            dq, dk = (g, None) if call == "dq2" else (None, g)
            return lambda: lib.streamkl_bwd_set2(*base, l1, l2, kl, None, dq, dk, path, None, 0, s)
        raise ValueError(f"unknown call {call!r} (fwd, splitk, dk_both, dq_both, dk1, dq1, dk2, dq2)")

    for call in calls:
        outs = [outputs(call) for _ in loaded]
        runs = [launcher(lib, call, o) for lib, o in zip(loaded, outs)]
        for r in runs:
            if r() != 0:
                raise RuntimeError(f"{call} failed")
        torch.cuda.synchronize()
        equal = all(torch.equal(a, b) for o in outs[1:] for a, b in zip(outs[0], o))
        rel = max(float((a - b).abs().max() / a.abs().max().clamp_min(1e-30)) for o in outs[1:]
                  for a, b in zip(outs[0], o)) if len(outs) > 1 else 0.0
        times = [[] for _ in loaded]
        for rnd in range(rounds):
            order = list(range(len(loaded)))
            for i in (order if rnd % 2 == 0 else order[::-1]):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                runs[i]()
                e0.record(stream)
                for _ in range(per):
                    runs[i]()
                e1.record(stream)
                torch.cuda.synchronize()
                times[i].append(e0.elapsed_time(e1) / per)
        med = [float(np.median(t)) for t in times]
        print(json.dumps({"ab": call, "workload": workload, "libs": libs, "median_ms": [round(m, 4) for m in med],
                          "ratio_vs_first": [round(m / med[0], 4) for m in med], "bitwise_equal": equal,
                          "max_rel_diff": rel, "rounds": rounds, "launches_per_round": per}), flush=True)
        del outs, runs
    del q1, k1, q2, k2, ws, state
    torch.cuda.empty_cache()


def calibrate_mode(reps: int = 5, mfma_seconds: float = 3.0):
    """The calibration probes (libstreamkl_probes.so): bf16 MFMA loops at 1 to
    3 waves per SIMD (sustained, with board watts), a v_exp_f32 stream, a plain
    8 GiB read and fp32 atomic adds into a 1 GiB and a 2 MiB buffer.  One JSON
    line; the other rates are medians of `reps` timed runs.  Cycle figures
    assume the nominal 2.4 GHz shader clock."""
    import torch
    from streaming_kl_divergence_amd import _lib
    P = _lib.probes()
    T = P.streamkl_probe_threads()
    stream = torch.cuda.current_stream()
    s = stream.cuda_stream
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    clk = 2.4e9

    def run(launch):
        def f():
            if launch() != 0:
                raise RuntimeError("probe launch failed")
        return float(np.median(_timed(f, stream, 2, reps)))

    out = {"probe": "calibration", "compute_units": cus, "nominal_clock_ghz": clk / 1e9}
    ps = PowerSampler()
    # Matrix cores, sustained (each probe runs back to back for `mfma_seconds`,
    # long enough for the board to settle at its power limit), at 1, 2 and 3
    # waves per SIMD: one workgroup per CU per wave-per-SIMD, all resident at
    # once, ~10 ms per call.  Constant operands, then realistic ones (random
    # bf16 changing on every MFMA) from registers, with A from LDS (one b128 read
    # per lane per MFMA) and with A from LDS through transposing reads.
    wg_max = 4 * cus
    sink = torch.empty(wg_max * T, device="cuda")
    src = torch.randn(wg_max * T * 128, device="cuda").to(torch.bfloat16)   # 256 bytes per thread
    best = 0.0
    # The reuse kinds repeat the register B chunk across consecutive MFMAs
    # (pairs, with A from registers or LDS; fours, registers): whether an
    # operand that stays put between instructions saves energy.
    modes = {"random_regs": 0, "random_lds": 1, "random_ldstr": 2, "random_lds_bpairs": 3, "random_regs_bpairs": 4,
             "random_regs_bquads": 5}
    for kind, per_trip, base_iters in (("const", 4, 150000), ("random_regs", 8, 75000), ("random_lds", 8, 75000),
                                       ("random_ldstr", 8, 75000), ("random_regs_bpairs", 8, 75000),
                                       ("random_regs_bquads", 8, 75000), ("random_lds_bpairs", 8, 75000)):
        for wps in (1, 2, 3):
            wg, iters = wps * cus, base_iters // wps
            if kind == "const":
                launch = lambda: P.streamkl_probe_mfma(wps, wg, iters, sink.data_ptr(), sink.numel(), s)
            else:
                lds = modes[kind]
                launch = lambda: P.streamkl_probe_mfma_data(src.data_ptr(), src.numel() * 2, lds, wps, wg, iters,
                                                            sink.data_ptr(), sink.numel(), s)
            if launch() != 0:
                raise RuntimeError("probe launch failed")
            ms, a, b = _loop_for(launch, mfma_seconds)
            tf = wg * 4 * iters * per_trip * 32768 / (ms * 1e-3) / 1e12
            print(f"calibrate: mfma {kind} at {wps} wave(s)/SIMD {tf:.1f} TFLOP/s", file=sys.stderr, flush=True)
            out[f"mfma_bf16_{kind}_w{wps}_tflops"] = round(tf, 1)
            out[f"mfma_bf16_{kind}_w{wps}_watts"] = ps.median(a, b)
            if kind != "const":
                best = max(best, tf)
            time.sleep(1.0)
    out["mfma_bf16_random_best_tflops"] = round(best, 1)
    out["mfma_bf16_random_best_frac_of_peak"] = round(best / PEAK_BF16_TFLOPS, 4)
    ps.stop()
    del src
    # v_exp_f32: 8 per lane per trip, 16 waves per CU
    wg, iters = 4 * cus, 20000
    ms = run(lambda: P.streamkl_probe_exp(wg, iters, sink.data_ptr(), sink.numel(), s))
    wave_insts = wg * 4 * iters * 8
    out["exp_wave_insts_per_s"] = wave_insts / (ms * 1e-3)
    out["exp_cycles_per_wave_inst_per_simd"] = round(4 * cus * clk * (ms * 1e-3) / wave_insts, 2)
    # exp beside FMA: two waves per SIMD, both exp, both FMA, or one of each
    # (equal instructions per wave); if the mixed run takes the mean of the two
    # pure runs the instructions take turns, if half the slower one they overlap
    mix_sink = torch.empty(cus * 512, device="cuda")
    mix = {}
    for name, mode in (("exp", 0), ("fma", 1), ("mixed", 2)):
        mix[name] = run(lambda: P.streamkl_probe_exp_fma(mode, cus, 100000, mix_sink.data_ptr(), mix_sink.numel(), s))
        out[f"exp_fma_{name}_ms"] = round(mix[name], 3)
    simd_insts = 2 * 100000 * 8                       # per SIMD: two waves x trips x 8
    out["fma_cycles_per_wave_inst_per_simd"] = round(clk * mix["fma"] * 1e-3 / simd_insts, 2)
    out["exp_fma_mixed_over_turns"] = round(mix["mixed"] / ((mix["exp"] + mix["fma"]) / 2), 3)
    out["exp_fma_mixed_over_overlap"] = round(mix["mixed"] / (max(mix["exp"], mix["fma"]) / 2), 3)
    del sink, mix_sink
    # HBM read: 8 GiB, 8 workgroups per CU
    nbytes = 8 << 30
    src = torch.empty(nbytes // 4, device="cuda", dtype=torch.float32).fill_(1.0)
    for nt, tag in ((0, ""), (1, "nt_")):
        best = 0.0
        for wgr in (4 * cus, 8 * cus, 16 * cus, 32 * cus):
            snk = torch.empty(wgr * T, device="cuda", dtype=torch.int32)
            ms = run(lambda: P.streamkl_probe_read(src.data_ptr(), nbytes, nt, wgr, snk.data_ptr(), snk.numel() * 4, s))
            out[f"read_{tag}gbs_{wgr}wg"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            best = max(best, nbytes / (ms * 1e-3) / 1e9)
            del snk
        out[f"read_{tag}gbs_best"] = round(best, 1)
        out[f"read_{tag}frac_of_hbm_peak"] = round(best / PEAK_HBM_GBS, 4)
    del src
    # fp32 atomics: 1 GiB (the size of one 64K-causal dQ) and 2 MiB (fits one XCD's L2)
    for name, n, r in (("1GiB", (1 << 30) // 4, 2), ("2MiB", (2 << 20) // 4, 512)):
        dst = torch.zeros(n, device="cuda", dtype=torch.float32)
        ms = run(lambda: P.streamkl_probe_atomic(dst.data_ptr(), n, 8 * cus, r, s))
        out[f"atomic_f32_payload_gbs_{name}"] = round(4 * n * r / (ms * 1e-3) / 1e9, 1)
        del dst
    torch.cuda.empty_cache()
    print(json.dumps(out), flush=True)


def cpu_sample(w: W.Workload):
    """The one-head sub-workload the CPU baseline runs, and its description."""
    if w.causal:
        m = min(w.n_q, 16384)
        sub = w.replace(n_q=m, n_k=m + (w.n_k - w.n_q), heads=1)
        return sub, f"first {m} queries x {sub.n_k} keys (causal)"
    m = min(w.n_q, 8192)
    sub = w.replace(n_q=m, n_k=min(w.n_k, (1 << 25) // m), heads=1)
    return sub, f"first {m} queries x first {sub.n_k} keys"


def cpu_baseline(w: W.Workload):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload,
    forward + Setting 1 + Setting 2 backward on head 0.  Causal: the first
    (at most) 16384 queries with every key they may see (the top-left block of
    the real problem; for the 64K causal workload, rows 0..16383 against keys
    0..16383).  Non-causal: the first (at most) 8192 queries against the first
    keys, at most 2^25 pairs in all."""
    import oracle
    sub, what = cpu_sample(w)
    q1, k1, q2, k2 = W.head_inputs(sub, 0)   # prefix rows of head 0's draws
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.forward_head(q1, k1, q2, k2, w.scale, w.causal)
    oracle.backward_head(1, q1, k1, q2, k2, w.scale, w.causal)
    oracle.backward_head(2, q1, k1, q2, k2, w.scale, w.causal)
    dt = time.perf_counter() - t0
    flop = 20 * w.head_dim * sub.elements()
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"head 0 of {w.name}, {what}, fwd + bwd Setting 1 + "
                      f"Setting 2, fp64 numpy/BLAS; {dt:.1f} s for {flop / 1e12:.3f} TFLOP"}


def ceiling_part(seconds: float = 4.0) -> dict:
    """The matrix cores' sustained rate on this GPU with the operand pattern of
    the step's kernels (random bf16 operands, one of them streamed from LDS for
    every MFMA), measured beside the step: one wave per SIMD, as in the
    both-settings kernels, and two, as in the forward and the single-setting
    kernels.  Each probe runs back to back for `seconds` so the board settles
    at its power limit.  Boards of the pool differ by up to ~12% in the work
    that power buys; a kernel's rate divided by the probe's on the same board
    does not."""
    import torch
    from streaming_kl_divergence_amd import _lib
    P = _lib.probes()
    T = P.streamkl_probe_threads()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    s = torch.cuda.current_stream().cuda_stream
    src = torch.randn(2 * cus * T * 128, device="cuda").to(torch.bfloat16)   # 256 bytes per thread
    sink = torch.empty(2 * cus * T, device="cuda")
    out = {}
    for wps in (1, 2):
        wg, iters = wps * cus, 75000 // wps
        launch = lambda: P.streamkl_probe_mfma_data(src.data_ptr(), src.numel() * 2, 1, wps, wg, iters,
                                                    sink.data_ptr(), sink.numel(), s)
        if launch() != 0:
            raise RuntimeError("probe launch failed")
        ms, _, _ = _loop_for(launch, seconds)
        out[f"lds_operand_{wps}_wave_per_simd_tflops"] = round(wg * 4 * iters * 8 * 32768 / (ms * 1e-3) / 1e12, 1)
    del src, sink
    torch.cuda.empty_cache()
    return out


def decode_part(reps: int = 20) -> dict:
    """The 512K-key decode workload (32 heads, one query, split-K with the
    automatic count) timed beside the step: HBM read rate of its inputs."""
    import torch
    import streaming_kl_divergence_amd as skl
    w = W.WORKLOADS["decode512k"]
    q1, k1, q2, k2 = upload(w, min(16, os.cpu_count() or 1))
    d = w.head_dim
    ws = torch.empty(max(16, skl.splitk_workspace_bytes(w.n_q, w.n_k, w.heads, d, 0)), device="cuda",
                     dtype=torch.uint8)
    ms = _timed_batches(lambda: skl.fwd_splitk(q1, k1, q2, k2, w.scale, w.causal, 0, ws),
                        torch.cuda.current_stream(), 3, reps)
    byts = 2 * w.heads * (w.n_k + w.n_q) * d * 2
    gbs = byts / (ms * 1e-3) / 1e9
    del q1, k1, q2, k2, ws
    torch.cuda.empty_cache()
    return {"ms": round(ms, 4), "gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
            "splits": skl.splitk_auto(w.n_q, w.n_k, w.heads, d),
            "work": "split-K forward, 32 heads x 1 query x 524288 keys, d=128, bf16: K1, K2, Q1, Q2 read once"}


def decode_mode(w: W.Workload, args, inputs, t_up: float):
    """One query per head (decode): one step is the split-K forward with the
    library's automatic split count, the partial kernel and then the combine
    kernel (a few microseconds).  Bound by HBM: the rate is the bytes of
    K1, K2, Q1, Q2 read once per step over the step's time."""
    import torch
    import streaming_kl_divergence_amd as skl
    q1, k1, q2, k2 = inputs
    d = w.head_dim
    stream = torch.cuda.current_stream()
    splits = skl.splitk_auto(w.n_q, w.n_k, w.heads, d)
    ws = torch.empty(max(16, skl.splitk_workspace_bytes(w.n_q, w.n_k, w.heads, d, 0)), device="cuda",
                     dtype=torch.uint8)
    call = lambda: skl.fwd_splitk(q1, k1, q2, k2, w.scale, w.causal, 0, ws)
    # exactly `steps` calls back to back between two events, synchronised on
    # both sides (the host enqueues ahead of the GPU: no host time between calls)
    ms = _timed_batches(call, stream, args.warmup, args.steps, rounds=1)
    esize = 2 if w.dtype == "bf16" else 4
    byts = 2 * w.heads * (w.n_k + w.n_q) * d * esize
    gbs = byts / (ms * 1e-3) / 1e9
    out = {
        "metric": f"split-K decode HBM read rate ({w.heads} heads, N_Q={w.n_q}, N_K={w.n_k}, d={d}, {w.dtype})",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.heads} heads, N_Q={w.n_q}, N_K={w.n_k}, head_dim={d}, {w.dtype}, "
                               f"non-causal, independent teacher and student; step = split-K forward",
                   "heads": w.heads, "n_q": w.n_q, "n_k": w.n_k, "head_dim": d, "causal": w.causal,
                   "splits": splits},
        "parts": {"upload_s": round(t_up, 1)},
        "roofline": {"bound": "hbm", "kernel": "fwd_kernel (split-K partials; the timed call includes the combine)",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic("fwd_kernel", w.name),
                     "avg_launch_ms": round(ms, 4),
                     "work_per_launch": f"K1, K2, Q1, Q2 read once = {byts} bytes"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w)
    print(json.dumps(out), flush=True)


def cpu_baseline_decode(w: W.Workload, heads: int = 0):
    """The fp64 oracle's forward on the first `heads` heads (0 = all) of a
    decode workload (each head's one query against all its keys), as the
    same bytes-per-second rate; inputs are drawn before the clock starts."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    heads = heads or w.heads
    dt = 0.0
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for a in ex.map(lambda h: W.head_inputs(w, h), range(heads)):
            t0 = time.perf_counter()
            oracle.forward_head(*a, w.scale, w.causal)
            dt += time.perf_counter() - t0
    esize = 2 if w.dtype == "bf16" else 4
    byts = heads * 2 * (w.n_k + w.n_q) * w.head_dim * esize
    return {"value": byts / dt / 1e9, "unit": "GB/s", "cores": cores, "host_cores": os.cpu_count(),
            "kind": "oracle",
            "sample": f"heads 0..{heads - 1} of {w.name} (all keys), forward, fp64 numpy/BLAS; "
                      f"{dt:.1f} s for {byts / 1e9:.2f} GB of inputs"}


def gemm_reference(n: int = 16384, reps: int = 10) -> float:
    """Dense bf16 GEMM throughput of the platform library (torch.mm, which
    calls hipBLASLt) on this GPU, TFLOP/s: a measured reference for what the
    matrix cores deliver on a plain contraction, beside the published peak."""
    import torch
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    t = _timed(lambda: torch.mm(a, b, out=c), torch.cuda.current_stream(), 3, reps)
    del a, b, c
    return 2.0 * n ** 3 / (float(np.median(t)) * 1e-3) / 1e12


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gemm-ref", action="store_true", help="also time a 16384^3 bf16 GEMM (torch.mm) as context")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the matrix-core probe measured beside the step (parts.mfma_ceiling)")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the 512K-key split-K decode measured beside the step (parts.decode512k)")
    ap.add_argument("--no-gemm-ref", action="store_true", help=argparse.SUPPRESS)   # the default; kept for old commands
    ap.add_argument("--workload", default="causal64k")
    ap.add_argument("--configs", action="store_true")
    ap.add_argument("--sweep", choices=("crossover", "splitk", "context"))
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--calibrate", action="store_true",
                    help="run the calibration probes (MFMA loop, v_exp_f32, HBM read, fp32 atomics)")
    ap.add_argument("--ab", metavar="LIB_A,LIB_B",
                    help="time two builds of libstreamkl.so against each other in one process (with --workload, "
                         "--ab-calls); see ab_mode")
    ap.add_argument("--ab-calls", help="comma-separated: fwd, splitk, dk_both, dq_both, dk1, dq1, dk2, dq2")
    ap.add_argument("--ab-rounds", type=int, default=8)
    ap.add_argument("--power", action="store_true",
                    help="board power while each kernel of the 64K causal step runs back to back, and probes")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--sq-summary", nargs="+", metavar="DIR")
    ap.add_argument("--bwd-path", choices=("both", "separate"), default="both",
                    help="backward of the step: both settings from one recomputation (default), or the two "
                         "single-setting passes with the library's path choice")
    args = ap.parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload)
        return
    if args.sq_summary:
        sq_summary(args.sq_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no exchange between them).", file=sys.stderr)
        sys.exit(1)

    import torch
    import streaming_kl_divergence_amd as skl

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, device="cuda", dtype=torch.float32)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.ab:
        ab_mode(args.ab.split(","), args.workload or "causal64k",
                args.ab_calls.split(",") if args.ab_calls else None, args.ab_rounds)
        return
    if args.calibrate:
        calibrate_mode()
        return
    if args.power:
        power_mode()
        return
    if args.configs:
        configs_mode()
        return
    if args.sweep:
        sweep_mode(args.sweep)
        return
    w = W.WORKLOADS[args.workload]
    threads = min(16, os.cpu_count() or 1)
    t_up = time.perf_counter()
    q1, k1, q2, k2 = upload(w, threads)
    t_up = time.perf_counter() - t_up
    if w.n_q == 1:
        decode_mode(w, args, (q1, k1, q2, k2), t_up)
        return
    scale, causal = w.scale, w.causal
    E = w.elements()
    d = w.head_dim
    flop_fwd = 4 * d * E
    flop_bwd = 8 * d * E
    flop_step = flop_fwd + 2 * flop_bwd
    stream = torch.cuda.current_stream()
    # the step needs both settings' gradients: by default one recomputation
    # serves both (streamkl_bwd_both); --bwd-path separate times the two
    # single-setting backward passes instead
    path = args.bwd_path if args.bwd_path == "both" else skl.bwd_select(w.n_q, w.n_k, w.heads, d, causal)
    # every call below launches one kernel, so the events around it time that kernel
    if path == "both":
        calls = [("fwd_kernel", 4), ("bwd_kv_both_kernel", 8), ("bwd_q_both_kernel", 8)]
    elif path == "separate":
        calls = [("fwd_kernel", 4), ("bwd_kv_kernel set1", 6), ("bwd_q_kernel set1", 6),
                 ("bwd_kv_kernel set2", 6), ("bwd_q_kernel set2", 6)]
    else:
        calls = [("fwd_kernel", 4), ("bwd_kv_kernel fused set1", 8), ("bwd_kv_kernel fused set2", 8)]
    grads = [torch.empty(w.heads, n, d, device="cuda", dtype=torch.float32) for n in (w.n_q, w.n_k, w.n_q, w.n_k)]
    dq, dk = grads[0], grads[1]

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
        if path == "both":
            dq1, dk1, dq2, dk2 = grads
            skl.bwd_both(q1, k1, q2, k2, scale, causal, l1, l2, kl, path="dk_only", dk1=dk1, dk2=dk2)
            mark()
            skl.bwd_both(q1, k1, q2, k2, scale, causal, l1, l2, kl, path="dq_only", dq1=dq1, dq2=dq2)
            mark()
            return
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
    bwd_ms = float(mean_call[1:].sum())
    parts["fwd_ms"] = round(fwd_ms_, 3)
    parts["fwd_tflops"] = round(flop_fwd / (fwd_ms_ * 1e-3) / 1e12, 1)
    parts["bwd_both_settings_ms"] = round(bwd_ms, 3)
    parts["bwd_both_settings_tflops"] = round(2 * flop_bwd / (bwd_ms * 1e-3) / 1e12, 1)
    if path != "both":
        bwd1_ms = float(mean_call[1:1 + (len(calls) - 1) // 2].sum())
        bwd2_ms = float(mean_call[1 + (len(calls) - 1) // 2:].sum())
        parts["bwd_set1_ms"] = round(bwd1_ms, 3)
        parts["bwd_set2_ms"] = round(bwd2_ms, 3)
        parts["bwd_set1_tflops"] = round(flop_bwd / (bwd1_ms * 1e-3) / 1e12, 1)
        parts["bwd_set2_tflops"] = round(flop_bwd / (bwd2_ms * 1e-3) / 1e12, 1)
    peak = peak_tflops(w.dtype)
    parts["pct_mfma_peak_step"] = round(100 * value / peak, 2)
    if args.gemm_ref and not args.no_gemm_ref:
        gemm = gemm_reference()
        parts["gemm_bf16_16384_tflops"] = round(gemm, 1)
    parts["wall_s_timed"] = round(wall, 3)
    parts["upload_s"] = round(t_up, 1)
    if not args.no_decode:
        parts["decode512k"] = decode_part()

    # dominant kernel: the single launch with the largest mean duration
    j = int(np.argmax(mean_call))
    kname, kflop = calls[j]
    achieved = kflop * d * E / (mean_call[j] * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(float(achieved), 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(float(achieved) / peak, 4),
                "traffic": measured_traffic(kname, w.name),
                "avg_launch_ms": round(float(mean_call[j]), 3),
                "work_per_launch": f"{kflop}*d flop x {E} unmasked pairs = {kflop * d * E / 1e12:.3f} TFLOP"}
    if w.dtype != "bf16":
        parts["mfma_ceiling"] = {"skipped": "the probes run bf16 MFMAs; this workload is " + w.dtype}
    elif not args.no_ceiling:
        # each kernel's executed MFMA rate (k*d flop per pair, as it runs)
        # against the probe at its occupancy: the both-settings and fused
        # kernels run one wave per SIMD, the others two
        try:
            ceil = ceiling_part()
        except ImportError as e:   # the probes are a library of their own; the step does not need them
            ceil = {"skipped": str(e)}
        else:
            for name, k in calls:
                wps = 1 if ("both" in name or "fused" in name) else 2
                ceil[f"{name}_frac"] = round(k * d * E / (parts[name]["ms"] * 1e-3) / 1e12
                                             / ceil[f"lds_operand_{wps}_wave_per_simd_tflops"], 3)
        parts["mfma_ceiling"] = ceil
    mask = "causal" if causal else "non-causal"
    sizes = f"N_Q=N_K={w.n_q}" if w.n_q == w.n_k else f"N_Q={w.n_q}, N_K={w.n_k}"
    out = {
        "metric": METRIC if w.name == "causal64k" else
        f"fwd/bwd TFLOP/s + ms, {w.heads} heads d={d} {w.dtype} {mask} {sizes}; % MFMA peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.heads} heads, {sizes}, head_dim={d}, {w.dtype}, {mask}, "
                               f"{w.student} student; step = fwd + bwd Setting 1 + bwd Setting 2",
                   "heads": w.heads, "n_q": w.n_q, "n_k": w.n_k, "head_dim": d, "causal": causal,
                   "bwd_path": path},
        "parts": parts,
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
