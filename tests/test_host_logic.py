"""Host-side logic on the CPU: the seeded input generators shared by the GPU
path and the oracle, and bench.py's kernel naming and counter arithmetic."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_round_bf16_matches_torch_nearest_even():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * np.float32(10) ** rng.integers(-30, 30, 100000),
        # exact ties between two bf16 neighbours, both parities of the kept bit
        (np.arange(1, 2000, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.0e38, -3.0e38, 1e-40, -1e-40], dtype=np.float32),
    ]).astype(np.float32)
    ours = W.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    # the result is exactly representable: the low half-word is zero
    assert not np.any(ours.view(np.uint32) & np.uint32(0xFFFF))
    assert np.array_equal(W.bf16_bits(ours), (ours.view(np.uint32) >> 16).astype(np.uint16))


def test_generators_are_deterministic_and_row_prefixes():
    w = W.WORKLOADS["noncausal128k"].replace(n_q=700, n_k=900)
    a = W.head_inputs(w, 3)
    b = W.head_inputs(w, 3)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # a shorter draw from the same stream is a prefix: smallq128k's queries are
    # the first rows of noncausal128k's, and the CPU baseline's 16K block is the
    # top-left corner of the 64K causal workload
    short = W.head_inputs(w.replace(n_q=300, n_k=500), 3)
    for x, y, n in zip(short, a, (300, 500, 300, 500)):
        assert np.array_equal(x, y[:n])
    assert W.WORKLOADS["smallq128k"].seed == W.WORKLOADS["noncausal128k"].seed
    # different heads and tensors draw different numbers
    c = W.head_inputs(w, 4)
    assert not np.array_equal(a[0], c[0]) and not np.array_equal(a[0], a[2])
    # bf16 workloads hold exact bf16 values; correlated students are close to their teachers
    wc = W.WORKLOADS["causal8k"].replace(n_q=64, n_k=64)
    q1, k1, q2, k2 = W.head_inputs(wc, 0)
    assert np.array_equal(W.round_bf16(q1), q1)
    assert 0.2 < np.std(q2 - q1) < 0.4


@pytest.mark.parametrize("n_q,n_k,causal", [(5, 5, True), (3, 8, True), (7, 2, False), (1, 9, True), (64, 200, True)])
def test_element_count_matches_brute_force(n_q, n_k, causal):
    w = W.Workload("t", 3, n_q, n_k, 64, "bf16", causal, "independent", 0)
    brute = 3 * sum(1 for i in range(n_q) for j in range(n_k) if (not causal) or j <= i + (n_k - n_q))
    assert w.elements() == brute


def test_kernel_labels():
    L = bench.kernel_label
    assert L("_ZN3skl10fwd_kernelIDF16bLi128ELi4ELb0EEEvNS_9FwdParamsE") == "fwd_kernel"
    assert L("_ZN3skl13bwd_kv_kernelIDF16bLi128ELi1ELb0ELb0EEEvNS_9BwdParamsE") == "bwd_kv_kernel set1"
    assert L("_ZN3skl13bwd_kv_kernelIDF16bLi128ELi2ELb1ELb0EEEvNS_9BwdParamsE") == "bwd_kv_kernel fused set2"
    assert L("_ZN3skl12bwd_q_kernelIDF16bLi128ELi2ELb0ELb1EEEvNS_9BwdParamsE") == "bwd_q_kernel set2"
    assert L("_ZN3skl21splitk_combine_kernelENS_9FwdParamsE") == "splitk_combine_kernel"
    assert L("_ZN3skl18bwd_kv_both_kernelILi128ELb0EEEvNS_9BwdParamsE") == "bwd_kv_both_kernel"
    assert L("_ZN3skl17bwd_q_both_kernelILi128ELb0ELb1EEEvNS_9BwdParamsE") == "bwd_q_both_kernel"
    # the profiler prints some names demangled
    assert L("void skl::bwd_kv_both_kernel<128, false>(skl::BwdParams)") == "bwd_kv_both_kernel"
    assert L("void skl::bwd_q_both_kernel<64, true, false>(skl::BwdParams)") == "bwd_q_both_kernel"
    assert L("void skl::bwd_kv_kernel<__bf16, 128, 2, true, false>(skl::BwdParams)") == "bwd_kv_kernel fused set2"
    assert L("void skl::bwd_q_kernel<__bf16, 128, 1, false, true>(skl::BwdParams)") == "bwd_q_kernel set1"
    assert L("void skl::fwd_kernel<__bf16, 128, 4, false>(skl::FwdParams)") == "fwd_kernel"
    assert L("skl::splitk_combine_kernel(skl::FwdParams)") == "splitk_combine_kernel"
    assert L("__amd_rocclr_copyBuffer") is None


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "pmc_counter_collection.csv"), "w") as f:
        f.write('"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"\n')
        for i, (k, c, v) in enumerate(rows):
            f.write(f'"{i}","{k}","{c}","{v}"\n')


def test_pmc_summary_scales_by_the_copy(tmp_path, monkeypatch):
    kv = "_ZN3skl13bwd_kv_kernelIDF16bLi128ELi1ELb0ELb0EEEvNS_9BwdParamsE"
    gib_kib = (1 << 30) / 1024
    # the counters read half the copy's bytes for FETCH and all of them for WRITE
    _counter_csv(tmp_path / "f", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib / 2), (kv, "FETCH_SIZE", 1000.0)])
    _counter_csv(tmp_path / "w", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib), (kv, "WRITE_SIZE", 300.0)])
    out = tmp_path / "profiles"
    out.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"))
    import json
    with open(out / "traffic.json") as f:
        t = json.load(f)
    assert abs(t["_calibration"]["fetch_factor"] - 2.0) < 1e-9
    assert abs(t["_calibration"]["write_factor"] - 1.0) < 1e-9
    e = t["bwd_kv_kernel set1"]
    assert e["fetch_bytes"] == 2 * 1000 * 1024 and e["write_bytes"] == 300 * 1024
    assert e["bytes_per_launch"] == 2300 * 1024 and e["source_hash"] == "abc"


def test_traffic_files_per_workload(tmp_path, monkeypatch):
    """Each workload's counter summary has its own file, and a summary is used
    only while the device sources hash to what it was taken with."""
    kv = "_ZN3skl13bwd_kv_kernelIDF16bLi128ELi1ELb0ELb0EEEvNS_9BwdParamsE"
    gib_kib = (1 << 30) / 1024
    _counter_csv(tmp_path / "f", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", gib_kib), (kv, "FETCH_SIZE", 10.0)])
    _counter_csv(tmp_path / "w", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", gib_kib), (kv, "WRITE_SIZE", 0.0)])
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h1")
    bench.pmc_summary(str(tmp_path / "f"), str(tmp_path / "w"), workload="decode512k")
    assert (tmp_path / "profiles" / "traffic_decode512k.json").exists()
    assert not (tmp_path / "profiles" / "traffic.json").exists()
    assert bench.measured_traffic("bwd_kv_kernel set1", "decode512k") == 10 * 1024
    assert bench.measured_traffic("bwd_kv_kernel set1") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h2")
    assert bench.measured_traffic("bwd_kv_kernel set1", "decode512k") is None


def test_bench_peak_and_cpu_sample_follow_the_workload():
    assert bench.peak_tflops("bf16") == 2516.6 and bench.peak_tflops("fp32") == 157.3
    for name, w in W.WORKLOADS.items():
        sub, what = bench.cpu_sample(w)
        assert sub.heads == 1 and sub.n_q <= w.n_q and sub.n_k <= w.n_k and sub.causal == w.causal
        assert (sub.dtype, sub.student, sub.seed, sub.head_dim) == (w.dtype, w.student, w.seed, w.head_dim)
        # bounded: at most 16384 causal rows (1.3e8 pairs) or 2^25 non-causal pairs
        assert sub.elements() <= max(16384 * 16385 // 2, 1 << 25), name
        if w.causal:   # the same causal offset: the top-left block of the real mask
            assert sub.n_k - sub.n_q == w.n_k - w.n_q
    sub, what = bench.cpu_sample(W.WORKLOADS["causal64k"])
    assert (sub.n_q, sub.n_k) == (16384, 16384) and what == "first 16384 queries x 16384 keys (causal)"
    sub, _ = bench.cpu_sample(W.WORKLOADS["smallq128k"])
    assert (sub.n_q, sub.n_k) == (512, 65536)
    # prefix rows: the sample's inputs are the first rows of the full workload's head 0
    w = W.WORKLOADS["causal8k"].replace(n_q=64, n_k=64)
    full = W.head_inputs(w, 0)
    part = W.head_inputs(w.replace(n_q=16, n_k=16), 0)
    for a, b in zip(full, part):
        assert np.array_equal(a[:16], b)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 1 and "one GPU" in r.stderr


def _undefined_names(path):
    """Names a function reads that nothing defines: not a local, a module-level
    name or a builtin (symtable's view; catches what only a GPU run would
    otherwise reach, such as a variable left over from an edit)."""
    import builtins
    import symtable
    with open(path) as f:
        top = symtable.symtable(f.read(), path, "exec")
    module = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported() or s.is_namespace()}
    bad = []

    def walk(t):
        for s in t.get_symbols():
            n = s.get_name()
            if (s.is_referenced() and s.is_global() and not s.is_declared_global() and n not in module
                    and not hasattr(builtins, n) and n not in ("__file__", "__name__")):
                bad.append((t.get_name(), t.get_lineno(), n))
        for c in t.get_children():
            walk(c)
    walk(top)
    return bad


def test_python_sources_reference_no_undefined_names():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = ["bench.py", "__graft_entry__.py", "workloads/__init__.py"]
    for d in ("streaming_kl_divergence_amd", "oracle", "tests"):
        files += [os.path.join(d, f) for f in sorted(os.listdir(os.path.join(root, d))) if f.endswith(".py")]
    found = {f: _undefined_names(os.path.join(root, f)) for f in files}
    assert not any(found.values()), {f: b for f, b in found.items() if b}
