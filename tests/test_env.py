"""Environment overrides and dispatch logging of the C-ABI library, on the CPU.

The library reads STREAMKL_LOG, STREAMKL_SPLITS and STREAMKL_BWD_PATH once per
process, so each case runs in a child process with its own environment.  Only
the helpers and calls that are rejected before any launch are made (no GPU is
touched); the GPU tests check the same overrides on real launches.
"""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys
from streaming_kl_divergence_amd import _lib as L
lib = L.lib()
F = 4096
out = {
    "auto": lib.streamkl_splitk_auto(1, 4096, 2, 128),
    "ws0": lib.streamkl_workspace_bytes(0, 1, 4096, 2, 128, 0, 0),
    "ws3": lib.streamkl_workspace_bytes(0, 1, 4096, 2, 128, 3, 0),
    "select": lib.streamkl_bwd_select(4096, 4096, 2, 128, 1),
    # rejected before launch: NULL output, workspace too small, unknown backward path
    "fwd_null": lib.streamkl_fwd(F, F, F, F, 16, 16, 2, 64, 0, 0.125, L.BF16, None, F, F, None),
    "splitk_ws": lib.streamkl_fwd_splitk(F, F, F, F, 1, 4096, 2, 128, 0, 0.125, L.BF16, 0, F, F, F, F, 16, None),
    "bwd_path": lib.streamkl_bwd_set1(F, F, F, F, 16, 16, 2, 128, 0, 0.125, L.FP32, F, F, None, F, F,
                                      9, None, 0, None),
}
sys.stderr.flush()
print(json.dumps(out))
"""


def run_child(**env):
    e = {k: v for k, v in os.environ.items() if not k.startswith("STREAMKL_")}
    e.update(env)
    e["PYTHONPATH"] = ROOT + os.pathsep + e.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", CHILD], env=e, cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    return json.loads(r.stdout.strip().splitlines()[-1]), r.stderr


def log_lines(err):
    return [l for l in err.splitlines() if l.startswith("streamkl: streamkl_")]


def test_defaults_print_nothing():
    out, err = run_child()
    assert out["select"] == 2                       # separate
    assert out["ws0"] == out["auto"] * 2 * 1 * 20   # splits x heads x n_q x 5 floats
    assert out["ws3"] == 3 * 2 * 1 * 20
    assert (out["fwd_null"], out["splitk_ws"], out["bwd_path"]) == (-1, -5, -3)
    assert log_lines(err) == []


def test_splits_override_sets_the_auto_count_and_its_workspace():
    base, _ = run_child()
    out, err = run_child(STREAMKL_SPLITS="5")
    # 4096 keys are 64 tiles of 64; 5 ranges of 13 tiles are all non-empty
    assert out["auto"] == 5 != base["auto"]
    assert out["ws0"] == 5 * 2 * 1 * 20
    assert out["ws3"] == 3 * 2 * 1 * 20             # an explicit count wins
    assert log_lines(err) == []
    # more ranges than whole tiles collapse to the non-empty ones
    out, _ = run_child(STREAMKL_SPLITS="1000")
    assert out["auto"] == 64


def test_bwd_path_override_changes_what_auto_resolves_to():
    out, _ = run_child(STREAMKL_BWD_PATH="fused")
    assert out["select"] == 1
    out, _ = run_child(STREAMKL_BWD_PATH="separate")
    assert out["select"] == 2


def test_unparsable_values_are_ignored_with_a_warning():
    base, _ = run_child()
    out, err = run_child(STREAMKL_SPLITS="lots", STREAMKL_BWD_PATH="sideways")
    assert out == base
    assert "STREAMKL_SPLITS=lots ignored" in err
    assert "STREAMKL_BWD_PATH=sideways ignored" in err
    out, err = run_child(STREAMKL_SPLITS="0")
    assert out == base and "STREAMKL_SPLITS=0 ignored" in err


def test_log_prints_one_line_per_compute_call():
    out, err = run_child(STREAMKL_LOG="1", STREAMKL_SPLITS="5")
    lines = log_lines(err)
    assert len(lines) == 3, err                     # helpers are not logged
    fwd, splitk, bwd = lines
    assert fwd.startswith("streamkl: streamkl_fwd heads=2 n_q=16 n_k=16 d=64 causal=0 bf16")
    assert fwd.endswith("-> a required pointer is NULL")
    assert "splits=5 (STREAMKL_SPLITS) keys_per_split=832 workgroups=10 workspace=200/16" in splitk
    assert splitk.endswith("-> workspace missing or too small")
    assert bwd.startswith("streamkl: streamkl_bwd_set1 heads=2 n_q=16 n_k=16 d=128 causal=0 fp32")
    assert bwd.endswith("-> unsupported head_dim, dtype, path or split count")
    _, err = run_child(STREAMKL_LOG="0")
    assert log_lines(err) == []
