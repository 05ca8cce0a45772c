"""Environment overrides on real launches: with STREAMKL_SPLITS and
STREAMKL_BWD_PATH set, the automatic choices run exactly what the explicit
arguments run (bitwise), and STREAMKL_LOG reports each launch.  The library
reads the environment once per process, so the launches run in a child
process (one more process on the GPU, small shapes)."""
import json
import os
import subprocess
import sys

import pytest

from tests.gpu_util import need_gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import json, sys
import torch
import streaming_kl_divergence_amd as skl
import workloads as W
from tests.gpu_util import device_inputs
print("child: 2 heads, 100 x 3000, d=128, causal, splits and fused overrides", file=sys.stderr, flush=True)
w = W.Workload("env", 2, 100, 3000, 128, "bf16", True, "correlated", 11)
q1, k1, q2, k2 = device_inputs(W.all_inputs(w), "bf16")
sc = w.scale
auto = skl.fwd_splitk(q1, k1, q2, k2, sc, True, num_splits=0)
given = skl.fwd_splitk(q1, k1, q2, k2, sc, True, num_splits=3)
kl, l1, l2 = given
g_auto = skl.bwd(1, q1, k1, q2, k2, sc, True, l1, l2, path="auto")
g_fused = skl.bwd(1, q1, k1, q2, k2, sc, True, l1, l2, path="fused")
g_sep = skl.bwd(1, q1, k1, q2, k2, sc, True, l1, l2, path="separate")
torch.cuda.synchronize()
same = lambda a, b: all(torch.equal(x, y) for x, y in zip(a, b))
rel = lambda a, b: float((a - b).norm() / b.norm())
# dK of the fused kernel is deterministic; its dQ is added with fp32 atomics
# in launch order, so it is compared by norm
print(json.dumps({"fwd": same(auto, given), "dk": torch.equal(g_auto[1], g_fused[1]),
                  "dq_rel": rel(g_auto[0], g_fused[0]), "sep_rel": rel(g_auto[0], g_sep[0])}))
"""


@pytest.mark.gpu
def test_overrides_run_what_the_explicit_arguments_run():
    need_gpu()
    e = {k: v for k, v in os.environ.items() if not k.startswith("STREAMKL_")}
    e.update(STREAMKL_LOG="1", STREAMKL_SPLITS="3", STREAMKL_BWD_PATH="fused",
             PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", CHILD], env=e, cwd=ROOT, capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-3000:]
    out = json.loads(r.stdout.strip().splitlines()[-1])
    assert out["fwd"] and out["dk"], out
    assert out["dq_rel"] < 1e-5 and out["sep_rel"] < 5e-3, out
    lines = [l for l in r.stderr.splitlines() if l.startswith("streamkl: streamkl_")]
    assert len(lines) == 5, r.stderr[-3000:]
    assert all(l.endswith("-> ok") for l in lines), lines
    assert "splits=3 (STREAMKL_SPLITS)" in lines[0] and "splits=3 (given)" in lines[1]
    assert "path=fused (asked auto, STREAMKL_BWD_PATH)" in lines[2]
    assert "path=fused (asked fused)" in lines[3]
    assert "path=separate (asked separate)" in lines[4]
