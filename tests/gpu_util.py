"""Device helpers for GPU tests: upload seeded inputs, call the library."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import workloads as W


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def device_inputs(arrs, dtype: str):
    return [to_device(a, dtype) for a in arrs]


def workload_device_inputs(w: W.Workload):
    """Upload a workload head by head (host memory stays per-head)."""
    import torch
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = [torch.empty(w.heads, n, w.head_dim, dtype=tdt, device="cuda")
           for n in (w.n_q, w.n_k, w.n_q, w.n_k)]
    for h in range(w.heads):
        for t, a in zip(out, W.head_inputs(w, h)):
            t[h].copy_(torch.from_numpy(a).to(tdt))
    torch.cuda.synchronize()
    return out
