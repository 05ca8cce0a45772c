"""Device helpers for GPU tests: upload seeded inputs, call the library."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

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


def host_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def workload_device_inputs(w: W.Workload):
    """Upload a workload head by head (host memory stays per-head); heads are
    generated in a thread pool."""
    import torch
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = [torch.empty(w.heads, n, w.head_dim, dtype=tdt, device="cuda")
           for n in (w.n_q, w.n_k, w.n_q, w.n_k)]

    def one(h):
        return h, [torch.from_numpy(a).to(tdt) for a in W.head_inputs(w, h)]

    with ThreadPoolExecutor(host_threads()) as ex:
        for h, parts in ex.map(one, range(w.heads)):
            for t, a in zip(out, parts):
                t[h].copy_(a)
    torch.cuda.synchronize()
    return out


def head64(w: W.Workload, h: int):
    """The seeded inputs of head h as fp64 arrays (converted once)."""
    return [np.asarray(a, dtype=np.float64) for a in W.head_inputs(w, h)]


def pmap(fn, items):
    """fn over items in a thread pool (numpy releases the GIL in BLAS and ufuncs)."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1), ThreadPoolExecutor(host_threads()) as ex:
        return list(ex.map(fn, items))


def chunks(rows, size: int = 256):
    rows = np.asarray(rows, dtype=np.int64)
    return [rows[i:i + size] for i in range(0, rows.size, size)]
