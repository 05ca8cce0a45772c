"""Torch-facing wrappers over the C ABI.  Every step runs in the HIP library;
these functions only check tensors, allocate outputs with torch and pass
pointers and the current stream of the inputs' device (made current for the
call)."""
from __future__ import annotations

import functools

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.BF16, torch.float32: _lib.FP32}
_PATH = {"auto": _lib.BWD_AUTO, "fused": _lib.BWD_FUSED, "separate": _lib.BWD_SEPARATE,
         "dk_only": _lib.BWD_DK_ONLY, "dq_only": _lib.BWD_DQ_ONLY}


def _inputs(q1, k1, q2, k2):
    for t in (q1, k1, q2, k2):
        if not t.is_cuda:
            raise ValueError("inputs must be device tensors")
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous [heads, n, head_dim]")
        if t.dim() != 3:
            raise ValueError("inputs must be [heads, n, head_dim]")
    if len({q1.device, k1.device, q2.device, k2.device}) != 1:
        raise ValueError("inputs must be on one device")
    if len({q1.dtype, k1.dtype, q2.dtype, k2.dtype}) != 1 or q1.dtype not in _DT:
        raise ValueError("inputs must share one dtype: bfloat16 or float32")
    heads, n_q, d = q1.shape
    n_k = k1.shape[1]
    if q2.shape != q1.shape or k1.shape != (heads, n_k, d) or k2.shape != k1.shape:
        raise ValueError("shape mismatch between Q1, K1, Q2, K2")
    return heads, n_q, n_k, d, _DT[q1.dtype]


def check_rows(t, name: str, heads: int, n_q: int, device) -> None:
    """A per-row array (lse1, lse2, kl, dkl): fp32 [heads, n_q], contiguous, on `device`."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}; the inputs are on {device}")
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (heads, n_q):
        raise ValueError(f"{name} must be a contiguous fp32 [{heads}, {n_q}] tensor")


def check_out(t, name: str, shape, device) -> None:
    """A caller-given gradient output: fp32 of `shape`, contiguous, on `device`."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}; the inputs are on {device}")
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous fp32 {list(shape)} tensor")


def check_disjoint(named) -> None:
    """Output tensors must not share memory (the kernels write them concurrently)."""
    spans = []
    for name, t in named:
        if t is None:
            continue
        lo = t.data_ptr()
        spans.append((lo, lo + t.numel() * t.element_size(), name))
    spans.sort()
    for (a0, a1, an), (b0, b1, bn) in zip(spans, spans[1:]):
        if b0 < a1:
            raise ValueError(f"outputs {an} and {bn} overlap")


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _on_device(fn):
    """Run an entry point with the inputs' device current, so the library
    launches on that device and on its current stream."""
    @functools.wraps(fn)
    def wrapped(*args, **kw):
        q1 = next((a for a in args if isinstance(a, torch.Tensor)), None)
        if q1 is None or not q1.is_cuda:
            return fn(*args, **kw)    # the entry point's own checks reject it
        with torch.cuda.device(q1.device):
            return fn(*args, **kw)
    return wrapped


def _ptr(t):
    return None if t is None else t.data_ptr()


@_on_device
def fwd(q1, k1, q2, k2, scale: float, causal: bool):
    """Per-row (KL, LSE1, LSE2), fp32 [heads, n_q]."""
    heads, n_q, n_k, d, dt = _inputs(q1, k1, q2, k2)
    out = [torch.empty(heads, n_q, device=q1.device, dtype=torch.float32) for _ in range(3)]
    st = _lib.lib().streamkl_fwd(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), n_q, n_k, heads, d,
                                 int(causal), float(scale), dt, *(o.data_ptr() for o in out), _stream())
    _lib.check("streamkl_fwd", st)
    return tuple(out)


def splitk_workspace_bytes(n_q, n_k, heads, head_dim, num_splits=0) -> int:
    return _lib.lib().streamkl_workspace_bytes(0, n_q, n_k, heads, head_dim, num_splits, 0)


@_on_device
def fwd_splitk(q1, k1, q2, k2, scale: float, causal: bool, num_splits: int = 0, workspace=None):
    """Split-K forward; num_splits = 0 lets the library choose."""
    heads, n_q, n_k, d, dt = _inputs(q1, k1, q2, k2)
    need = splitk_workspace_bytes(n_q, n_k, heads, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q1.device, dtype=torch.uint8)
    elif workspace.device != q1.device or not workspace.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {q1.device}")
    out = [torch.empty(heads, n_q, device=q1.device, dtype=torch.float32) for _ in range(3)]
    st = _lib.lib().streamkl_fwd_splitk(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), n_q, n_k,
                                        heads, d, int(causal), float(scale), dt, int(num_splits),
                                        *(o.data_ptr() for o in out), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream())
    _lib.check("streamkl_fwd_splitk", st)
    return tuple(out)


def splitk_auto(n_q, n_k, heads, head_dim) -> int:
    return _lib.lib().streamkl_splitk_auto(n_q, n_k, heads, head_dim)


@_on_device
def fwd_auto(q1, k1, q2, k2, scale: float, causal: bool):
    """The forward the library recommends for the shape: split-K when its
    split-count heuristic (streamkl_splitk_auto) asks for more than one key
    range, which it does when the query blocks alone cannot fill the GPU
    (short query sets, decode), else the one-pass kernel.  A STREAMKL_SPLITS
    override is what the heuristic then returns, so it picks the path too."""
    heads, n_q, n_k, d, _ = _inputs(q1, k1, q2, k2)
    if splitk_auto(n_q, n_k, heads, d) > 1:
        return fwd_splitk(q1, k1, q2, k2, scale, causal)
    return fwd(q1, k1, q2, k2, scale, causal)


def bwd_select(n_q, n_k, heads, head_dim, causal) -> str:
    return {_lib.BWD_FUSED: "fused", _lib.BWD_SEPARATE: "separate"}[
        _lib.lib().streamkl_bwd_select(n_q, n_k, heads, head_dim, int(causal))]


@_on_device
def bwd(setting: int, q1, k1, q2, k2, scale: float, causal: bool, lse1, lse2, kl=None, dkl=None,
        path: str = "auto", dq=None, dk=None):
    """(dQ, dK) of the setting's tensors (Setting 1: Q2, K2; Setting 2: Q1, K1), fp32.

    path: "auto", "fused", "separate", "dk_only" (dQ not computed, returned as
    None) or "dq_only" (dK not computed).  dq / dk may be given as outputs."""
    heads, n_q, n_k, d, dt = _inputs(q1, k1, q2, k2)
    if path not in _PATH:
        raise ValueError(f"unknown path {path!r}")
    if lse1 is None or lse2 is None:
        raise ValueError("the backward needs the forward's lse1 and lse2")
    for t, name in ((lse1, "lse1"), (lse2, "lse2"), (kl, "kl"), (dkl, "dkl")):
        check_rows(t, name, heads, n_q, q1.device)
    check_out(dq, "dq", (heads, n_q, d), q1.device)
    check_out(dk, "dk", (heads, n_k, d), q1.device)
    if path != "dk_only" and dq is None:
        dq = torch.empty(heads, n_q, d, device=q1.device, dtype=torch.float32)
    if path != "dq_only" and dk is None:
        dk = torch.empty(heads, n_k, d, device=q1.device, dtype=torch.float32)
    check_disjoint((("dq", dq if path != "dk_only" else None), ("dk", dk if path != "dq_only" else None)))
    L = _lib.lib()
    common = (q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), n_q, n_k, heads, d, int(causal),
              float(scale), dt, lse1.data_ptr(), lse2.data_ptr())
    if setting == 1:
        st = L.streamkl_bwd_set1(*common, _ptr(dkl), _ptr(dq), _ptr(dk), _PATH[path], None, 0, _stream())
    elif setting == 2:
        if kl is None:
            raise ValueError("Setting 2 needs the forward's KL rows")
        st = L.streamkl_bwd_set2(*common, kl.data_ptr(), _ptr(dkl), _ptr(dq), _ptr(dk), _PATH[path],
                                 None, 0, _stream())
    else:
        raise ValueError("setting must be 1 or 2")
    _lib.check(f"streamkl_bwd_set{setting}", st)
    return dq, dk


@_on_device
def bwd_both(q1, k1, q2, k2, scale: float, causal: bool, lse1, lse2, kl, dkl=None, path: str = "auto", dq1=None,
             dk1=None, dq2=None, dk2=None):
    """(dQ1, dK1, dQ2, dK2), fp32: Setting 2's and Setting 1's gradients of the
    same loss from one recomputation.  path: "auto"/"separate" (all four),
    "dk_only" (dQ1, dQ2 returned as None) or "dq_only" (dK1, dK2 None).
    Outputs may be given."""
    heads, n_q, n_k, d, dt = _inputs(q1, k1, q2, k2)
    if path not in ("auto", "separate", "dk_only", "dq_only"):
        raise ValueError(f"unknown path {path!r}")
    if lse1 is None or lse2 is None or kl is None:
        raise ValueError("the both-settings backward needs the forward's lse1, lse2 and KL rows")
    for t, name in ((lse1, "lse1"), (lse2, "lse2"), (kl, "kl"), (dkl, "dkl")):
        check_rows(t, name, heads, n_q, q1.device)
    outs = []
    for o, name, n, want in ((dq1, "dq1", n_q, path != "dk_only"), (dk1, "dk1", n_k, path != "dq_only"),
                             (dq2, "dq2", n_q, path != "dk_only"), (dk2, "dk2", n_k, path != "dq_only")):
        check_out(o, name, (heads, n, d), q1.device)
        if o is None and want:
            o = torch.empty(heads, n, d, device=q1.device, dtype=torch.float32)
        outs.append(o if want else None)
    check_disjoint(zip(("dq1", "dk1", "dq2", "dk2"), outs))
    L = _lib.lib()
    st = L.streamkl_bwd_both(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), n_q, n_k, heads, d,
                             int(causal), float(scale), dt, lse1.data_ptr(), lse2.data_ptr(), kl.data_ptr(),
                             _ptr(dkl), *[_ptr(o) for o in outs], _PATH[path], _stream())
    _lib.check("streamkl_bwd_both", st)
    return tuple(outs)
