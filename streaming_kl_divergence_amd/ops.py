"""Torch-facing wrappers over the C ABI.  Every step runs in the HIP library;
these functions only check tensors, allocate outputs with torch and pass
pointers and the current stream."""
from __future__ import annotations

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
    if len({q1.dtype, k1.dtype, q2.dtype, k2.dtype}) != 1 or q1.dtype not in _DT:
        raise ValueError("inputs must share one dtype: bfloat16 or float32")
    heads, n_q, d = q1.shape
    n_k = k1.shape[1]
    if q2.shape != q1.shape or k1.shape != (heads, n_k, d) or k2.shape != k1.shape:
        raise ValueError("shape mismatch between Q1, K1, Q2, K2")
    return heads, n_q, n_k, d, _DT[q1.dtype]


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


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


def fwd_splitk(q1, k1, q2, k2, scale: float, causal: bool, num_splits: int = 0, workspace=None):
    """Split-K forward; num_splits = 0 lets the library choose."""
    heads, n_q, n_k, d, dt = _inputs(q1, k1, q2, k2)
    need = splitk_workspace_bytes(n_q, n_k, heads, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), device=q1.device, dtype=torch.uint8)
    out = [torch.empty(heads, n_q, device=q1.device, dtype=torch.float32) for _ in range(3)]
    st = _lib.lib().streamkl_fwd_splitk(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), n_q, n_k,
                                        heads, d, int(causal), float(scale), dt, int(num_splits),
                                        *(o.data_ptr() for o in out), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), _stream())
    _lib.check("streamkl_fwd_splitk", st)
    return tuple(out)


def splitk_auto(n_q, n_k, heads, head_dim) -> int:
    return _lib.lib().streamkl_splitk_auto(n_q, n_k, heads, head_dim)


def bwd_select(n_q, n_k, heads, head_dim, causal) -> str:
    return {_lib.BWD_FUSED: "fused", _lib.BWD_SEPARATE: "separate"}[
        _lib.lib().streamkl_bwd_select(n_q, n_k, heads, head_dim, int(causal))]


def bwd(setting: int, q1, k1, q2, k2, scale: float, causal: bool, lse1, lse2, kl=None, dkl=None,
        path: str = "auto", dq=None, dk=None):
    """(dQ, dK) of the setting's tensors (Setting 1: Q2, K2; Setting 2: Q1, K1), fp32.

    path: "auto", "fused", "separate", "dk_only" (dQ not computed, returned as
    None) or "dq_only" (dK not computed).  dq / dk may be given as outputs."""
    heads, n_q, n_k, d, dt = _inputs(q1, k1, q2, k2)
    if path not in _PATH:
        raise ValueError(f"unknown path {path!r}")
    if path != "dk_only" and dq is None:
        dq = torch.empty(heads, n_q, d, device=q1.device, dtype=torch.float32)
    if path != "dq_only" and dk is None:
        dk = torch.empty(heads, n_k, d, device=q1.device, dtype=torch.float32)
    for t in (lse1, lse2, kl, dkl):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.shape != (heads, n_q)):
            raise ValueError("lse1, lse2, kl, dkl must be contiguous fp32 [heads, n_q]")
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


def bwd_both(q1, k1, q2, k2, scale: float, causal: bool, lse1, lse2, kl, dkl=None, path: str = "auto", dq1=None,
             dk1=None, dq2=None, dk2=None):
    """(dQ1, dK1, dQ2, dK2), fp32: Setting 2's and Setting 1's gradients of the
    same loss from one recomputation.  path: "auto"/"separate" (all four),
    "dk_only" (dQ1, dQ2 returned as None) or "dq_only" (dK1, dK2 None).
    Outputs may be given."""
    heads, n_q, n_k, d, dt = _inputs(q1, k1, q2, k2)
    if path not in ("auto", "separate", "dk_only", "dq_only"):
        raise ValueError(f"unknown path {path!r}")
    for t in (lse1, lse2, kl, dkl):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.shape != (heads, n_q)):
            raise ValueError("lse1, lse2, kl, dkl must be contiguous fp32 [heads, n_q]")
    if kl is None:
        raise ValueError("the both-settings backward needs the forward's KL rows")
    outs = []
    for o, n, want in ((dq1, n_q, path != "dk_only"), (dk1, n_k, path != "dq_only"),
                       (dq2, n_q, path != "dk_only"), (dk2, n_k, path != "dq_only")):
        if o is None and want:
            o = torch.empty(heads, n, d, device=q1.device, dtype=torch.float32)
        outs.append(o if want else None)
    L = _lib.lib()
    st = L.streamkl_bwd_both(q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), n_q, n_k, heads, d,
                             int(causal), float(scale), dt, lse1.data_ptr(), lse2.data_ptr(), kl.data_ptr(),
                             _ptr(dkl), *[_ptr(o) for o in outs], _PATH[path], _stream())
    _lib.check("streamkl_bwd_both", st)
    return tuple(outs)
