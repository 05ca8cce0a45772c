"""Comparison rule for GPU results against the fp64 oracle.

Element-wise: |gpu - ref| <= abs + rel * |ref| with (rel, abs) = (2e-3, 1e-4)
for fp32 inputs and (2e-2, 2e-3) for bf16 inputs, for per-row KL, LSE and all
gradients.  Normwise guard: ||gpu - ref||_2 <= rel * ||ref||_2 per tensor, so
that a tensor whose entries are all below `abs` (long rows make gradients
small) cannot pass while being wrong, e.g. all zeros.

`extra_abs` widens the element-wise bound for cases outside the stated
workloads where a derived rounding bound is larger (see bf16_ds_bound).
"""
from __future__ import annotations

import numpy as np

TOL = {"fp32": (2e-3, 1e-4), "bf16": (2e-2, 2e-3)}


def compare(gpu, ref, dtype: str, name: str = "", normwise: bool = True, extra_abs=None) -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    rel, ab = TOL[dtype]
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite GPU values"
    err = np.abs(gpu - ref)
    bound = ab + rel * np.abs(ref)
    if extra_abs is not None:
        bound = bound + extra_abs
    bad = err > bound
    nref = np.linalg.norm(ref)
    nerr = np.linalg.norm(gpu - ref)
    stats = {"name": name, "max_abs": float(err.max()) if err.size else 0.0,
             "worst_ratio": float((err / bound).max()) if err.size else 0.0,
             "norm_rel": float(nerr / nref) if nref > 0 else float(nerr),
             "frac_above_abs": float(np.mean(np.abs(ref) > ab)) if ref.size else 0.0}
    assert not bad.any(), (f"{name}: {int(bad.sum())}/{bad.size} elements out of tolerance; "
                           f"first at {np.argwhere(bad)[0].tolist()} gpu={gpu[bad][0]!r} ref={ref[bad][0]!r}; {stats}")
    if normwise and nref > 0:
        assert nerr <= rel * nref, f"{name}: normwise error {nerr / nref:.3e} > {rel}; {stats}"
    return stats


def bf16_ds_bound(oracle, setting, arrs, scale, causal, g=None):
    """Per-element bound of the error that rounding dS to bf16 (relative error
    at most 2^-9, taken as 2^-8 to cover fp32 accumulation) puts into dQ and dK:
    |d dQ| <= 2^-8 scale |dS| |K|,  |d dK| <= 2^-8 scale |dS|^T |Q|, per head."""
    q_t, k_t = (arrs[2], arrs[3]) if setting == 1 else (arrs[0], arrs[1])
    bq, bk = [], []
    for h in range(arrs[0].shape[0]):
        ds = np.abs(oracle.dlogits_head(setting, arrs[0][h], arrs[1][h], arrs[2][h], arrs[3][h], scale, causal,
                                        None if g is None else g[h]))
        bq.append(2.0 ** -8 * scale * ds @ np.abs(k_t[h].astype(np.float64)))
        bk.append(2.0 ** -8 * scale * ds.T @ np.abs(q_t[h].astype(np.float64)))
    return np.stack(bq), np.stack(bk)
