"""GPU backward (Setting 1 and Setting 2; fused and separate paths) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import device_inputs, log, need_gpu, workload_device_inputs
from tests.parity import bf16_ds_bound, compare
from tests.test_gpu_forward import _rand_case

pytestmark = pytest.mark.gpu


def _gpu_fwd_bwd(dev, scale, causal, setting, path, g=None):
    import torch
    import streaming_kl_divergence_amd as skl
    q1, k1, q2, k2 = dev
    kl, l1, l2 = skl.fwd(q1, k1, q2, k2, scale, causal)
    dkl = None if g is None else torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).cuda()
    dq, dk = skl.bwd(setting, q1, k1, q2, k2, scale, causal, l1, l2, kl=kl, dkl=dkl, path=path)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy()


def _check_full(arrs, dtype, scale, causal, setting, path, g=None, name="", derived=False):
    dev = device_inputs(arrs, dtype)
    dq, dk = _gpu_fwd_bwd(dev, scale, causal, setting, path, g)
    rdq, rdk = oracle.backward(setting, *arrs, scale, causal, dkl=g)
    eq = ek = None
    if derived:
        eq, ek = bf16_ds_bound(oracle, setting, arrs, scale, causal, g)
    compare(dq, rdq, dtype, f"{name} dq", extra_abs=eq)
    compare(dk, rdk, dtype, f"{name} dk", extra_abs=ek)
    return dq, dk


@pytest.mark.parametrize("path", ["separate", "fused"])
@pytest.mark.parametrize("setting", [1, 2])
def test_tiny_fp32_config(setting, path):
    need_gpu()
    w = W.WORKLOADS["tiny"]
    log(f"case tiny setting={setting} path={path}")
    _check_full(W.all_inputs(w), "fp32", w.scale, w.causal, setting, path, name="tiny")


BWD_EDGE = [
    # (heads, n_q, n_k, d, dtype, causal, scale_mult)
    (2, 1000, 1000, 128, "bf16", True, 1.0),
    (2, 257, 1000, 128, "bf16", False, 1.0),
    (2, 300, 1000, 128, "bf16", True, 1.0),
    (3, 200, 333, 64, "bf16", True, 1.0),
    (2, 130, 190, 64, "fp32", True, 1.0),
    (2, 100, 150, 128, "fp32", False, 1.0),
    (4, 1, 777, 128, "bf16", False, 1.0),
    (2, 70, 1, 128, "bf16", False, 1.0),
    (2, 400, 900, 128, "bf16", True, 4.0),
    (1, 128, 128, 128, "bf16", True, 1.0),
    (2, 200, 300, 128, "bf16", True, 0.0),    # scale 0: uniform rows, zero gradients
    (2, 300, 3000, 128, "bf16", True, 1.0),   # few query blocks, long keys: dQ over 3 key ranges, causal
    (3, 257, 4100, 64, "bf16", False, 1.0),   # dQ over 5 key ranges, ragged tail
]


@pytest.mark.parametrize("path", ["separate", "fused"])
@pytest.mark.parametrize("setting", [1, 2])
@pytest.mark.parametrize("idx", range(len(BWD_EDGE)), ids=[str(c) for c in BWD_EDGE])
def test_edge_shapes(idx, setting, path):
    need_gpu()
    case = BWD_EDGE[idx]
    heads, n_q, n_k, d, dtype, causal, sm = case
    log(f"case {case} setting={setting} path={path}")
    arrs = _rand_case(200 + idx, heads, n_q, n_k, d, dtype, corr=(sm != 4.0))
    g = np.random.default_rng(300 + idx).uniform(0.5, 1.5, (heads, n_q)).astype(np.float32)
    # logits 4x the standard scale: outside the stated workloads, the bound adds
    # the derived bf16-dS rounding term (tests/parity.py, bf16_ds_bound)
    dq, dk = _check_full(arrs, dtype, sm / np.sqrt(d), causal, setting, path, g=g, name=str(case),
                         derived=(sm != 1.0 and dtype == "bf16"))
    # each row of dS sums to zero, so sum_j dK_j = 0 (per head)
    assert np.abs(dk.sum(1)).max() <= 1e-3 * max(1e-6, np.abs(dk).max()) * n_k ** 0.5 + 1e-5


def test_paths_agree():
    need_gpu()
    arrs = _rand_case(21, 2, 700, 1500, 128, "bf16")
    dev = device_inputs(arrs, "bf16")
    for setting in (1, 2):
        a = _gpu_fwd_bwd(dev, 0.09, True, setting, "separate")
        b = _gpu_fwd_bwd(dev, 0.09, True, setting, "fused")
        for x, y in zip(a, b):
            assert np.linalg.norm(x - y) <= 5e-3 * np.linalg.norm(x)


def test_single_gradient_paths():
    """DK_ONLY then DQ_ONLY equals SEPARATE, and each leaves the other gradient untouched."""
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    arrs = _rand_case(22, 2, 300, 1100, 128, "bf16")
    dev = device_inputs(arrs, "bf16")
    kl, l1, l2 = skl.fwd(*dev, 0.09, True)
    for setting in (1, 2):
        ref_q, ref_k = skl.bwd(setting, *dev, 0.09, True, l1, l2, kl=kl, path="separate")
        sentinel = torch.full_like(ref_q, 7.0)
        dq, dk = skl.bwd(setting, *dev, 0.09, True, l1, l2, kl=kl, path="dk_only", dq=sentinel)
        assert torch.equal(dq, torch.full_like(ref_q, 7.0)) and torch.equal(dk, ref_k)
        sentinel = torch.full_like(ref_k, 7.0)
        dq, dk = skl.bwd(setting, *dev, 0.09, True, l1, l2, kl=kl, path="dq_only", dk=sentinel)
        assert torch.equal(dk, torch.full_like(ref_k, 7.0)) and torch.equal(dq, ref_q)


def test_causal8k_setting1_config():
    """32 heads, 8K causal bf16 correlated, Setting 1: heads 0 and 31 in full
    against the oracle; every head checked for sum_j dK_j = 0 and
    sum_i q_i . dQ_i = sum_j k_j . dK_j."""
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    w = W.WORKLOADS["causal8k"]
    log(f"case {w} setting=1")
    dev = workload_device_inputs(w)
    dq, dk = _gpu_fwd_bwd(dev, w.scale, w.causal, 1, "auto")
    for h in (0, w.heads - 1):
        a = W.head_inputs(w, h)
        rdq, rdk = oracle.backward_head(1, *a, w.scale, w.causal)
        compare(dq[h], rdq, "bf16", f"h{h} dq2")
        compare(dk[h], rdk, "bf16", f"h{h} dk2")
    q2 = dev[2].float().cpu().numpy()
    k2 = dev[3].float().cpu().numpy()
    lhs = np.einsum("hid,hid->h", q2.astype(np.float64), dq.astype(np.float64))
    rhs = np.einsum("hjd,hjd->h", k2.astype(np.float64), dk.astype(np.float64))
    scale_ref = np.abs(q2).mean() * np.abs(dq).sum(axis=(1, 2))
    assert np.all(np.abs(lhs - rhs) <= 2e-2 * scale_ref)
    colsum = np.abs(dk.astype(np.float64).sum(1))
    assert np.all(colsum <= 2e-2 * np.abs(dk).sum(1) / np.sqrt(w.n_k) + 1e-6)


def test_smallq128k_setting2_paths():
    """512 queries x 128K keys, 32 heads, Setting 2: fused and separate, heads 0
    and 31 against the oracle (all dQ rows, sampled dK rows)."""
    need_gpu()
    w = W.WORKLOADS["smallq128k"]
    log(f"case {w} setting=2")
    dev = workload_device_inputs(w)
    res = {path: _gpu_fwd_bwd(dev, w.scale, w.causal, 2, path) for path in ("fused", "separate")}
    keys = np.unique(np.concatenate([np.arange(40), w.n_k - 1 - np.arange(40),
                                     np.random.default_rng(8).integers(0, w.n_k, 300)]))
    for h in (0, w.heads - 1):
        a = W.head_inputs(w, h)
        rdq = oracle.dq_rows(2, *a, w.scale, w.causal, np.arange(w.n_q))
        rdk = oracle.dk_keys(2, *a, w.scale, w.causal, keys)
        for path, (dq, dk) in res.items():
            compare(dq[h], rdq, "bf16", f"{path} h{h} dq1")
            compare(dk[h, keys], rdk, "bf16", f"{path} h{h} dk1")


@pytest.mark.parametrize("path", ["separate", "fused"])
@pytest.mark.parametrize("causal", [False, True])
def test_identical_teacher_and_student_give_exact_zeros(causal, path):
    """(Q1, K1) = (Q2, K2): both distributions go through the same arithmetic,
    so KL and every gradient of both settings are exactly zero (bitwise)."""
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    log(f"case identical inputs causal={causal} path={path}")
    rng = np.random.default_rng(77)
    q = W.round_bf16(rng.standard_normal((2, 300, 128), dtype=np.float32))
    k = W.round_bf16(rng.standard_normal((2, 500, 128), dtype=np.float32))
    q1, k1, q2, k2 = device_inputs([q, k, q, k], "bf16")
    kl, l1, l2 = skl.fwd(q1, k1, q2, k2, 0.09, causal)
    assert torch.equal(kl, torch.zeros_like(kl)) and torch.equal(l1, l2)
    for setting in (1, 2):
        kw = dict(kl=kl) if setting == 2 else {}
        dq, dk = skl.bwd(setting, q1, k1, q2, k2, 0.09, causal, l1, l2, path=path, **kw)
        torch.cuda.synchronize()
        assert not bool(dq.any()) and not bool(dk.any()), f"setting {setting}: nonzero gradient"
