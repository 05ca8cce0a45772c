"""GPU backward of both settings from one recomputation (streamkl_bwd_both)
against the fp64 oracle, and against the two single-setting launches."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import device_inputs, log, need_gpu
from tests.parity import bf16_ds_bound, compare
from tests.test_gpu_backward import BWD_EDGE
from tests.test_gpu_forward import _rand_case

pytestmark = pytest.mark.gpu


def _both(dev, scale, causal, g=None):
    import torch
    import streaming_kl_divergence_amd as skl
    kl, l1, l2 = skl.fwd(*dev, scale, causal)
    dkl = None if g is None else torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).cuda()
    out = skl.bwd_both(*dev, scale, causal, l1, l2, kl, dkl=dkl)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out], (kl, l1, l2, dkl)


@pytest.mark.parametrize("with_g", [False, True])
@pytest.mark.parametrize("idx", range(len(BWD_EDGE)), ids=[str(c) for c in BWD_EDGE])
def test_edge_shapes(idx, with_g):
    need_gpu()
    case = BWD_EDGE[idx]
    heads, n_q, n_k, d, dtype, causal, sm = case
    log(f"case both {case} g={with_g}")
    arrs = _rand_case(200 + idx, heads, n_q, n_k, d, dtype, corr=(sm != 4.0))
    g = np.random.default_rng(300 + idx).uniform(0.5, 1.5, (heads, n_q)).astype(np.float32) if with_g else None
    scale = sm / np.sqrt(d)
    (dq1, dk1, dq2, dk2), _ = _both(device_inputs(arrs, dtype), scale, causal, g)
    derived = sm != 1.0 and dtype == "bf16"
    for setting, (dq, dk) in ((1, (dq2, dk2)), (2, (dq1, dk1))):
        rdq, rdk = oracle.backward(setting, *arrs, scale, causal, dkl=g)
        eq = ek = None
        if derived:
            eq, ek = bf16_ds_bound(oracle, setting, arrs, scale, causal, g)
        compare(dq, rdq, dtype, f"{case} setting {setting} dq", extra_abs=eq)
        compare(dk, rdk, dtype, f"{case} setting {setting} dk", extra_abs=ek)


@pytest.mark.parametrize("causal", [False, True])
def test_matches_single_setting_launches(causal):
    """The same per-pair arithmetic and accumulation order as the dK-only and
    dQ-only kernels of each setting: equal up to fp32 reassociation."""
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    arrs = _rand_case(23, 2, 700, 1500 if not causal else 700, 128, "bf16")
    dev = device_inputs(arrs, "bf16")
    g = np.random.default_rng(5).uniform(0.5, 1.5, (2, 700)).astype(np.float32)
    both, (kl, l1, l2, dkl) = _both(dev, 0.09, causal, g)
    for setting, ref in ((1, both[2:]), (2, both[:2])):
        kw = dict(kl=kl) if setting == 2 else {}
        dq, dk = skl.bwd(setting, *dev, 0.09, causal, l1, l2, dkl=dkl, path="separate", **kw)
        torch.cuda.synchronize()
        for a, b, n in ((ref[0], dq.cpu().numpy(), "dq"), (ref[1], dk.cpu().numpy(), "dk")):
            assert np.abs(a - b).max() <= 1e-5 * np.abs(b).max(), f"setting {setting} {n}"


def test_rejects_missing_kl():
    need_gpu()
    import streaming_kl_divergence_amd as skl
    arrs = _rand_case(24, 1, 64, 64, 64, "bf16")
    dev = device_inputs(arrs, "bf16")
    kl, l1, l2 = skl.fwd(*dev, 0.125, False)
    with pytest.raises(ValueError):
        skl.bwd_both(*dev, 0.125, False, l1, l2, None)


@pytest.mark.parametrize("causal", [False, True])
def test_identical_teacher_and_student_give_exact_zeros(causal):
    """(Q1, K1) = (Q2, K2): P1 and P2 come out of the same arithmetic, so
    dS2 = P2 - P1 and dS1 = P1 (r - KL) vanish exactly and all four gradients
    of the both-settings kernels are zero (bitwise), with and without g."""
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    log(f"case both identical inputs causal={causal}")
    rng = np.random.default_rng(78)
    q = W.round_bf16(rng.standard_normal((2, 300, 128), dtype=np.float32))
    k = W.round_bf16(rng.standard_normal((2, 500, 128), dtype=np.float32))
    dev = device_inputs([q, k, q, k], "bf16")
    kl, l1, l2 = skl.fwd(*dev, 0.09, causal)
    g = torch.from_numpy(rng.uniform(0.5, 1.5, (2, 300)).astype(np.float32)).cuda()
    for dkl in (None, g):
        out = skl.bwd_both(*dev, 0.09, causal, l1, l2, kl, dkl=dkl)
        torch.cuda.synchronize()
        for name, t in zip(("dq1", "dk1", "dq2", "dk2"), out):
            assert not bool(t.any()), f"{name} nonzero (g={'given' if dkl is not None else 'ones'})"
