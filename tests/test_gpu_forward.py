"""GPU forward (fused one-pass and split-K) against the fp64 oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_util import device_inputs, log, need_gpu, workload_device_inputs
from tests.parity import compare

pytestmark = pytest.mark.gpu


def _run_fwd(arrs, dtype, scale, causal, splits=None):
    import torch
    import streaming_kl_divergence_amd as skl
    q1, k1, q2, k2 = device_inputs(arrs, dtype)
    if splits is None:
        out = skl.fwd(q1, k1, q2, k2, scale, causal)
    else:
        out = skl.fwd_splitk(q1, k1, q2, k2, scale, causal, num_splits=splits)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def _check_all_rows(arrs, dtype, scale, causal, splits=None, name=""):
    kl, l1, l2 = _run_fwd(arrs, dtype, scale, causal, splits)
    rkl, rl1, rl2 = oracle.forward(*arrs, scale, causal)
    compare(l1, rl1, dtype, name + " lse1")
    compare(l2, rl2, dtype, name + " lse2")
    compare(kl, rkl, dtype, name + " kl", normwise=bool(np.abs(rkl).max() > 0))
    return kl, rkl


def test_tiny_fp32_config():
    need_gpu()
    w = W.WORKLOADS["tiny"]
    log(f"case {w}")
    _check_all_rows(W.all_inputs(w), "fp32", w.scale, w.causal, name="tiny")


def _rand_case(seed, heads, n_q, n_k, d, dtype, corr=True):
    rng = np.random.default_rng(seed)
    q1 = rng.standard_normal((heads, n_q, d), dtype=np.float32)
    k1 = rng.standard_normal((heads, n_k, d), dtype=np.float32)
    q2 = rng.standard_normal((heads, n_q, d), dtype=np.float32)
    k2 = rng.standard_normal((heads, n_k, d), dtype=np.float32)
    if corr:
        q2 = q1 + np.float32(0.3) * q2
        k2 = k1 + np.float32(0.3) * k2
    arrs = [q1, k1, q2, k2]
    if dtype == "bf16":
        arrs = [W.round_bf16(a) for a in arrs]
    return arrs


EDGE = [
    # (heads, n_q, n_k, d, dtype, causal, scale_mult)
    (2, 1000, 1000, 128, "bf16", True, 1.0),     # ragged tails, causal, several tiles
    (2, 257, 1000, 128, "bf16", False, 1.0),     # ragged, non-causal, n_q != n_k
    (2, 300, 1000, 128, "bf16", True, 1.0),      # causal bottom-right, n_q < n_k
    (3, 200, 333, 64, "bf16", True, 1.0),        # d = 64
    (2, 130, 190, 64, "fp32", True, 1.0),        # fp32 causal
    (2, 100, 150, 128, "fp32", False, 1.0),      # fp32 d = 128
    (4, 1, 777, 128, "bf16", False, 1.0),        # one query
    (4, 1, 777, 128, "bf16", True, 1.0),         # one query, causal = full row
    (2, 70, 1, 128, "bf16", False, 1.0),         # one key: KL = 0
    (2, 500, 640, 128, "bf16", False, 0.0),      # scale 0: uniform rows, KL = 0
    (2, 400, 900, 128, "bf16", True, 4.0),       # large logits (4 / sqrt(d))
    (1, 64, 64, 128, "bf16", True, 1.0),         # exactly one tile
    (2, 32, 3000, 128, "bf16", False, 1.0),      # one-wave workgroups, many key tiles
    (3, 17, 2049, 64, "bf16", True, 1.0),        # one-wave, causal bottom-right, ragged
    (2, 5, 40, 128, "bf16", False, 1.0),         # one-wave, a single partial key tile
    (2, 1, 300, 64, "fp32", False, 1.0),         # one query, fp32
    (3, 1, 1, 128, "bf16", True, 1.0),           # one query, one key
]


@pytest.mark.parametrize("idx", range(len(EDGE)), ids=[str(c) for c in EDGE])
def test_edge_shapes(idx):
    need_gpu()
    case = EDGE[idx]
    heads, n_q, n_k, d, dtype, causal, sm = case
    log(f"case {case}")
    arrs = _rand_case(100 + idx, heads, n_q, n_k, d, dtype, corr=(sm != 4.0))
    _check_all_rows(arrs, dtype, sm / np.sqrt(d), causal, name=str(case))


def _drift_case(seed, heads, n_q, n_k, d, rising: bool):
    """Logits that drift along the keys by about 256 binary orders over a row
    (queries near 8u, keys near ramp_j * u for a random unit u): rising, every
    few tiles a score exceeds the running offset by more than 2^64, so the
    forward must raise its offsets mid-row; falling, later tiles underflow."""
    rng = np.random.default_rng(seed)
    d_ = np.float32
    arrs = [np.empty((heads, n, d), dtype=np.float32) for n in (n_q, n_k, n_q, n_k)]
    for h in range(heads):
        u = rng.standard_normal(d).astype(d_)
        u /= np.linalg.norm(u)
        t = np.arange(n_k, dtype=d_) / n_k
        ramp = d_(251.0) * (t if rising else 1 - t)
        q1 = 8 * u + d_(0.5) * rng.standard_normal((n_q, d), dtype=d_)
        k1 = ramp[:, None] * u + d_(0.5) * rng.standard_normal((n_k, d), dtype=d_)
        arrs[0][h], arrs[1][h] = q1, k1
        arrs[2][h] = q1 + d_(0.3) * rng.standard_normal((n_q, d), dtype=d_)
        arrs[3][h] = k1 + d_(0.3) * rng.standard_normal((n_k, d), dtype=d_)
    return [W.round_bf16(a) for a in arrs]


@pytest.mark.parametrize("rising,causal", [(True, False), (True, True), (False, True)])
def test_drifting_logits(rising, causal):
    need_gpu()
    log(f"case drifting logits rising={rising} causal={causal}")
    arrs = _drift_case(14 + 2 * rising + causal, 2, 96, 2048, 128, rising)
    _check_all_rows(arrs, "bf16", 1 / np.sqrt(128), causal, name=f"drift rising={rising} causal={causal}")


@pytest.mark.parametrize("splits", [1, 2, 7, 0])
def test_splitk_matches_oracle(splits):
    need_gpu()
    log(f"case splitk splits={splits}")
    arrs = _rand_case(11, 3, 37, 3000, 128, "bf16", corr=False)
    _check_all_rows(arrs, "bf16", 1 / np.sqrt(128), False, splits=splits, name=f"splits={splits}")
    arrs = _rand_case(12, 2, 200, 1000, 128, "bf16")
    _check_all_rows(arrs, "bf16", 1 / np.sqrt(128), True, splits=splits, name=f"causal splits={splits}")
    # one-wave workgroups: key ranges of a few tiles each, the last one ragged
    arrs = _rand_case(15, 2, 8, 3001, 128, "bf16")
    for causal in (False, True):
        _check_all_rows(arrs, "bf16", 1 / np.sqrt(128), causal, splits=splits, name=f"8 queries causal={causal} splits={splits}")


def test_splitk_equals_fused():
    """Every split count gives the same rows as the one-pass kernel (to fp32 rounding)."""
    need_gpu()
    arrs = _rand_case(13, 2, 33, 5000, 128, "bf16", corr=False)
    base = _run_fwd(arrs, "bf16", 0.09, False)
    for s in (1, 3, 16, 0):
        got = _run_fwd(arrs, "bf16", 0.09, False, splits=s)
        for a, b in zip(got, base):
            assert np.allclose(a, b, rtol=1e-4, atol=1e-5), s


def test_causal8k_config():
    """32 heads, 8K causal bf16 correlated: heads 0 and 31 in full, sampled rows of the rest."""
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    w = W.WORKLOADS["causal8k"]
    log(f"case {w}")
    q1, k1, q2, k2 = workload_device_inputs(w)
    kl, l1, l2 = [o.cpu().numpy() for o in skl.fwd(q1, k1, q2, k2, w.scale, w.causal)]
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    for h in range(w.heads):
        a = W.head_inputs(w, h)
        if h in (0, w.heads - 1):
            rows = np.arange(w.n_q)
        else:
            rows = np.unique(np.concatenate([np.arange(70), w.n_q - 1 - np.arange(70),
                                             rng.integers(0, w.n_q, 200), [127, 128, 129, 4095, 4096]]))
        rkl, rl1, rl2 = oracle.forward_head(*a, w.scale, w.causal, rows)
        compare(kl[h, rows], rkl, "bf16", f"h{h} kl")
        compare(l1[h, rows], rl1, "bf16", f"h{h} lse1")
        compare(l2[h, rows], rl2, "bf16", f"h{h} lse2")


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("splits", [None, 4])
def test_non_finite_inputs_stay_in_their_rows(splits):
    """One NaN row of Q1 (head 0) and one infinite entry of K2 (head 1, key
    500): every row whose scores are all finite still matches the oracle, in
    particular the other queries that share a wave with the NaN row, and the
    rows that see a non-finite score come out non-finite, as the oracle's do."""
    need_gpu()
    heads, n_q, n_k, d = 2, 300, 700, 128
    log(f"case non-finite inputs, {heads}x{n_q}x{n_k} d={d} causal, splits={splits}")
    arrs = _rand_case(77, heads, n_q, n_k, d, "bf16")
    arrs[0][0, 37, :] = np.nan
    arrs[3][1, 500, 5] = np.inf
    scale = 1 / np.sqrt(d)
    kl, l1, l2 = _run_fwd(arrs, "bf16", scale, True, splits)
    rkl, rl1, rl2 = oracle.forward(*arrs, scale, True)
    bad = ~(np.isfinite(rkl) & np.isfinite(rl1) & np.isfinite(rl2))
    # the rows the planted values reach: row 37 of head 0; head 1's rows that see key 500
    expect = np.zeros_like(bad)
    expect[0, 37] = True
    expect[1, 500 - (n_k - n_q):] = True
    assert np.array_equal(bad, expect)
    got_bad = ~(np.isfinite(kl) & np.isfinite(l1) & np.isfinite(l2))
    assert np.array_equal(got_bad, expect), np.argwhere(got_bad != expect)[:10].tolist()
    ok = ~expect
    compare(l1[ok], rl1[ok], "bf16", "finite rows lse1")
    compare(l2[ok], rl2[ok], "bf16", "finite rows lse2")
    compare(kl[ok], rkl[ok], "bf16", "finite rows kl")
