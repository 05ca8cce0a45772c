"""The comparison rule must reject wrong answers that a plain element-wise
tolerance would let through on long rows.  CPU only.

At 4096 keys, causal, with the correlated student of the long-context
workloads, about half of the gradient entries are below the bf16 absolute
tolerance (2e-3), and gradient entries shrink as rows get longer.
``tests/parity.compare`` (element-wise bound plus the normwise guard) must
reject an all-zero gradient, the gradients of the other setting, and per-row
KL values that leave out the LSE terms of the pages' row loss
(acc / l1 + LSE2 - LSE1; StreamKL gist.science technical summary,
Methodology 1).  The zero gradient must also fail the normwise guard by
itself.  A correct answer carrying bf16-sized rounding noise must still pass,
so the rule is not vacuous.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.parity import compare

N = 4096


@pytest.fixture(scope="module")
def case():
    w = W.WORKLOADS["causal8k"].replace(heads=1, n_q=N, n_k=N)
    a = [x.astype(np.float64) for x in W.head_inputs(w, 0)]
    kl, l1, l2 = oracle.forward_head(*a, w.scale, True)
    grads = {s: oracle.backward_head(s, *a, w.scale, True) for s in (1, 2)}
    return w, a, (kl, l1, l2), grads


def _rejects(gpu, ref, name):
    with pytest.raises(AssertionError):
        compare(gpu, ref, "bf16", name)


@pytest.mark.parametrize("setting", [1, 2])
def test_rejects_all_zero_gradients(case, setting):
    _, _, _, grads = case
    for g, name in zip(grads[setting], ("dq", "dk")):
        _rejects(np.zeros_like(g), g, f"zero {name}")
        # the guard alone: entries below the absolute tolerance zeroed and the
        # rest 3% short is within the element-wise bound everywhere (every
        # |g| here is far below 0.2), so only the normwise guard can reject it
        with pytest.raises(AssertionError, match="normwise"):
            compare(np.where(np.abs(g) <= 2e-3, 0.0, g * 0.97), g, "bf16", f"{name} small entries zeroed")


def test_rejects_swapped_settings(case):
    _, _, _, grads = case
    for i, name in enumerate(("dq", "dk")):
        _rejects(grads[1][i], grads[2][i], f"setting 1 {name} as setting 2")
        _rejects(grads[2][i], grads[1][i], f"setting 2 {name} as setting 1")


def test_rejects_kl_without_lse_terms(case):
    _, _, (kl, l1, l2), _ = case
    # sum_j P1 (S1 - S2), i.e. the row loss without LSE2 - LSE1
    _rejects(kl - (l2 - l1), kl, "kl without lse")


def test_accepts_bf16_sized_noise(case):
    """A correct answer with relative noise of a few bf16 ulps still passes."""
    _, _, (kl, l1, l2), grads = case
    rng = np.random.default_rng(5)
    for x, name in ((kl, "kl"), (l1, "lse1"), (l2, "lse2"), *((g, f"s{s} grad") for s in (1, 2) for g in grads[s])):
        noisy = x * (1 + 4e-3 * rng.standard_normal(x.shape))
        compare(noisy, x, "bf16", name)
