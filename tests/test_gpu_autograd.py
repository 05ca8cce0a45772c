"""The autograd wrapper (attention_kl) on the GPU against the fp64 oracle:
per-row KL, and the gradients each setting routes to each tensor under an
upstream weight g, with frozen sides left without gradients."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import log, need_gpu
from tests.parity import compare
from tests.test_gpu_forward import _rand_case

pytestmark = pytest.mark.gpu


def _leaves(arrs, dtype, req):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return [torch.from_numpy(np.ascontiguousarray(a)).to(tdt).cuda().requires_grad_(r) for a, r in zip(arrs, req)]


CASES = [
    # (setting, requires_grad of q1, k1, q2, k2, dtype, causal)
    ("student", (False, False, True, True), "fp32", True),
    ("student", (True, True, True, True), "bf16", False),     # teacher tensors frozen by the setting
    ("student", (False, False, False, True), "bf16", True),   # only dK2 wanted: the dK-only launch
    ("teacher", (True, True, False, False), "fp32", False),
    ("teacher", (True, False, True, True), "bf16", True),     # only dQ1 of the teacher: the dQ-only launch
    ("both", (True, True, True, True), "fp32", True),
]


@pytest.mark.parametrize("idx", range(len(CASES)), ids=[f"{c[0]}-{c[2]}-{c[3]}-{''.join('1' if r else '0' for r in c[1])}"
                                                        for c in CASES])
def test_attention_kl_autograd(idx):
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    setting, req, dtype, causal = CASES[idx]
    log(f"case autograd {CASES[idx]}")
    heads, n_q, n_k, d = 2, 150, 230, 64
    arrs = _rand_case(400 + idx, heads, n_q, n_k, d, dtype)
    g = np.random.default_rng(500 + idx).uniform(0.5, 1.5, (heads, n_q)).astype(np.float32)
    scale = 1 / np.sqrt(d)
    t = _leaves(arrs, dtype, req)
    kl = skl.attention_kl(*t, scale=scale, causal=causal, setting=setting)
    (kl * torch.from_numpy(g).cuda()).sum().backward()
    torch.cuda.synchronize()
    rkl, _, _ = oracle.forward(*arrs, scale, causal)
    compare(kl.detach().cpu().numpy(), rkl, dtype, "kl")
    want = {0: setting in ("teacher", "both"), 1: setting in ("teacher", "both"),
            2: setting in ("student", "both"), 3: setting in ("student", "both")}
    ref = {}
    if setting in ("student", "both"):
        ref[2], ref[3] = oracle.backward(1, *arrs, scale, causal, dkl=g)
    if setting in ("teacher", "both"):
        ref[0], ref[1] = oracle.backward(2, *arrs, scale, causal, dkl=g)
    names = ["q1", "k1", "q2", "k2"]
    for i, tt in enumerate(t):
        if want[i] and req[i]:
            assert tt.grad is not None, names[i]
            assert tt.grad.dtype == tt.dtype
            # bf16 leaves receive the fp32 gradient rounded once more to bf16
            compare(tt.grad.float().cpu().numpy(), ref[i], dtype, f"grad {names[i]}")
        else:
            assert tt.grad is None, f"{names[i]} should get no gradient in setting {setting}"


@pytest.mark.parametrize("causal", [False, True])
def test_attention_kl_short_queries_take_split_k(causal):
    """40 queries against 3000 keys: too few query blocks to fill the GPU, so
    the forward runs split-K (bitwise what fwd_splitk returns) and the loss and
    all four gradients still match the oracle."""
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    heads, n_q, n_k, d, dtype = 2, 40, 3000, 128, "bf16"
    log(f"case autograd short queries causal={causal}")
    assert skl.splitk_auto(n_q, n_k, heads, d) > 1
    arrs = _rand_case(450 + int(causal), heads, n_q, n_k, d, dtype)
    g = np.random.default_rng(550).uniform(0.5, 1.5, (heads, n_q)).astype(np.float32)
    scale = 1 / np.sqrt(d)
    t = _leaves(arrs, dtype, (True, True, True, True))
    kl = skl.attention_kl(*t, scale=scale, causal=causal, setting="both")
    ksp, _, _ = skl.fwd_splitk(*(x.detach() for x in t), scale, causal)
    assert torch.equal(kl.detach(), ksp)
    (kl * torch.from_numpy(g).cuda()).sum().backward()
    torch.cuda.synchronize()
    rkl, _, _ = oracle.forward(*arrs, scale, causal)
    compare(kl.detach().cpu().numpy(), rkl, dtype, "kl")
    ref = dict(zip((2, 3), oracle.backward(1, *arrs, scale, causal, dkl=g)))
    ref.update(zip((0, 1), oracle.backward(2, *arrs, scale, causal, dkl=g)))
    for i, name in enumerate(("q1", "k1", "q2", "k2")):
        compare(t[i].grad.float().cpu().numpy(), ref[i], dtype, f"grad {name}")


def test_attention_kl_rejects_unknown_setting():
    import streaming_kl_divergence_amd as skl
    with pytest.raises(ValueError):
        skl.attention_kl(None, None, None, None, scale=1.0, setting="neither")
