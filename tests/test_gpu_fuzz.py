"""Seeded random shapes through every entry point (forward, split-K, both
backward settings on both paths, both settings at once) against the fp64
oracle: head count, query and key counts (a quarter of the cases with few
queries against 1K-5K keys, where the dQ kernels split the keys into
ranges), head_dim, dtype, mask, student correlation, upstream weights and
split count drawn per case."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import device_inputs, log, need_gpu
from tests.parity import compare
from tests.test_gpu_forward import _rand_case

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        dtype = "fp32" if rng.random() < 0.25 else "bf16"
        heads = int(rng.integers(1, 4))
        n_k = int(rng.integers(1, 700))
        if rng.random() < 0.25:
            # few queries against long keys: the dQ kernel splits the keys into ranges
            n_k = int(rng.integers(1024, 5000))
        causal = bool(rng.random() < 0.5)
        n_q = int(rng.integers(1, min(n_k, 400) + 1)) if causal else int(rng.integers(1, 400))
        corr = bool(rng.random() < 0.7)
        splits = int(rng.integers(0, 9))
        out.append((i, heads, n_q, n_k, d, dtype, causal, corr, splits))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-h{c[1]}-q{c[2]}-k{c[3]}-d{c[4]}-{c[5]}-{'c' if c[6] else 'n'}"
                                             for c in CASES])
def test_random_shape(case):
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    i, heads, n_q, n_k, d, dtype, causal, corr, splits = case
    log(f"case fuzz {case}")
    arrs = _rand_case(1000 + i, heads, n_q, n_k, d, dtype, corr=corr)
    scale = 1 / np.sqrt(d)
    dev = device_inputs(arrs, dtype)
    host = lambda t: t.cpu().numpy()

    rkl, rl1, rl2 = oracle.forward(*arrs, scale, causal)
    kl, l1, l2 = skl.fwd(*dev, scale, causal)
    ksp = skl.fwd_splitk(*dev, scale, causal, num_splits=splits)
    for tag, (a, b, c) in (("fwd", (kl, l1, l2)), (f"splitk {splits}", ksp)):
        compare(host(b), rl1, dtype, f"{tag} lse1")
        compare(host(c), rl2, dtype, f"{tag} lse2")
        compare(host(a), rkl, dtype, f"{tag} kl", normwise=bool(np.abs(rkl).max() > 0))

    g = np.random.default_rng(2000 + i).uniform(0.5, 1.5, (heads, n_q)).astype(np.float32)
    dkl = torch.from_numpy(g).cuda()
    ref = {s: oracle.backward(s, *arrs, scale, causal, dkl=g) for s in (1, 2)}
    for setting in (1, 2):
        rdq, rdk = ref[setting]
        for path in ("separate", "fused"):
            dq, dk = skl.bwd(setting, *dev, scale, causal, l1, l2, kl=kl if setting == 2 else None, dkl=dkl,
                             path=path)
            compare(host(dq), rdq, dtype, f"set{setting} {path} dq")
            compare(host(dk), rdk, dtype, f"set{setting} {path} dk")
    dq1, dk1, dq2, dk2 = skl.bwd_both(*dev, scale, causal, l1, l2, kl, dkl=dkl)
    for name, got, want in (("dq2", dq2, ref[1][0]), ("dk2", dk2, ref[1][1]), ("dq1", dq1, ref[2][0]),
                            ("dk1", dk1, ref[2][1])):
        compare(host(got), want, dtype, f"both {name}")
