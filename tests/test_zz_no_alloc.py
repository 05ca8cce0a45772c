"""The split-K forward that allocates nothing (streamkl_fwd_splitk_noalloc),
through the C ABI, against the split-K forward with a caller workspace
(streamkl_fwd_splitk) and against the fp64 oracle: two calls in a row, the
second on a smaller input, each equal bit for bit to the workspace call with
the same split count (same kernels, same order of operations), and neither
changing device free memory.  (That a call too large for the fixed scratch is
refused before anything runs is checked on the CPU, tests/test_boundary.py.)"""
import numpy as np
import pytest

import oracle
from tests.gpu_util import device_inputs, log, need_gpu
from tests.parity import compare

pytestmark = pytest.mark.gpu


def _case(seed, heads, n_q, n_k, d):
    rng = np.random.default_rng(seed)
    import workloads as W
    a = [W.round_bf16(rng.standard_normal((heads, n, d), dtype=np.float32)) for n in (n_q, n_k, n_q, n_k)]
    return a


def _call_both(L, lib, arrs, n_q, n_k, heads, d, causal, splits):
    import torch
    q1, k1, q2, k2 = device_inputs(arrs, "bf16")
    scale = 1 / np.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    args = (q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), n_q, n_k, heads, d, int(causal), scale,
            L.BF16, splits)
    a = [torch.empty(heads, n_q, device="cuda") for _ in range(3)]
    b = [torch.empty(heads, n_q, device="cuda").fill_(float("nan")) for _ in range(3)]
    need = lib.streamkl_workspace_bytes(0, n_q, n_k, heads, d, splits, 0)
    assert 0 < need <= L.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    assert lib.streamkl_fwd_splitk(*args, *(t.data_ptr() for t in a), ws.data_ptr(), need, stream) == 0
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    assert lib.streamkl_fwd_splitk_noalloc(*args, *(t.data_ptr() for t in b), stream) == 0
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0
    return [t.cpu().numpy() for t in a], [t.cpu().numpy() for t in b]


def test_noalloc_matches_workspace_call_twice_then_smaller():
    need_gpu()
    from streaming_kl_divergence_amd import _lib as L
    lib = L.lib()
    cases = [  # (heads, n_q, n_k, d, causal, splits): the second one smaller
        (8, 200, 6000, 128, True, 0),
        (3, 5, 1500, 64, False, 7),
    ]
    for i, (heads, n_q, n_k, d, causal, splits) in enumerate(cases):
        log(f"case noalloc call {i}: heads={heads} n_q={n_q} n_k={n_k} d={d} causal={causal} splits={splits}")
        arrs = _case(100 + i, heads, n_q, n_k, d)
        ref, got = _call_both(L, lib, arrs, n_q, n_k, heads, d, causal, splits)
        for r, g, name in zip(ref, got, ("kl", "lse1", "lse2")):
            assert np.array_equal(r.view(np.uint32), g.view(np.uint32)), f"call {i}: {name} differs"
        rkl, rl1, rl2 = oracle.forward(*arrs, 1 / np.sqrt(d), causal)
        compare(got[1], rl1, "bf16", f"call {i} lse1")
        compare(got[2], rl2, "bf16", f"call {i} lse2")
        compare(got[0], rkl, "bf16", f"call {i} kl")
