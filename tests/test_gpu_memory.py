"""Device memory of the library's calls (the pages' memory claim: the saved
state is O(N_Q) and the footprint does not grow with the key count; StreamKL
gist.science technical summary, Methodology 2 and Experimental Results).

* The library allocates nothing itself: device free memory (hipMemGetInfo) is
  unchanged by a call whose outputs and workspace the caller allocated.
* Through the torch binding, the extra device memory of a call is exactly its
  outputs (and the split-K workspace), up to the caching allocator's rounding,
  and it is the same for 4K and 16K keys at the same N_Q.
"""
import numpy as np
import pytest

from tests.gpu_util import device_inputs, log, need_gpu

pytestmark = pytest.mark.gpu

H, NQ, D = 4, 2048, 128
SLACK = 2 << 20   # the caching allocator rounds a large block up to a 2 MiB multiple


def _inputs(n_k, seed=3):
    rng = np.random.default_rng(seed)
    a = [rng.standard_normal((H, n, D), dtype=np.float32) for n in (NQ, n_k, NQ, n_k)]
    return device_inputs(a, "bf16")


def _free():
    import torch
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


def _extra(fn):
    """Peak torch-allocated bytes added while fn() runs, and what it returned."""
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    out = fn()
    torch.cuda.synchronize()
    return torch.cuda.max_memory_allocated() - base, out


def _nbytes(ts):
    return sum(t.numel() * t.element_size() for t in ts if t is not None)


def test_library_allocates_nothing():
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    from streaming_kl_divergence_amd import _lib
    log(f"case memory: library allocations, {H}x{NQ}x4096")
    NK = 4096
    q1, k1, q2, k2 = _inputs(NK)
    scale = 1 / np.sqrt(D)
    L = _lib.lib()
    kl, l1, l2 = [torch.empty(H, NQ, device="cuda") for _ in range(3)]
    # dQ1, dK1, dQ2, dK2: dQ has NQ rows per head, dK has NK
    grads = [torch.empty(H, n, D, device="cuda") for n in (NQ, NK, NQ, NK)]
    ws = torch.empty(max(16, skl.splitk_workspace_bytes(NQ, NK, H, D, 0)), device="cuda", dtype=torch.uint8)
    s = torch.cuda.current_stream().cuda_stream
    ptrs = (q1.data_ptr(), k1.data_ptr(), q2.data_ptr(), k2.data_ptr(), NQ, NK, H, D, 1, scale, _lib.BF16)
    # every buffer handed to the library below has the size its call writes
    assert all(t.shape == (H, NQ) for t in (kl, l1, l2))
    assert [tuple(g.shape) for g in grads] == [(H, NQ, D), (H, NK, D), (H, NQ, D), (H, NK, D)]
    assert k1.shape == (H, NK, D) and q1.shape == (H, NQ, D)

    def calls():
        assert L.streamkl_fwd(*ptrs, kl.data_ptr(), l1.data_ptr(), l2.data_ptr(), s) == 0
        assert L.streamkl_fwd_splitk(*ptrs, 0, kl.data_ptr(), l1.data_ptr(), l2.data_ptr(), ws.data_ptr(),
                                     ws.numel(), s) == 0
        assert L.streamkl_bwd_set1(*ptrs, l1.data_ptr(), l2.data_ptr(), None, grads[0].data_ptr(),
                                   grads[1].data_ptr(), _lib.BWD_SEPARATE, None, 0, s) == 0
        assert L.streamkl_bwd_set2(*ptrs, l1.data_ptr(), l2.data_ptr(), kl.data_ptr(), None, grads[0].data_ptr(),
                                   grads[1].data_ptr(), _lib.BWD_FUSED, None, 0, s) == 0
        assert L.streamkl_bwd_both(*ptrs, l1.data_ptr(), l2.data_ptr(), kl.data_ptr(), None,
                                   *(g.data_ptr() for g in grads), _lib.BWD_AUTO, s) == 0

    calls()                       # first launches load the code objects
    before = _free()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        calls()
    assert _free() == before
    assert torch.cuda.memory_allocated() == alloc0


@pytest.mark.parametrize("n_k", [4096, 16384])
def test_binding_extra_memory_is_the_outputs(n_k):
    need_gpu()
    import torch
    import streaming_kl_divergence_amd as skl
    log(f"case memory: binding outputs, {H}x{NQ}x{n_k}")
    q1, k1, q2, k2 = _inputs(n_k)
    scale = 1 / np.sqrt(D)
    row_bytes = 3 * H * NQ * 4                      # KL, LSE1, LSE2

    extra, (kl, l1, l2) = _extra(lambda: skl.fwd(q1, k1, q2, k2, scale, True))
    assert _nbytes((kl, l1, l2)) == row_bytes
    assert row_bytes <= extra <= row_bytes + SLACK, (extra, row_bytes)

    ws_bytes = skl.splitk_workspace_bytes(NQ, n_k, H, D, 0)
    extra, out = _extra(lambda: skl.fwd_splitk(q1, k1, q2, k2, scale, True))
    assert row_bytes + ws_bytes <= extra <= row_bytes + ws_bytes + SLACK, (extra, row_bytes, ws_bytes)
    del out

    grad_bytes = 2 * H * NQ * D * 4 + 2 * H * n_k * D * 4
    extra, g = _extra(lambda: skl.bwd_both(q1, k1, q2, k2, scale, True, l1, l2, kl))
    assert _nbytes(g) == grad_bytes
    assert grad_bytes <= extra <= grad_bytes + 4 * SLACK, (extra, grad_bytes)
    del g
    for setting in (1, 2):
        extra, g = _extra(lambda: skl.bwd(setting, q1, k1, q2, k2, scale, True, l1, l2, kl=kl))
        assert grad_bytes // 2 <= extra <= grad_bytes // 2 + 2 * SLACK, (setting, extra)
        del g
    # what the materialised pair of distributions would take, for scale
    log(f"n_k={n_k}: saved state {row_bytes} B; P1 + P2 materialised in bf16 {2 * H * NQ * n_k * 2} B")
