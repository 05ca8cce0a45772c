"""The C-ABI library on the CPU: it loads, exports every function that
include/streamkl.h declares, and rejects invalid arguments with the documented
status codes before anything is enqueued (no GPU is touched)."""
import ctypes
import math
import os
import re

import pytest

from streaming_kl_divergence_amd import _lib as L

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HEADER = os.path.join(INCLUDE, "streamkl.h")
PROBES_HEADER = os.path.join(INCLUDE, "streamkl_probes.h")
FAKE = 4096  # a non-NULL, 16-byte aligned address that is never dereferenced


def declared_functions(header=HEADER):
    with open(header) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(streamkl_\w+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = L.lib()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)


def test_probe_library_exports_and_validates():
    lib = L.probes()
    names = declared_functions(PROBES_HEADER)
    assert set(names) == set(L.PROBE_EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    # invalid arguments are refused before any launch
    t = lib.streamkl_probe_threads()
    assert t == 256
    assert lib.streamkl_probe_mfma(1, 4, 10, FAKE, 4 * t - 1, None) == -1
    assert lib.streamkl_probe_mfma(4, 4, 10, FAKE, 4 * t, None) == -1              # 1 to 3 waves per SIMD
    assert lib.streamkl_probe_mfma(0, 4, 10, FAKE, 4 * t, None) == -1
    assert lib.streamkl_probe_mfma_data(FAKE, 4 * t * 256, 0, 4, 4, 10, FAKE, 4 * t, None) == -1
    assert lib.streamkl_probe_mfma_data(FAKE, 4 * t * 256, 6, 1, 4, 10, FAKE, 4 * t, None) == -1   # operand mode 0-5
    assert lib.streamkl_probe_mfma_data(FAKE, 4 * t * 256, -1, 1, 4, 10, FAKE, 4 * t, None) == -1
    assert lib.streamkl_probe_mfma_data(FAKE, 4 * t * 256 - 16, 1, 2, 4, 10, FAKE, 4 * t, None) == -1
    assert lib.streamkl_probe_exp(0, 10, FAKE, 4 * t, None) == -1
    assert lib.streamkl_probe_exp_fma(3, 4, 10, FAKE, 4 * 512, None) == -1      # modes 0 to 2
    assert lib.streamkl_probe_exp_fma(2, 4, 10, FAKE, 4 * 512 - 1, None) == -1  # sink too small
    assert lib.streamkl_probe_read(FAKE, 100, 0, 4, FAKE, 4 * t * 4, None) == -1      # not a multiple of 16
    assert lib.streamkl_probe_read(FAKE + 4, 64, 1, 4, FAKE, 4 * t * 4, None) == -1   # misaligned
    assert lib.streamkl_probe_atomic(None, 16, 4, 1, None) == -1


def _fwd(**kw):
    a = dict(q1=FAKE, k1=FAKE, q2=FAKE, k2=FAKE, n_q=16, n_k=16, heads=2, d=64, causal=0, scale=0.125, dt=L.BF16,
             kl=FAKE, l1=FAKE, l2=FAKE)
    a.update(kw)
    return L.lib().streamkl_fwd(a["q1"], a["k1"], a["q2"], a["k2"], a["n_q"], a["n_k"], a["heads"], a["d"],
                                a["causal"], a["scale"], a["dt"], a["kl"], a["l1"], a["l2"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q1=None), L.ERR_NULL), (dict(k2=None), L.ERR_NULL), (dict(kl=None), L.ERR_NULL),
    (dict(n_q=0), L.ERR_SHAPE), (dict(n_k=-1), L.ERR_SHAPE), (dict(heads=0), L.ERR_SHAPE),
    (dict(n_q=32, n_k=16, causal=1), L.ERR_SHAPE), (dict(heads=1 << 20, n_q=1 << 12), L.ERR_SHAPE),
    (dict(d=96), L.ERR_UNSUPPORTED), (dict(d=256), L.ERR_UNSUPPORTED), (dict(dt=7), L.ERR_UNSUPPORTED),
    (dict(scale=math.nan), L.ERR_SCALE), (dict(scale=math.inf), L.ERR_SCALE), (dict(scale=-1.0), L.ERR_SCALE),
    (dict(q2=FAKE + 2), L.ERR_ALIGN),
])
def test_forward_validation(kw, code):
    assert _fwd(**kw) == code


def test_splitk_validation():
    lib = L.lib()
    args = [FAKE] * 4 + [1, 4096, 2, 128, 0, 0.1, L.BF16]
    outs = [FAKE] * 3
    need = lib.streamkl_workspace_bytes(0, 1, 4096, 2, 128, 4, 0)
    assert need > 0 and need != ctypes.c_size_t(-1).value
    assert lib.streamkl_fwd_splitk(*args, 4, *outs, None, need, None) == L.ERR_WORKSPACE
    assert lib.streamkl_fwd_splitk(*args, 4, *outs, FAKE, need - 1, None) == L.ERR_WORKSPACE
    assert lib.streamkl_fwd_splitk(*args, -1, *outs, FAKE, need, None) == L.ERR_UNSUPPORTED
    assert lib.streamkl_fwd_splitk(*args, 2000, *outs, FAKE, need, None) == L.ERR_UNSUPPORTED
    assert lib.streamkl_workspace_bytes(0, 1, 4096, 2, 96, 4, 0) == ctypes.c_size_t(-1).value
    assert lib.streamkl_workspace_bytes(5, 1, 4096, 2, 128, 4, 0) == ctypes.c_size_t(-1).value
    assert lib.streamkl_workspace_bytes(1, 1, 4096, 2, 128, 0, 9) == ctypes.c_size_t(-1).value
    assert lib.streamkl_workspace_bytes(1, 1, 4096, 2, 128, 0, 0) == 0


def test_splitk_refuses_a_grid_beyond_32_bit_work_indices():
    lib = L.lib()
    # 2^30 queries of one head: 2^23 query blocks x 1024 splits = 2^33 workgroups
    n = 1 << 30
    args = [FAKE] * 4 + [n, n, 1, 128, 0, 0.1, L.BF16]
    assert lib.streamkl_fwd_splitk(*args, 1024, FAKE, FAKE, FAKE, FAKE, 1 << 62, None) == L.ERR_SHAPE
    assert lib.streamkl_fwd_splitk_noalloc(*args, 1024, FAKE, FAKE, FAKE, None) == L.ERR_SHAPE
    # the same head with 255 splits stays below 2^31 workgroups and reaches the workspace check
    assert lib.streamkl_fwd_splitk(*args, 255, FAKE, FAKE, FAKE, FAKE, 16, None) == L.ERR_WORKSPACE


def test_noalloc_splitk_refuses_more_than_its_scratch():
    """streamkl_fwd_splitk_noalloc validates like streamkl_fwd_splitk and
    refuses a problem whose partial states exceed its fixed 8 MiB scratch,
    before any device call."""
    lib = L.lib()
    heads, n_q, n_k, d = 64, 4096, 8192, 128
    need = lib.streamkl_workspace_bytes(0, n_q, n_k, heads, d, 16, 0)
    assert need > L.NOALLOC_SCRATCH_BYTES
    args = [FAKE] * 4 + [n_q, n_k, heads, d, 0, 0.1, L.BF16]
    assert lib.streamkl_fwd_splitk_noalloc(*args, 16, FAKE, FAKE, FAKE, None) == L.ERR_TOO_LARGE
    assert b"8 MiB" in lib.streamkl_strerror(L.ERR_TOO_LARGE)
    assert lib.streamkl_fwd_splitk_noalloc(*args, 16, None, FAKE, FAKE, None) == L.ERR_NULL
    assert lib.streamkl_fwd_splitk_noalloc(*args, 2000, FAKE, FAKE, FAKE, None) == L.ERR_UNSUPPORTED
    bad = list(args)
    bad[7] = 96
    assert lib.streamkl_fwd_splitk_noalloc(*bad, 16, FAKE, FAKE, FAKE, None) == L.ERR_UNSUPPORTED


def test_splitk_auto_is_a_valid_split_count():
    lib = L.lib()
    for n_q, n_k in ((1, 524288), (1, 64), (37, 3000), (65536, 65536)):
        s = lib.streamkl_splitk_auto(n_q, n_k, 32, 128)
        assert 1 <= s <= 1024
        # every range holds at least one key tile
        assert (s - 1) * 64 < n_k


def test_backward_validation():
    lib = L.lib()
    base = [FAKE] * 4 + [16, 16, 2, 64, 1, 0.125, L.BF16, FAKE, FAKE]
    # Setting 1: lse1 lse2 dkl dq dk path ws wsb stream
    assert lib.streamkl_bwd_set1(*base, None, FAKE, FAKE, 9, None, 0, None) == L.ERR_UNSUPPORTED
    assert lib.streamkl_bwd_set1(*base, None, None, FAKE, 0, None, 0, None) == L.ERR_NULL
    assert lib.streamkl_bwd_set1(*base, None, FAKE + 4, FAKE, 0, None, 0, None) == L.ERR_ALIGN
    bad = list(base)
    bad[11] = None  # lse1
    assert lib.streamkl_bwd_set1(*bad, None, FAKE, FAKE, 0, None, 0, None) == L.ERR_NULL
    # Setting 2 needs kl
    assert lib.streamkl_bwd_set2(*base, None, None, FAKE, FAKE, 0, None, 0, None) == L.ERR_NULL
    bad = list(base)
    bad[4] = 32  # n_q > n_k with causal
    assert lib.streamkl_bwd_set2(*bad, FAKE, None, FAKE, FAKE, 0, None, 0, None) == L.ERR_SHAPE


def test_both_settings_validation():
    lib = L.lib()
    base = [FAKE] * 4 + [16, 16, 2, 64, 1, 0.125, L.BF16, FAKE, FAKE]
    # lse1 lse2 | kl dkl dq1 dk1 dq2 dk2 path stream
    assert lib.streamkl_bwd_both(*base, None, None, FAKE, FAKE, FAKE, FAKE, 0, None) == L.ERR_NULL   # kl
    assert lib.streamkl_bwd_both(*base, FAKE, None, FAKE, FAKE, None, FAKE, 0, None) == L.ERR_NULL   # dq2
    assert lib.streamkl_bwd_both(*base, FAKE, None, FAKE, FAKE + 8, FAKE, FAKE, 0, None) == L.ERR_ALIGN
    assert lib.streamkl_bwd_both(*base, FAKE, None, FAKE, FAKE, FAKE, FAKE, L.BWD_FUSED, None) == L.ERR_UNSUPPORTED
    assert lib.streamkl_bwd_both(*base, FAKE, None, FAKE, FAKE, FAKE, FAKE, 9, None) == L.ERR_UNSUPPORTED
    # DK_ONLY needs no dQ outputs; DQ_ONLY no dK outputs (these checks stop before any launch: bad head_dim)
    bad = list(base)
    bad[7] = 96  # head_dim
    assert lib.streamkl_bwd_both(*bad, FAKE, None, None, FAKE, None, FAKE, L.BWD_DK_ONLY, None) == L.ERR_UNSUPPORTED
    assert lib.streamkl_bwd_both(*bad, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == L.ERR_UNSUPPORTED
    bad = list(base)
    bad[9] = float("nan")
    assert lib.streamkl_bwd_both(*bad, FAKE, None, FAKE, FAKE, FAKE, FAKE, 0, None) == L.ERR_SCALE


def test_strerror_covers_every_code():
    lib = L.lib()
    for code in (L.OK, L.ERR_NULL, L.ERR_SHAPE, L.ERR_UNSUPPORTED, L.ERR_SCALE, L.ERR_WORKSPACE, L.ERR_HIP,
                 L.ERR_ALIGN, L.ERR_TOO_LARGE):
        assert lib.streamkl_strerror(code) not in (None, b"unknown status")
    assert lib.streamkl_strerror(12345) == b"unknown status"


def test_bwd_select():
    lib = L.lib()
    # measured on MI355X: the separate kernels beat the atomic-dQ fused kernel
    # at every size (64 .. 16K queries x 128K keys), so AUTO is always separate
    for shape in [(512, 131072, 32, 128, 0), (65536, 65536, 32, 128, 1), (64, 131072, 32, 128, 0),
                  (256, 256, 1, 64, 0)]:
        assert lib.streamkl_bwd_select(*shape) == L.BWD_SEPARATE, shape


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(L, "_lib", None)
    monkeypatch.setattr(L, "LIB_PATH", "/nonexistent/libstreamkl.so")
    with pytest.raises(ImportError):
        L.lib()


def test_wrapper_rejects_bad_saved_state_and_outputs():
    """The torch wrapper checks every tensor it hands to the library (device,
    dtype, contiguity, shape, overlap) so that a host pointer or an undersized
    buffer never reaches a kernel."""
    import torch
    from streaming_kl_divergence_amd import ops
    cpu, gpu = torch.device("cpu"), torch.device("cuda", 0)
    good = torch.zeros(2, 16)
    ops.check_rows(good, "lse1", 2, 16, cpu)
    ops.check_rows(None, "dkl", 2, 16, cpu)
    with pytest.raises(ValueError, match="is on cpu"):
        ops.check_rows(good, "lse1", 2, 16, gpu)            # host memory for device inputs
    with pytest.raises(ValueError, match="fp32"):
        ops.check_rows(good.double(), "kl", 2, 16, cpu)
    with pytest.raises(ValueError, match="fp32"):
        ops.check_rows(torch.zeros(2, 15), "kl", 2, 16, cpu)
    with pytest.raises(ValueError, match="fp32"):
        ops.check_rows(torch.zeros(16, 2).t(), "dkl", 2, 16, cpu)   # not contiguous
    with pytest.raises(TypeError):
        ops.check_rows([0.0] * 32, "lse2", 2, 16, cpu)
    out = torch.zeros(2, 16, 64)
    ops.check_out(out, "dq", (2, 16, 64), cpu)
    with pytest.raises(ValueError, match="is on cpu"):
        ops.check_out(out, "dq", (2, 16, 64), gpu)
    with pytest.raises(ValueError, match="fp32"):
        ops.check_out(torch.zeros(2, 16, 64, dtype=torch.bfloat16), "dk", (2, 16, 64), cpu)
    with pytest.raises(ValueError, match="fp32"):
        ops.check_out(torch.zeros(2, 8, 64), "dk", (2, 16, 64), cpu)   # too small
    with pytest.raises(ValueError, match="fp32"):
        ops.check_out(torch.zeros(2, 64, 16).transpose(1, 2), "dq", (2, 16, 64), cpu)
    big = torch.zeros(4, 16, 64)
    ops.check_disjoint((("dq1", big[:2]), ("dq2", big[2:]), ("dk1", None)))
    with pytest.raises(ValueError, match="overlap"):
        ops.check_disjoint((("dq1", big[:3]), ("dq2", big[2:])))
