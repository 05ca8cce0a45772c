"""ctypes view of the C ABI declared in include/streamkl.h (marshalling only)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libstreamkl.so")

# status codes (include/streamkl.h)
OK = 0
ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_SCALE, ERR_WORKSPACE, ERR_HIP, ERR_ALIGN, ERR_TOO_LARGE = (
    -1, -2, -3, -4, -5, -6, -7, -8)
NOALLOC_SCRATCH_BYTES = 8 << 20
BF16, FP32 = 0, 1
BWD_AUTO, BWD_FUSED, BWD_SEPARATE, BWD_DK_ONLY, BWD_DQ_ONLY = 0, 1, 2, 3, 4

EXPORTS = ("streamkl_fwd", "streamkl_fwd_splitk", "streamkl_fwd_splitk_noalloc", "streamkl_bwd_set1",
           "streamkl_bwd_set2", "streamkl_bwd_both",
           "streamkl_workspace_bytes", "streamkl_splitk_auto", "streamkl_bwd_select", "streamkl_strerror")

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t
_IN = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I]   # q1 k1 q2 k2 n_q n_k heads head_dim causal scale dtype

_SIGS = {
    "streamkl_fwd": (_I, _IN + [_P, _P, _P, _P]),
    "streamkl_fwd_splitk": (_I, _IN + [_I, _P, _P, _P, _P, _Z, _P]),
    "streamkl_fwd_splitk_noalloc": (_I, _IN + [_I, _P, _P, _P, _P]),
    "streamkl_bwd_set1": (_I, _IN + [_P, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "streamkl_bwd_set2": (_I, _IN + [_P, _P, _P, _P, _P, _P, _I, _P, _Z, _P]),
    "streamkl_bwd_both": (_I, _IN + [_P, _P, _P, _P, _P, _P, _P, _P, _I, _P]),
    "streamkl_workspace_bytes": (_Z, [_I, _I, _I, _I, _I, _I, _I]),
    "streamkl_splitk_auto": (_I, [_I, _I, _I, _I]),
    "streamkl_bwd_select": (_I, [_I, _I, _I, _I, _I]),
    "streamkl_strerror": (ctypes.c_char_p, [_I]),
}

_lib = None

PROBES_PATH = os.path.join(PKG, "libstreamkl_probes.so")
PROBE_EXPORTS = ("streamkl_probe_threads", "streamkl_probe_mfma", "streamkl_probe_mfma_data", "streamkl_probe_exp",
                 "streamkl_probe_exp_fma",
                 "streamkl_probe_read", "streamkl_probe_atomic")
_PROBE_SIGS = {
    "streamkl_probe_threads": (_I, []),
    "streamkl_probe_mfma": (_I, [_I, _I, _I, _P, _Z, _P]),
    "streamkl_probe_mfma_data": (_I, [_P, _Z, _I, _I, _I, _I, _P, _Z, _P]),
    "streamkl_probe_exp": (_I, [_I, _I, _P, _Z, _P]),
    "streamkl_probe_exp_fma": (_I, [_I, _I, _I, _P, _Z, _P]),
    "streamkl_probe_read": (_I, [_P, _Z, _I, _I, _P, _Z, _P]),
    "streamkl_probe_atomic": (_I, [_P, _Z, _I, _I, _P]),
}
_probes = None


def probes() -> ctypes.CDLL:
    """Load libstreamkl_probes.so (calibration kernels; bench.py --calibrate)."""
    global _probes
    if _probes is None:
        if not os.path.exists(PROBES_PATH):
            raise ImportError(f"{PROBES_PATH} is not built; run `python -m streaming_kl_divergence_amd.build`")
        l = ctypes.CDLL(PROBES_PATH)
        for name, (res, args) in _PROBE_SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _probes = l
    return _probes


class StreamKLError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({lib().streamkl_strerror(status).decode()})")


def lib() -> ctypes.CDLL:
    """Load libstreamkl.so; there is no fallback if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m streaming_kl_divergence_amd.build` "
                              "(the HIP library is the only implementation)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def check(fn: str, status: int) -> None:
    if status != OK:
        raise StreamKLError(fn, status)
