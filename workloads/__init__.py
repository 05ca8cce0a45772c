"""Seeded synthetic inputs for the attention-KL workloads.

This module only draws and rounds random numbers; it holds none of the KL
method's arithmetic.  It is the one piece shared by the fp64 oracle's tests and
by the GPU path's tests and benchmark, so both always see the same values.

Shapes follow the pages' own workload (long-context attention inputs, 32 heads,
BF16, 4K..512K context; the StreamKL gist.science technical summary,
"Problem Statement" and "Experimental Results").  The pages name no dataset, so
these Gaussian inputs are the workload itself and stand in for nothing else.

Recipe (per head, so that any head can be generated on its own):
  * stream for (seed, tensor id, head) = numpy default_rng([seed, tid, h]);
    tensor ids: Q1 = 0, K1 = 1, Q2-draw = 2, K2-draw = 3;
  * each draw is float32 standard_normal of shape [N, d];
  * "correlated" student: Q2 = Q1 + 0.3 * draw2, K2 = K1 + 0.3 * draw3 (fp32);
    "independent" student: Q2 = draw2, K2 = draw3;
  * for bf16 workloads every tensor is then rounded to bf16 (round to nearest,
    ties to even); both the GPU and the oracle read those rounded values.
A draw of N rows is a prefix of a draw of more rows from the same stream, so a
workload that uses the first rows of another one (decode, small N_Q) gets
exactly those rows.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np

Q1, K1, Q2, K2 = 0, 1, 2, 3


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    heads: int
    n_q: int
    n_k: int
    head_dim: int
    dtype: str          # "bf16" or "fp32"
    causal: bool
    student: str        # "correlated" or "independent"
    seed: int

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(self.head_dim))

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def elements(self) -> int:
        """Unmasked (query, key) pairs summed over heads."""
        if not self.causal:
            return self.heads * self.n_q * self.n_k
        off = self.n_k - self.n_q
        # query i sees min(n_k, i + off + 1) keys
        i = np.arange(self.n_q, dtype=np.int64)
        return int(self.heads * np.minimum(self.n_k, i + off + 1).sum())


WORKLOADS = {
    # 1 head, 256 x 256, d = 64, fp32, non-causal, i.i.d. inputs, seed 0
    "tiny": Workload("tiny", 1, 256, 256, 64, "fp32", False, "independent", 0),
    # 32 heads, 8K causal, bf16, student near teacher
    "causal8k": Workload("causal8k", 32, 8192, 8192, 128, "bf16", True, "correlated", 1),
    # 32 heads, 64K causal, bf16, student near teacher: the pages' 64K case
    "causal64k": Workload("causal64k", 32, 65536, 65536, 128, "bf16", True, "correlated", 2),
    # decode: one query against 512K keys, teacher and student independent
    "decode512k": Workload("decode512k", 32, 1, 524288, 128, "bf16", False, "independent", 3),
    # non-causal 128K, independent teacher and student (large KL)
    "noncausal128k": Workload("noncausal128k", 32, 131072, 131072, 128, "bf16", False, "independent", 4),
    # the first 512 queries of noncausal128k against all of its keys
    "smallq128k": Workload("smallq128k", 32, 512, 131072, 128, "bf16", False, "independent", 4),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding exact bf16 values."""
    b = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    t = b >> np.uint32(16)
    t &= np.uint32(1)
    t += np.uint32(0x7FFF)
    b += t
    b &= np.uint32(0xFFFF0000)
    return b.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp32 values that are already exact bf16."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _draw(seed: int, tid: int, h: int, n: int, d: int) -> np.ndarray:
    return np.random.default_rng([seed, tid, h]).standard_normal((n, d), dtype=np.float32)


def head_inputs(w: Workload, h: int):
    """(q1, k1, q2, k2) of head h as fp32 arrays holding the exact input values."""
    q1 = _draw(w.seed, Q1, h, w.n_q, w.head_dim)
    k1 = _draw(w.seed, K1, h, w.n_k, w.head_dim)
    q2 = _draw(w.seed, Q2, h, w.n_q, w.head_dim)
    k2 = _draw(w.seed, K2, h, w.n_k, w.head_dim)
    if w.student == "correlated":
        q2 = q1 + np.float32(0.3) * q2
        k2 = k1 + np.float32(0.3) * k2
    elif w.student != "independent":
        raise ValueError(w.student)
    out = (q1, k1, q2, k2)
    if w.dtype == "bf16":
        out = tuple(round_bf16(t) for t in out)
    return out


def all_inputs(w: Workload, threads: int = 8):
    """(q1, k1, q2, k2) as fp32 [H, N, d] arrays (small workloads only)."""
    with ThreadPoolExecutor(threads) as ex:
        per = list(ex.map(lambda h: head_inputs(w, h), range(w.heads)))
    return tuple(np.stack([p[t] for p in per]) for t in range(4))


def upstream_weights(w: Workload, seed: int = 99) -> np.ndarray:
    """A seeded non-trivial per-row upstream gradient g = dKL, fp32 [H, N_Q]."""
    rng = np.random.default_rng([w.seed, seed])
    return (0.5 + rng.random((w.heads, w.n_q))).astype(np.float32)
