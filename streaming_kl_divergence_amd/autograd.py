"""Attention KL divergence as a differentiable loss (torch.autograd).

"StreamKL: Fast and Memory-Efficient KL Divergence for Boosting Attention
Distillation" (gist.science technical summary), Methodology 2, Recomputation
Strategy: the forward keeps only KL, LSE1 and LSE2 per row; the backward
regenerates the probabilities tile by tile.  The pages name two settings:
  Setting 1 - the teacher distribution P1 is held fixed and gradients flow to
              the student's Q2, K2 ("student");
  Setting 2 - the student distribution P2 is held fixed and gradients flow to
              the teacher's Q1, K1 ("teacher").
P1 does not depend on (Q2, K2) and P2 does not depend on (Q1, K1), so each
setting's gradients are the true partial derivatives, and "both" (the two
settings together) is the full gradient of the loss.

Every step runs in the HIP library: the forward (the one-pass kernel, or the
split-K pair of Methodology 3 when the query blocks alone cannot fill the GPU,
as the library's split-count heuristic decides), and in the backward only the
kernels for the gradients autograd asks for (the dK-only or dQ-only launch
when just one of Q, K needs one).  The library's gradients are fp32;
they are returned in the inputs' dtype, as autograd requires.
"""
from __future__ import annotations

import torch

from . import ops

_SETTINGS = ("student", "teacher", "both")


class _AttentionKL(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q1, k1, q2, k2, scale, causal, setting):
        kl, lse1, lse2 = ops.fwd_auto(q1, k1, q2, k2, scale, causal)
        ctx.save_for_backward(q1, k1, q2, k2, kl, lse1, lse2)
        ctx.scale, ctx.causal, ctx.setting = scale, causal, setting
        return kl

    @staticmethod
    def backward(ctx, g):
        q1, k1, q2, k2, kl, lse1, lse2 = ctx.saved_tensors
        need = ctx.needs_input_grad
        g = g.contiguous().float()
        grads = [None, None, None, None]

        def run(setting, iq, ik):
            want_q, want_k = need[iq], need[ik]
            if not (want_q or want_k):
                return
            path = "separate" if (want_q and want_k) else ("dq_only" if want_q else "dk_only")
            kw = dict(kl=kl) if setting == 2 else {}
            dq, dk = ops.bwd(setting, q1, k1, q2, k2, ctx.scale, ctx.causal, lse1, lse2, dkl=g, path=path, **kw)
            if want_q:
                grads[iq] = dq.to(q1.dtype)
            if want_k:
                grads[ik] = dk.to(k1.dtype)

        if ctx.setting == "both" and all(need[:4]):
            # all four gradients: one recomputation serves both settings
            dq1, dk1, dq2, dk2 = ops.bwd_both(q1, k1, q2, k2, ctx.scale, ctx.causal, lse1, lse2, kl, dkl=g)
            grads = [dq1.to(q1.dtype), dk1.to(k1.dtype), dq2.to(q2.dtype), dk2.to(k2.dtype)]
            return grads[0], grads[1], grads[2], grads[3], None, None, None
        if ctx.setting in ("student", "both"):
            run(1, 2, 3)   # Setting 1: dQ2, dK2
        if ctx.setting in ("teacher", "both"):
            run(2, 0, 1)   # Setting 2: dQ1, dK1
        return grads[0], grads[1], grads[2], grads[3], None, None, None


def attention_kl(q1, k1, q2, k2, scale: float | None = None, causal: bool = False, setting: str = "student"):
    """Per-row KL(P1 || P2), fp32 [heads, n_q], with P_t = softmax(scale Q_t K_t^T)
    (bottom-right causal mask when causal).  Inputs are contiguous
    [heads, n, head_dim] device tensors of one dtype (bfloat16 or float32).

    setting: "student" (Setting 1: teacher frozen, gradients to q2, k2),
    "teacher" (Setting 2: student frozen, gradients to q1, k1) or "both".
    Tensors of the frozen side get no gradient whatever their requires_grad.
    """
    if setting not in _SETTINGS:
        raise ValueError(f"setting must be one of {_SETTINGS}")
    if scale is None:
        scale = q1.shape[-1] ** -0.5
    return _AttentionKL.apply(q1, k1, q2, k2, float(scale), bool(causal), setting)
