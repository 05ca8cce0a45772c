"""Checks that pin the fp64 oracle to facts outside itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with an
independent statement of the mathematics: brute force with the textbook
formula, a library routine (torch autograd and kl_div), finite differences,
closed forms, invariants, and the streaming five-scalar recurrence that the
StreamKL pages print ("StreamKL: Fast and Memory-Efficient KL Divergence for
Boosting Attention Distillation", gist.science technical summary, Methodology 1
"Online Formulation": L = acc / l1 + LSE2 - LSE1 with LSE_t = m_t + log l_t).

The functions take the oracle module as an argument so that the mutation tests
can hand them a deliberately broken copy and check that some pin fails.
"""
from __future__ import annotations

import math

import numpy as np


def _rand(rng, n, d, s=1.0):
    return s * rng.standard_normal((n, d))


def _case(rng, n_q, n_k, d, s=1.0):
    return [_rand(rng, n_q, d, s), _rand(rng, n_k, d, s), _rand(rng, n_q, d, s), _rand(rng, n_k, d, s)]


# ---- P1: brute force, textbook formula, unshifted exponentials ---------------

def brute_force_row(q1, k1, q2, k2, scale, causal, i):
    """KL, LSE1, LSE2 of row i straight from the definition, pure Python."""
    n_q, n_k = len(q1), len(k1)
    keys = [j for j in range(n_k) if (not causal) or j <= i + (n_k - n_q)]
    s1 = [scale * sum(a * b for a, b in zip(q1[i], k1[j])) for j in keys]
    s2 = [scale * sum(a * b for a, b in zip(q2[i], k2[j])) for j in keys]
    z1 = sum(math.exp(v) for v in s1)
    z2 = sum(math.exp(v) for v in s2)
    p1 = [math.exp(v) / z1 for v in s1]
    p2 = [math.exp(v) / z2 for v in s2]
    kl = sum(a * math.log(a / b) for a, b in zip(p1, p2) if a > 0)
    return kl, math.log(z1), math.log(z2)


def pin_brute_force(oracle, seed=0):
    rng = np.random.default_rng(seed)
    for (n_q, n_k, d, causal) in [(1, 1, 1, False), (3, 5, 2, False), (5, 5, 3, True),
                                  (4, 7, 4, True), (8, 8, 4, False), (2, 8, 3, True)]:
        q1, k1, q2, k2 = _case(rng, n_q, n_k, d, 0.8)
        scale = 0.7
        kl, l1, l2 = oracle.forward_head(q1, k1, q2, k2, scale, causal)
        for i in range(n_q):
            bkl, bl1, bl2 = brute_force_row(q1.tolist(), k1.tolist(), q2.tolist(), k2.tolist(), scale, causal, i)
            assert abs(kl[i] - bkl) <= 1e-12 + 1e-10 * abs(bkl), (n_q, n_k, d, causal, i, kl[i], bkl)
            assert abs(l1[i] - bl1) <= 1e-12 * max(1, abs(bl1)), (i, l1[i], bl1)
            assert abs(l2[i] - bl2) <= 1e-12 * max(1, abs(bl2)), (i, l2[i], bl2)


def pin_bernoulli(oracle, seed=1):
    """Two keys: KL of two Bernoulli laws, sigma(a) vs sigma(b)."""
    rng = np.random.default_rng(seed)
    for _ in range(20):
        q1, k1, q2, k2 = _case(rng, 1, 2, 3)
        scale = 0.9
        a = scale * (q1[0] @ (k1[0] - k1[1]))
        b = scale * (q2[0] @ (k2[0] - k2[1]))
        sa, sb = 1 / (1 + math.exp(-a)), 1 / (1 + math.exp(-b))
        ref = sa * math.log(sa / sb) + (1 - sa) * math.log((1 - sa) / (1 - sb))
        kl, _, _ = oracle.forward_head(q1, k1, q2, k2, scale, False)
        assert abs(kl[0] - ref) <= 1e-13 + 1e-11 * ref, (kl[0], ref)


# ---- P2: library routine (torch fp64 kl_div + autograd) ----------------------

def _torch_kl_and_grads(q1, k1, q2, k2, scale, causal, g, setting):
    import torch
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q1, k1, q2, k2)]
    n_q, n_k = q1.shape[0], k1.shape[0]
    i = torch.arange(n_q)[:, None]
    j = torch.arange(n_k)[None, :]
    allowed = (j <= i + (n_k - n_q)) if causal else torch.ones(n_q, n_k, dtype=torch.bool)
    s1 = scale * t[0] @ t[1].T
    s2 = scale * t[2] @ t[3].T
    s1 = s1.masked_fill(~allowed, -1e30)  # exp underflows to exactly 0 in fp64
    s2 = s2.masked_fill(~allowed, -1e30)
    lp1 = torch.log_softmax(s1, dim=-1)
    lp2 = torch.log_softmax(s2, dim=-1)
    if setting == 1:
        lp1 = lp1.detach()   # P1 fixed
    else:
        lp2 = lp2.detach()   # P2 fixed
    kl = torch.nn.functional.kl_div(lp2, lp1, reduction="none", log_target=True).sum(-1)
    loss = (torch.tensor(g, dtype=torch.float64) * kl).sum()
    loss.backward()
    if setting == 1:
        return kl.detach().numpy(), t[2].grad.numpy(), t[3].grad.numpy()
    return kl.detach().numpy(), t[0].grad.numpy(), t[1].grad.numpy()


def pin_torch_autograd(oracle, seed=2):
    rng = np.random.default_rng(seed)
    for (n_q, n_k, d, causal) in [(16, 16, 8, False), (16, 16, 8, True), (9, 23, 5, True), (12, 31, 6, False)]:
        q1, k1, q2, k2 = _case(rng, n_q, n_k, d)
        g = 0.5 + rng.random(n_q)
        scale = 1 / math.sqrt(d)
        kl, _, _ = oracle.forward_head(q1, k1, q2, k2, scale, causal)
        for setting in (1, 2):
            tkl, tdq, tdk = _torch_kl_and_grads(q1, k1, q2, k2, scale, causal, g, setting)
            assert np.allclose(kl, tkl, rtol=1e-11, atol=1e-13), (setting, np.abs(kl - tkl).max())
            dq, dk = oracle.backward_head(setting, q1, k1, q2, k2, scale, causal, g)
            assert np.allclose(dq, tdq, rtol=1e-10, atol=1e-13), (setting, np.abs(dq - tdq).max())
            assert np.allclose(dk, tdk, rtol=1e-10, atol=1e-13), (setting, np.abs(dk - tdk).max())
            # the per-row and per-key entry points give the same numbers
            rows = np.array([0, n_q // 2, n_q - 1])
            assert np.allclose(oracle.dq_rows(setting, q1, k1, q2, k2, scale, causal, rows, g), dq[rows],
                               rtol=1e-12, atol=1e-14)
            keys = np.array([0, n_k // 3, n_k - 1])
            assert np.allclose(oracle.dk_keys(setting, q1, k1, q2, k2, scale, causal, keys, g), dk[keys],
                               rtol=1e-12, atol=1e-14)
            # dK columns from the saved per-row statistics, against torch's dK directly
            skl, sl1, sl2 = oracle.forward_head(q1, k1, q2, k2, scale, causal)
            dks = oracle.dk_keys_from_state(setting, q1, k1, q2, k2, scale, causal, keys, sl1, sl2, skl, g)
            assert np.allclose(dks, tdk[keys], rtol=1e-10, atol=1e-13), (setting, np.abs(dks - tdk[keys]).max())
            # the logit gradient itself: contracted with the setting's keys and
            # queries it must give torch's dQ and dK, and each of its rows sums
            # to zero (Setting 1: sum P2 - sum P1 = 0; Setting 2: sum P1 r = KL)
            ds = oracle.dlogits_head(setting, q1, k1, q2, k2, scale, causal, g)
            q_t, k_t = (q2, k2) if setting == 1 else (q1, k1)
            assert np.allclose(scale * ds @ k_t, tdq, rtol=1e-10, atol=1e-13), setting
            assert np.allclose(scale * ds.T @ q_t, tdk, rtol=1e-10, atol=1e-13), setting
            assert np.abs(ds.sum(1)).max() <= 1e-13 * max(1.0, np.abs(ds).max()), setting
            mask = oracle.allowed_mask(np.arange(n_q), n_q, n_k, causal)
            assert not np.any(ds[~mask]), setting


# ---- P3: invariants ------------------------------------------------------------

def pin_invariants(oracle, seed=3):
    rng = np.random.default_rng(seed)
    n_q, n_k, d = 24, 40, 8
    for causal in (False, True):
        q1, k1, q2, k2 = _case(rng, n_q, n_k, d)
        scale = 1 / math.sqrt(d)
        # identical teacher and student: KL = 0 exactly, no gradient
        kl, l1, l2 = oracle.forward_head(q1, k1, q1, k1, scale, causal)
        assert np.all(np.abs(kl) <= 1e-14) and np.array_equal(l1, l2)
        for setting in (1, 2):
            dq, dk = oracle.backward_head(setting, q1, k1, q1, k1, scale, causal)
            assert np.abs(dq).max() <= 1e-14 and np.abs(dk).max() <= 1e-14
        # KL >= 0, and each P row sums to 1: sum_j exp(s_j - LSE) = 1
        kl, l1, l2 = oracle.forward_head(q1, k1, q2, k2, scale, causal)
        assert np.all(kl >= -1e-15)
        mask = oracle.allowed_mask(np.arange(n_q), n_q, n_k, causal)
        for q, k, lse in ((q1, k1, l1), (q2, k2, l2)):
            s = scale * q @ k.T
            rowsum = np.where(mask, np.exp(s - lse[:, None]), 0).sum(1)
            assert np.allclose(rowsum, 1.0, atol=1e-13)
        # a key shift by one constant vector shifts every logit of a row by one
        # constant: KL is unchanged, LSE moves by scale * q . c
        c1, c2 = rng.standard_normal(d), rng.standard_normal(d)
        kls, l1s, l2s = oracle.forward_head(q1, k1 + c1, q2, k2 + c2, scale, causal)
        assert np.allclose(kls, kl, rtol=1e-10, atol=1e-12)
        assert np.allclose(l1s, l1 + scale * q1 @ c1, atol=1e-11)
        assert np.allclose(l2s, l2 + scale * q2 @ c2, atol=1e-11)
        # gradients: each row of dS sums to zero, hence sum_j dK_j = 0
        for setting in (1, 2):
            _, dk = oracle.backward_head(setting, q1, k1, q2, k2, scale, causal)
            assert np.abs(dk.sum(0)).max() <= 1e-12
        # scale 0: uniform rows, KL = 0, LSE = log(number of allowed keys)
        kl0, l10, _ = oracle.forward_head(q1, k1, q2, k2, 0.0, causal)
        assert np.all(np.abs(kl0) <= 1e-15)
        assert np.allclose(l10, np.log(mask.sum(1)), atol=1e-14)
    # causal, N_Q = N_K: row 0 sees one key, KL = 0 and its dQ row is zero
    q1, k1, q2, k2 = _case(rng, 16, 16, 4)
    kl, _, _ = oracle.forward_head(q1, k1, q2, k2, 0.5, True)
    assert abs(kl[0]) <= 1e-15
    for setting in (1, 2):
        dq, _ = oracle.backward_head(setting, q1, k1, q2, k2, 0.5, True)
        assert np.abs(dq[0]).max() <= 1e-15
    # N_K = 1: every row is one point mass, KL = 0
    q1, k1, q2, k2 = _case(rng, 5, 1, 4)
    kl, _, _ = oracle.forward_head(q1, k1, q2, k2, 0.5, False)
    assert np.all(np.abs(kl) <= 1e-15)


# ---- P4: closed form -------------------------------------------------------------

def pin_uniform_teacher(oracle, seed=4):
    """Q1 = 0 makes P1 uniform over the allowed keys, and then
    KL_i = LSE2_i - mean_{allowed j} s2_ij - log |A_i|."""
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        n_q, n_k, d = 20, 33, 6
        _, k1, q2, k2 = _case(rng, n_q, n_k, d)
        q1 = np.zeros((n_q, d))
        scale = 0.6
        kl, _, l2 = oracle.forward_head(q1, k1, q2, k2, scale, causal)
        mask = oracle.allowed_mask(np.arange(n_q), n_q, n_k, causal)
        s2 = scale * q2 @ k2.T
        cnt = mask.sum(1)
        mean_s2 = np.where(mask, s2, 0).sum(1) / cnt
        # LSE2 by its own definition, unshifted
        lse2 = np.log(np.where(mask, np.exp(s2), 0).sum(1))
        assert np.allclose(l2, lse2, atol=1e-12)
        assert np.allclose(kl, lse2 - mean_s2 - np.log(cnt), atol=1e-12)


# ---- P5: central finite differences -------------------------------------------

def pin_finite_differences(oracle, seed=5):
    rng = np.random.default_rng(seed)
    n_q, n_k, d = 7, 11, 5
    for causal in (False, True):
        q1, k1, q2, k2 = _case(rng, n_q, n_k, d)
        g = 0.5 + rng.random(n_q)
        scale = 0.45

        def loss(a):
            kl, _, _ = oracle.forward_head(*a, scale, causal)
            return float(g @ kl)

        for setting, (iq, ik) in ((1, (2, 3)), (2, (0, 1))):
            dq, dk = oracle.backward_head(setting, q1, k1, q2, k2, scale, causal, g)
            for which, grad in ((iq, dq), (ik, dk)):
                for _ in range(6):
                    r, c = rng.integers(grad.shape[0]), rng.integers(d)
                    h = 1e-6
                    ap = [x.copy() for x in (q1, k1, q2, k2)]
                    am = [x.copy() for x in (q1, k1, q2, k2)]
                    ap[which][r, c] += h
                    am[which][r, c] -= h
                    fd = (loss(ap) - loss(am)) / (2 * h)
                    assert abs(fd - grad[r, c]) <= 1e-7 + 1e-6 * abs(fd), (setting, which, r, c, fd, grad[r, c])


# ---- P6: the pages' streaming identity, five scalars per row -------------------

def streaming_row(s1, s2, tiles):
    """The online recurrence of the pages over key tiles (fp64).

    State per row: running maxima m1, m2; exp-sums l1, l2; acc, the P1-weighted
    logit difference, rescaled with l1 whenever m1 moves.  Returns the partial
    state; finish() turns it into (L, LSE1, LSE2).
    """
    m1 = m2 = -math.inf
    l1 = l2 = acc = 0.0
    for lo, hi in tiles:
        t1, t2 = s1[lo:hi], s2[lo:hi]
        n1, n2 = max(m1, max(t1)), max(m2, max(t2))
        a1, a2 = math.exp(m1 - n1), math.exp(m2 - n2)
        p1 = [math.exp(v - n1) for v in t1]
        p2 = [math.exp(v - n2) for v in t2]
        l1 = a1 * l1 + sum(p1)
        l2 = a2 * l2 + sum(p2)
        acc = a1 * acc + sum(p * (x - y) for p, x, y in zip(p1, t1, t2))
        m1, m2 = n1, n2
    return m1, l1, acc, m2, l2


def merge_states(states):
    """Combine partial (m1, l1, acc, m2, l2) states over disjoint key ranges."""
    M1 = max(s[0] for s in states)
    M2 = max(s[3] for s in states)
    w1 = [math.exp(s[0] - M1) for s in states]
    w2 = [math.exp(s[3] - M2) for s in states]
    return (M1, sum(w * s[1] for w, s in zip(w1, states)), sum(w * s[2] for w, s in zip(w1, states)),
            M2, sum(w * s[4] for w, s in zip(w2, states)))


def finish(state):
    m1, l1, acc, m2, l2 = state
    lse1 = m1 + math.log(l1)
    lse2 = m2 + math.log(l2)
    return acc / l1 + lse2 - lse1, lse1, lse2


def pin_streaming_identity(oracle, seed=6):
    rng = np.random.default_rng(seed)
    for causal in (False, True):
        n_q, n_k, d = 6, 50, 7
        q1, k1, q2, k2 = _case(rng, n_q, n_k, d, 1.3)
        scale = 0.5
        kl, l1, l2 = oracle.forward_head(q1, k1, q2, k2, scale, causal)
        for i in range(n_q):
            n_allowed = i + (n_k - n_q) + 1 if causal else n_k
            s1 = (scale * q1[i] @ k1[:n_allowed].T).tolist()
            s2 = (scale * q2[i] @ k2[:n_allowed].T).tolist()
            # random tile boundaries
            cuts = sorted(set(rng.integers(1, n_allowed, size=4).tolist())) if n_allowed > 1 else []
            bounds = [0] + cuts + [n_allowed]
            tiles = list(zip(bounds[:-1], bounds[1:]))
            one = finish(streaming_row(s1, s2, tiles))
            # split the key range into parts, stream each, then merge the states
            parts = [streaming_row(s1, s2, [t]) for t in tiles]
            merged = finish(merge_states(parts))
            for got in (one, merged):
                assert abs(got[0] - kl[i]) <= 1e-12, (causal, i, got[0], kl[i])
                assert abs(got[1] - l1[i]) <= 1e-12 and abs(got[2] - l2[i]) <= 1e-12


# ---- P2': the multi-head entry points against one batched library computation ----

def pin_multihead(oracle, seed=7):
    """oracle.forward / oracle.backward on [H, N, d] inputs against torch fp64
    over the whole batch at once (batched matmul, log_softmax, kl_div and
    autograd), with a different upstream weight per head and row."""
    import torch
    rng = np.random.default_rng(seed)
    H, n_q, n_k, d = 3, 10, 14, 6
    for causal in (False, True):
        x = [rng.standard_normal((H, n, d)) for n in (n_q, n_k, n_q, n_k)]
        g = 0.5 + rng.random((H, n_q))
        scale = 0.55
        kl, l1, l2 = oracle.forward(*x, scale, causal)
        i = torch.arange(n_q)[:, None]
        j = torch.arange(n_k)[None, :]
        allowed = (j <= i + (n_k - n_q)) if causal else torch.ones(n_q, n_k, dtype=torch.bool)
        for setting in (1, 2):
            t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in x]
            s1 = (scale * torch.matmul(t[0], t[1].transpose(1, 2).contiguous())).masked_fill(~allowed, -1e30)
            s2 = (scale * torch.matmul(t[2], t[3].transpose(1, 2).contiguous())).masked_fill(~allowed, -1e30)
            assert np.allclose(l1, torch.logsumexp(s1, -1).detach().numpy(), rtol=1e-12, atol=1e-12)
            assert np.allclose(l2, torch.logsumexp(s2, -1).detach().numpy(), rtol=1e-12, atol=1e-12)
            lp1, lp2 = torch.log_softmax(s1, -1), torch.log_softmax(s2, -1)
            lp1, lp2 = (lp1.detach(), lp2) if setting == 1 else (lp1, lp2.detach())
            tkl = torch.nn.functional.kl_div(lp2, lp1, reduction="none", log_target=True).sum(-1)
            assert np.allclose(kl, tkl.detach().numpy(), rtol=1e-11, atol=1e-13)
            (torch.tensor(g) * tkl).sum().backward()
            dq, dk = oracle.backward(setting, *x, scale, causal, g)
            iq, ik = (2, 3) if setting == 1 else (0, 1)
            assert np.allclose(dq, t[iq].grad.numpy(), rtol=1e-10, atol=1e-13), setting
            assert np.allclose(dk, t[ik].grad.numpy(), rtol=1e-10, atol=1e-13), setting


ALL_PINS = [pin_brute_force, pin_bernoulli, pin_torch_autograd, pin_invariants,
            pin_uniform_teacher, pin_finite_differences, pin_streaming_identity, pin_multihead]
