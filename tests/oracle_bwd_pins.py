"""Pins for a single-head backward fn(q, k, v, do, scale, causal) -> (dq, dk, dv, delta).

Each pin checks fn against something other than its own formula: central
finite differences of the forward definition (itself pinned), torch autograd
through explicit float64 softmax ops, closed forms for two keys, one key and
Q = 0, and invariants the mathematics fixes. test_oracle.py runs them on the
oracle; test_oracle_mutants.py checks that planted mistakes fail one.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import attention
from tests.oracle_pins import _close, _rng


def _loss_grad_fd(q, k, v, do, scale, causal, h=1e-6):
    """Gradients of sum(dO * O(q, k, v)) by central differences of the forward oracle."""
    def loss(q_, k_, v_):
        O, _ = attention(q_, k_, v_, scale, causal)
        return float(np.sum(O * do))
    grads = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        g = np.zeros_like(args[which])
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() for a in args]
            minus = [a.copy() for a in args]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


def pin_bwd_finite_differences(fn):
    rng = _rng(201)
    for Nq, Nk, d, causal in [(1, 1, 2, False), (2, 3, 2, False), (3, 3, 3, True), (5, 4, 2, False),
                              (4, 4, 1, True), (3, 6, 3, False)]:
        q, k, v = (rng.standard_normal((n, d)) for n in (Nq, Nk, Nk))
        do = rng.standard_normal((Nq, d))
        scale = float(rng.uniform(0.3, 1.2))
        dq, dk, dv, _ = fn(q, k, v, do, scale, causal)
        fq, fk, fv = _loss_grad_fd(q, k, v, do, scale, causal)
        what = f"Nq={Nq} Nk={Nk} d={d} causal={causal}"
        _close(dq, fq, 1e-7, "dq vs finite differences " + what)
        _close(dk, fk, 1e-7, "dk vs finite differences " + what)
        _close(dv, fv, 1e-7, "dv vs finite differences " + what)


def pin_bwd_autograd(fn):
    import torch
    rng = _rng(203)
    for Nq, Nk, d, causal in [(9, 9, 8, True), (9, 9, 8, False), (6, 13, 4, False)]:
        q, k, v = (rng.standard_normal((n, d)) for n in (Nq, Nk, Nk))
        do = rng.standard_normal((Nq, d))
        scale = 0.37
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        S = scale * tq @ tk.T
        if causal:
            S = S.masked_fill(torch.triu(torch.ones(Nq, Nk, dtype=torch.bool), 1), float("-inf"))
        O = torch.softmax(S, dim=1) @ tv
        O.backward(torch.from_numpy(do))
        dq, dk, dv, _ = fn(q, k, v, do, scale, causal)
        _close(dq, tq.grad.numpy(), 1e-12, "dq vs autograd")
        _close(dk, tk.grad.numpy(), 1e-12, "dk vs autograd")
        _close(dv, tv.grad.numpy(), 1e-12, "dv vs autograd")


def pin_bwd_two_keys(fn):
    """Nq = 1, Nk = 2, d = 1: O = p v0 + (1 - p) v1 with p = sigmoid(c q (k0 - k1)), so
    dq = dO c p (1-p) (k0-k1)(v0-v1), dk0 = -dk1 = dO c q p (1-p) (v0-v1),
    dv0 = dO p, dv1 = dO (1-p)."""
    for (q, k0, k1, v0, v1, do, c) in [(0.7, 1.3, -0.4, 2.0, -1.0, 0.9, 0.8),
                                        (-1.1, 0.2, 0.5, -0.3, 1.7, -2.0, 1.5)]:
        p = 1 / (1 + math.exp(-c * q * (k0 - k1)))
        dq, dk, dv, delta = fn(np.array([[q]]), np.array([[k0], [k1]]), np.array([[v0], [v1]]),
                               np.array([[do]]), c, False)
        _close(dq, [[do * c * p * (1 - p) * (k0 - k1) * (v0 - v1)]], 1e-12, "two keys dq")
        g = do * c * q * p * (1 - p) * (v0 - v1)
        _close(dk, [[g], [-g]], 1e-12, "two keys dk")
        _close(dv, [[do * p], [do * (1 - p)]], 1e-12, "two keys dv")
        _close(delta, [do * (p * v0 + (1 - p) * v1)], 1e-12, "two keys delta")


def pin_bwd_single_key(fn):
    """One visible key: P = 1 whatever q and k are, so dq = dk = 0 and dv0 = sum of dO."""
    rng = _rng(207)
    q, k, v, do = rng.standard_normal((4, 3)), rng.standard_normal((1, 3)), \
        rng.standard_normal((1, 3)), rng.standard_normal((4, 3))
    dq, dk, dv, _ = fn(q, k, v, do, 0.9, False)
    _close(dq, np.zeros_like(q), 1e-12, "single key dq")
    _close(dk, np.zeros_like(k), 1e-12, "single key dk")
    _close(dv, do.sum(axis=0, keepdims=True), 1e-12, "single key dv")


def pin_bwd_zero_query(fn):
    """Q = 0: P_ij = 1/n_i over the n_i visible keys, so dk = 0,
    dv_j = sum over rows i that see j of dO_i / n_i, and
    dq_i = scale/n_i sum_j (dP_ij - mean_j dP_ij) k_j with dP_ij = dO_i . v_j."""
    rng = _rng(209)
    for causal in (False, True):
        N, d = 6, 3
        q = np.zeros((N, d))
        k, v, do = (rng.standard_normal((N, d)) for _ in range(3))
        scale = 0.6
        dq, dk, dv, _ = fn(q, k, v, do, scale, causal)
        dv_want = np.zeros((N, d))
        dq_want = np.zeros((N, d))
        for i in range(N):
            vis = list(range(i + 1)) if causal else list(range(N))
            n = len(vis)
            dp = [float(do[i] @ v[j]) for j in vis]
            mean = sum(dp) / n
            for j, dpj in zip(vis, dp):
                dv_want[j] += do[i] / n
                dq_want[i] += scale / n * (dpj - mean) * k[j]
        _close(dk, np.zeros_like(k), 1e-12, f"zero-Q dk causal={causal}")
        _close(dv, dv_want, 1e-12, f"zero-Q dv causal={causal}")
        _close(dq, dq_want, 1e-12, f"zero-Q dq causal={causal}")


def pin_bwd_invariants(fn):
    """Shifting every key by one vector leaves O unchanged, so the dk rows sum to 0;
    P rows sum to 1, so the dv rows sum to the dO rows' sum; delta_i = dO_i . O_i
    with O from the forward definition."""
    rng = _rng(211)
    for Nq, Nk, causal in [(7, 7, True), (5, 9, False)]:
        q, k, v = (rng.standard_normal((n, 4)) for n in (Nq, Nk, Nk))
        do = rng.standard_normal((Nq, 4))
        dq, dk, dv, delta = fn(q, k, v, do, 0.5, causal)
        _close(dk.sum(axis=0), np.zeros(4), 1e-12, "sum of dk rows")
        _close(dv.sum(axis=0), do.sum(axis=0), 1e-12, "sum of dv rows")
        O, _ = attention(q, k, v, 0.5, causal)
        _close(delta, np.sum(do * O, axis=1), 1e-12, "delta = rowsum(dO * O)")


def pin_bwd_zero_grad(fn):
    rng = _rng(213)
    q, k, v = (rng.standard_normal((5, 3)) for _ in range(3))
    dq, dk, dv, delta = fn(q, k, v, np.zeros((5, 3)), 0.7, True)
    for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (delta, "delta")):
        _close(x, np.zeros_like(x), 0.0, f"zero dO gives zero {n}")


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_autograd, pin_bwd_two_keys, pin_bwd_single_key,
            pin_bwd_zero_query, pin_bwd_invariants, pin_bwd_zero_grad]
