"""Plain float64 attention backward: the gradients of the definition.

TEST INFRASTRUCTURE ONLY (see the package docstring). Parity: pinned by the
CPU tests (central finite differences of the forward definition, torch
autograd in float64, invariants and closed forms, planted mistakes).

Sources (page titles and sections):
  * "FlashAttention/zh" (marovi.ai wiki), section 為何標準注意力運行緩慢:
    O = P V with P = softmax(S), S = Q K^T scaled.
  * same page, section 反向傳遞與重計算 (backward pass and recomputation):
    the backward needs P, and FlashAttention does not keep it: it recomputes
    S and P from the saved log-sum-exp L and the incoming gradient dO. With
    L_i = m_i + ln l_i from the forward, P_ij = exp(S_ij - L_i) exactly.

The pages give no gradient formulas; these are the chain rule through the
definition (the plainest reading), for a loss whose gradient with respect to
O is dO:
    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij (dP_ij - D_i),   D_i = sum_j P_ij dP_ij   (= dO_i . O_i)
    dQ = scale dS K
    dK = scale dS^T Q
The masks are those of the forward: causal (query i sees keys j <= i, Nq ==
Nk), the banded mask (window, as in attention.py) and the key padding mask
(as in padding.py: remove the padding, take the gradients of the valid
tokens, put them back with zeros at padding positions). Masked pairs have
P = 0 and so carry no gradient; a row that sees no key has P = 0 and D = 0.
"""
from __future__ import annotations

import numpy as np

from .attention import ORACLE_DTYPE, attention_probs


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=ORACLE_DTYPE)


def attention_backward(q, k, v, do, scale: float, causal: bool = False, window=None):
    """One head: q (Nq,d), k (Nk,d), v (Nk,dv), do (Nq,dv) -> (dq, dk, dv, delta), float64.

    delta is D_i = sum_j P_ij dP_ij, the per-row term of the softmax gradient.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    P = attention_probs(q, k, scale, causal, window=window)   # (Nq, Nk), masked entries 0
    dv = P.T @ do
    dP = do @ v.T
    delta = np.sum(P * dP, axis=1)
    dS = P * (dP - delta[:, None])
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    return dq, dk, dv, delta


def attention_backward_dense(q, k, v, do, scale: float, causal: bool = False,
                             batches=None, heads=None, window=None):
    """Equal-length batch, (B, N, H, d) layouts. Returns dq, dk, dv in the input
    layouts (for the selected batches and heads) and delta (nb, nh, Nq)."""
    B, Nq, H, _ = q.shape
    Nk = k.shape[1]
    bs = range(B) if batches is None else list(batches)
    hs = range(H) if heads is None else list(heads)
    dq = np.zeros((len(bs), Nq, len(hs), q.shape[3]), dtype=ORACLE_DTYPE)
    dk = np.zeros((len(bs), Nk, len(hs), k.shape[3]), dtype=ORACLE_DTYPE)
    dv = np.zeros((len(bs), Nk, len(hs), v.shape[3]), dtype=ORACLE_DTYPE)
    delta = np.zeros((len(bs), len(hs), Nq), dtype=ORACLE_DTYPE)
    for bi, b in enumerate(bs):
        for hi, h in enumerate(hs):
            g = attention_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, causal,
                                   window)
            dq[bi, :, hi], dk[bi, :, hi], dv[bi, :, hi], delta[bi, hi] = g
    return dq, dk, dv, delta


def attention_backward_varlen(q, k, v, do, cu_seqlens, scale: float, causal: bool = False,
                              window=None):
    """Packed batch, (total, H, d) layouts; each sequence attends only to itself.
    Returns dq, dk, dv (total, H, d) and delta (H, total)."""
    total, H, _ = q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    dq = np.zeros((total, H, q.shape[2]), dtype=ORACLE_DTYPE)
    dk = np.zeros((total, H, k.shape[2]), dtype=ORACLE_DTYPE)
    dv = np.zeros((total, H, v.shape[2]), dtype=ORACLE_DTYPE)
    delta = np.zeros((H, total), dtype=ORACLE_DTYPE)
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        for h in range(H):
            g = attention_backward(q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h], scale, causal,
                                   window)
            dq[a:b, h], dk[a:b, h], dv[a:b, h], delta[h, a:b] = g
    return dq, dk, dv, delta


def attention_backward_padded(q, k, v, do, mask, scale: float, causal: bool = False):
    """Padded batch (B, S, H, d) with a key padding mask (B, S), nonzero = valid:
    the gradients of the valid tokens' attention, zeros at padding positions;
    delta (B, H, S) is 0 there."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    mask = np.asarray(mask)
    B, S, H, _ = q.shape
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    delta = np.zeros((B, H, S), dtype=ORACLE_DTYPE)
    for b in range(B):
        idx = np.nonzero(mask[b])[0]
        if idx.size == 0:
            continue
        for h in range(H):
            g = attention_backward(q[b, idx, h], k[b, idx, h], v[b, idx, h], do[b, idx, h], scale,
                                   causal)
            dq[b, idx, h], dk[b, idx, h], dv[b, idx, h], delta[b, h, idx] = g
    return dq, dk, dv, delta
