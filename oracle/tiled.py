"""Blockwise (online-softmax) attention forward in float64: a second route.

TEST INFRASTRUCTURE ONLY (see the package docstring). It reaches the same
result as attention.attention by a different evaluation order; the CPU tests
check that the two agree, which pins the definition against the blockwise
method the pages describe ("FlashAttention/zh" (marovi.ai wiki), sections
在線 softmax 技巧 and FlashAttention 算法; "YOLOv12官版镜像集成Flash
Attention v2，提速原理浅析", section 3.2).

Structure. For one query block, every key block yields a partial summary
(m, l, A): the row maxima m of its scores, the sums l of e^{s - m} and the
unnormalised outputs A = e^{s - m} V. Two summaries over disjoint key sets
combine exactly into the summary of their union:

    m = max(m1, m2),  l = l1 e^{m1 - m} + l2 e^{m2 - m},
    A = A1 e^{m1 - m} + A2 e^{m2 - m},

and O = A / l, L = m + ln l at the end. The combination is associative and
commutative, so any grouping of the key blocks gives the same result:
  form="local"   folds the block summaries left to right;
  form="tree"    combines them pairwise, as a balanced tree;
  form="running" never forms a block summary: it keeps one running triple and
                 exponentiates each block against the already-updated maximum
                 (the update of the YOLOv12 page, section 3.2).

Reading where the pages are silent: with a causal or banded mask, a row can
see no key of a block (m = -inf). Such a summary is the identity of the
combination (l = 0, A = 0) and contributes nothing. A row that sees no key
at all ends with l = 0: its output is 0 and L = -inf. The band (window =
(left, right)) is the one attention.py defines: query i sees key j iff
i + off - left <= j <= i + off + right, off = Nk - Nq.
"""
from __future__ import annotations

import numpy as np


def _scores(Qi, k, r0, c0, c1, scale, causal, window, Nq, Nk):
    """Scaled scores of query rows r0.. against keys [c0, c1), masked to -inf."""
    S = scale * (Qi @ k[c0:c1].T)
    rows = np.arange(r0, r0 + Qi.shape[0])[:, None]
    cols = np.arange(c0, c1)[None, :]
    hidden = np.zeros(S.shape, dtype=bool)
    if causal:
        hidden |= cols > rows
    if window is not None:
        left, right = window
        big = Nk + Nq
        lo = rows + (Nk - Nq) - (big if left is None else left)
        hi = rows + (Nk - Nq) + (big if right is None else right)
        hidden |= (cols < lo) | (cols > hi)
    return np.where(hidden, -np.inf, S)


def _shift(x, m):
    """e^{x - m} per row, 0 where the row's m is -inf (nothing seen)."""
    finite = ~np.isneginf(m)
    safe = np.where(finite, m, 0.0)
    return np.where(finite[:, None] if x.ndim == 2 else finite,
                    np.exp(x - (safe[:, None] if x.ndim == 2 else safe)), 0.0)


def _summary(S, Vj):
    """(m, l, A) of one key block: block maxima, sums and unnormalised outputs."""
    m = S.max(axis=1)
    E = _shift(S, m)
    return m, E.sum(axis=1), E @ Vj


def _combine(a, b):
    """Summary of the union of two disjoint key sets."""
    m1, l1, A1 = a
    m2, l2, A2 = b
    m = np.maximum(m1, m2)
    f1 = _shift(m1, m)        # e^{m1 - m}; 0 if the first part saw nothing
    f2 = _shift(m2, m)
    return m, l1 * f1 + l2 * f2, A1 * f1[:, None] + A2 * f2[:, None]


def _finish(summary):
    m, l, A = summary
    empty = l == 0
    O = A / np.where(empty, 1.0, l)[:, None]
    with np.errstate(divide="ignore"):
        L = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, l)))
    return O, L


def attention_tiled(q, k, v, scale: float, causal: bool = False,
                    block_rows: int = 16, block_cols: int = 16, form: str = "local",
                    window=None):
    """One head, blockwise. Returns (O (Nq,dv), L (Nq,)) in float64."""
    if form not in ("local", "tree", "running"):
        raise ValueError(form)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq != Nk:
        raise ValueError("causal attention is defined here only for Nq == Nk")
    dv = v.shape[1]
    O = np.zeros((Nq, dv))
    L = np.zeros(Nq)
    for r0 in range(0, Nq, block_rows):
        Qi = q[r0:r0 + block_rows]
        n = Qi.shape[0]
        empty = (np.full(n, -np.inf), np.zeros(n), np.zeros((n, dv)))
        blocks = [(c0, min(c0 + block_cols, Nk)) for c0 in range(0, Nk, block_cols)]
        if form == "running":
            m, l, A = empty
            for c0, c1 in blocks:
                S = _scores(Qi, k, r0, c0, c1, scale, causal, window, Nq, Nk)
                m_new = np.maximum(m, S.max(axis=1))
                f = _shift(m, m_new)
                E = _shift(S, m_new)
                m, l, A = m_new, l * f + E.sum(axis=1), A * f[:, None] + E @ v[c0:c1]
            total = (m, l, A)
        else:
            parts = [_summary(_scores(Qi, k, r0, c0, c1, scale, causal, window, Nq, Nk),
                              v[c0:c1]) for c0, c1 in blocks]
            if form == "local":
                total = empty
                for p in parts:
                    total = _combine(total, p)
            else:
                while len(parts) > 1:
                    nxt = [_combine(parts[i], parts[i + 1]) for i in range(0, len(parts) - 1, 2)]
                    if len(parts) % 2:
                        nxt.append(parts[-1])
                    parts = nxt
                total = parts[0] if parts else empty
        O[r0:r0 + n], L[r0:r0 + n] = _finish(total)
    return O, L
