"""Blockwise online-softmax attention forward in float64, as the pages lay it out.

TEST INFRASTRUCTURE ONLY (see the package docstring). This is a second,
independent route to the same result as attention.attention; the CPU tests
check that the two agree, which pins the definition against the algorithm.

Source: "FlashAttention/zh" (marovi.ai wiki), section FlashAttention 算法
(the algorithm), whose steps are:
  1. split Q into blocks of B_r rows and K, V into blocks of B_c rows;
  2. for each query block Q_i start from O_i = 0, m_i = -inf, l_i = 0;
  3. for each key/value block compute S_ij = Q_i K_j^T * scale, its row
     maxima m_ij and the local exponentials P~_ij = e^{S_ij - m_ij};
  4. merge: m_new = max(m_i, m_ij); rescale O_i and l_i by e^{m_i - m_new};
     add P~_ij V_j * e^{m_ij - m_new} to O_i and rowsum(P~_ij) * e^{m_ij - m_new}
     to l_i;
  5. after the last block, O_i / l_i is the output and L_i = m_i + log l_i.

form="running" takes the equivalent update of "YOLOv12官版镜像集成Flash
Attention v2，提速原理浅析" (section 3.2): the block's exponentials are taken
against the new running maximum directly, l_new = l_old e^{m_old - m_new} +
sum e^{s - m_new}. The two are equal in exact arithmetic.

Reading where the pages are silent: with a causal or banded mask a block can
be fully masked for some rows (m_ij = -inf). Such a row's block contributes
nothing: its exponentials are 0 and its merge factor e^{m_ij - m_new} is taken
as 0. A row that sees no key at all ends with l = 0; its output is 0 and
L = -inf. The band (window = (left, right)) is the one attention.py defines:
query i sees key j iff i + off - left <= j <= i + off + right, off = Nk - Nq.
"""
from __future__ import annotations

import numpy as np


def attention_tiled(q, k, v, scale: float, causal: bool = False,
                    block_rows: int = 16, block_cols: int = 16, form: str = "local",
                    window=None):
    """One head, blockwise. Returns (O (Nq,dv), L (Nq,)) in float64."""
    if form not in ("local", "running"):
        raise ValueError(form)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq != Nk:
        raise ValueError("causal attention is defined here only for Nq == Nk")
    O = np.zeros((Nq, v.shape[1]))
    L = np.zeros(Nq)
    for r0 in range(0, Nq, block_rows):
        r1 = min(r0 + block_rows, Nq)
        Qi = q[r0:r1]
        Oi = np.zeros((r1 - r0, v.shape[1]))
        mi = np.full(r1 - r0, -np.inf)
        li = np.zeros(r1 - r0)
        for c0 in range(0, Nk, block_cols):
            c1 = min(c0 + block_cols, Nk)
            Sij = scale * (Qi @ k[c0:c1].T)
            rows = np.arange(r0, r1)[:, None]
            cols = np.arange(c0, c1)[None, :]
            if causal:
                Sij = np.where(cols > rows, -np.inf, Sij)
            if window is not None:
                left, right = window
                lo = rows + (Nk - Nq) - (left if left is not None else Nk + Nq)
                hi = rows + (Nk - Nq) + (right if right is not None else Nk + Nq)
                Sij = np.where((cols < lo) | (cols > hi), -np.inf, Sij)
            mij = Sij.max(axis=1)
            m_new = np.maximum(mi, mij)
            # e^{m_i - m_new}; a row that has seen nothing yet has O_i = l_i = 0.
            alpha = np.where(np.isneginf(mi), 0.0, np.exp(mi - np.where(np.isneginf(m_new), 0.0, m_new)))
            if form == "local":
                seen = ~np.isneginf(mij)
                safe_mij = np.where(seen, mij, 0.0)
                Pij = np.where(seen[:, None], np.exp(Sij - safe_mij[:, None]), 0.0)
                beta = np.where(seen, np.exp(safe_mij - np.where(seen, m_new, 0.0)), 0.0)
                Oi = Oi * alpha[:, None] + (Pij @ v[c0:c1]) * beta[:, None]
                li = li * alpha + Pij.sum(axis=1) * beta
            else:
                seen = ~np.isneginf(m_new)
                safe_m = np.where(seen, m_new, 0.0)
                Pij = np.where(seen[:, None], np.exp(Sij - safe_m[:, None]), 0.0)
                Oi = Oi * alpha[:, None] + Pij @ v[c0:c1]
                li = li * alpha + Pij.sum(axis=1)
            mi = m_new
        empty = li == 0
        O[r0:r1] = Oi / np.where(empty, 1.0, li)[:, None]
        with np.errstate(divide="ignore"):
            L[r0:r1] = np.where(empty, -np.inf, mi + np.log(np.where(empty, 1.0, li)))
    return O, L
