"""Plain float64 attention with a local window on a token map plus global
anchor tokens.

TEST INFRASTRUCTURE ONLY (see the package docstring). Parity: pinned by the
CPU tests (a pure-Python brute force that walks the map, reductions to the
pinned banded and plain oracles, closed forms, a closed-form pair count,
planted mistakes; the gradients by central finite differences of the pinned
forward and by the pinned banded backward).

Sources (page titles and sections):
  * "YOLOv12官版镜像集成Flash Attention v2，提速原理浅析", section 4.2 (dynamic
    sparse attention): the detector mixes a local window with a few global
    tokens; each token attends only its neighbourhood on the feature map (a
    5 x 5 window is the page's example) plus a small set of global anchors.
    Window attention restricts the range of key blocks and skips the rest;
    the anchors' K and V are loaded on their own and attended by the
    windowed queries.
  * same page, section 4.1: the tokens are the cells of a 40 x 40 map (1600
    tokens).
  * "FlashAttention/zh" (marovi.ai wiki), section 為何標準注意力運行緩慢: the
    attention itself, softmax(scale q k^T) v, with L = m + ln l as in
    attention.py.

Readings where the page is silent:
  * The anchors are the first n_global tokens of the sequence; the other
    N - n_global tokens are the map, in row-major order with map_w tokens
    per row (token t >= n_global sits at row (t - n_global) // map_w, column
    (t - n_global) % map_w; the last row may be short).
  * Query i sees key j iff
        (i < n_global  or  j < n_global  or  the map positions of i and j
         differ by at most win_rows rows and at most win_cols columns)
    and, when causal, j <= i. So every query sees the anchors, and an anchor
    query, being a global token, sees every key.
  * Every row sees at least one key (itself), so no row is empty.
"""
from __future__ import annotations

import numpy as np

from .attention import ORACLE_DTYPE


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=ORACLE_DTYPE)


def local_visible(N: int, n_global: int, map_w: int, win_rows: int, win_cols: int,
                  causal: bool = False) -> np.ndarray:
    """The (N, N) boolean mask: entry (i, j) says whether query i sees key j."""
    if map_w < 1 or win_rows < 0 or win_cols < 0 or n_global < 0:
        raise ValueError("map_w >= 1, win_rows >= 0, win_cols >= 0, n_global >= 0")
    t = np.arange(N)
    is_anchor = t < n_global
    pos = np.maximum(t - n_global, 0)
    row, col = pos // map_w, pos % map_w
    near = (np.abs(row[:, None] - row[None, :]) <= win_rows) & \
           (np.abs(col[:, None] - col[None, :]) <= win_cols)
    vis = is_anchor[:, None] | is_anchor[None, :] | near
    if causal:
        vis &= t[None, :] <= t[:, None]
    return vis


def attention_local(q, k, v, scale: float, n_global: int, map_w: int, win_rows: int,
                    win_cols: int, causal: bool = False):
    """One head: q, k (N, d), v (N, dv) -> (O (N, dv), L (N,)), float64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    N = q.shape[0]
    if k.shape[0] != N:
        raise ValueError("the local pattern is defined for self-attention (Nq == Nk)")
    if N == 0:
        return np.zeros((0, v.shape[1])), np.zeros((0,))
    S = scale * (q @ k.T)
    S = np.where(local_visible(N, n_global, map_w, win_rows, win_cols, causal), S, -np.inf)
    m = np.max(S, axis=1, keepdims=True)      # finite: every row sees itself
    e = np.exp(S - m)
    l = np.sum(e, axis=1, keepdims=True)
    return (e / l) @ v, m[:, 0] + np.log(l[:, 0])


def attention_local_dense(q, k, v, scale: float, n_global: int, map_w: int, win_rows: int,
                          win_cols: int, causal: bool = False, batches=None, heads=None):
    """(B, N, H, d) tensors -> O (nb, N, nh, d) and L (nb, nh, N) for the selected
    batches and heads (None = all)."""
    B, N, H, _ = q.shape
    bs = range(B) if batches is None else list(batches)
    hs = range(H) if heads is None else list(heads)
    O = np.empty((len(bs), N, len(hs), v.shape[3]), dtype=ORACLE_DTYPE)
    L = np.empty((len(bs), len(hs), N), dtype=ORACLE_DTYPE)
    for bi, b in enumerate(bs):
        for hi, h in enumerate(hs):
            O[bi, :, hi], L[bi, hi] = attention_local(q[b, :, h], k[b, :, h], v[b, :, h], scale,
                                                      n_global, map_w, win_rows, win_cols, causal)
    return O, L


def local_pairs(N: int, n_global: int, map_w: int, win_rows: int, win_cols: int,
                causal: bool = False) -> int:
    """Number of visible (query, key) pairs (for FLOP counts)."""
    return int(np.count_nonzero(local_visible(N, n_global, map_w, win_rows, win_cols, causal)))


def attention_local_backward(q, k, v, do, scale: float, n_global: int, map_w: int,
                             win_rows: int, win_cols: int, causal: bool = False):
    """One head: gradients of attention_local for a loss with dL/dO = do, by the
    chain rule through the definition (as in backward.py: dV = P^T dO,
    dS = P (dO V^T - D), D_i = sum_j P_ij (dO V^T)_ij, dQ = scale dS K,
    dK = scale dS^T Q) with P the local pattern's probabilities.
    Returns (dq, dk, dv, delta), float64."""
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    N = q.shape[0]
    S = scale * (q @ k.T)
    S = np.where(local_visible(N, n_global, map_w, win_rows, win_cols, causal), S, -np.inf)
    e = np.exp(S - np.max(S, axis=1, keepdims=True))
    P = e / np.sum(e, axis=1, keepdims=True)
    dP = do @ v.T
    delta = np.sum(P * dP, axis=1)
    dS = P * (dP - delta[:, None])
    return scale * (dS @ k), scale * (dS.T @ q), P.T @ do, delta


def attention_local_backward_dense(q, k, v, do, scale: float, n_global: int, map_w: int,
                                   win_rows: int, win_cols: int, causal: bool = False):
    """(B, N, H, d) tensors -> dq, dk, dv in the input layouts and delta (B, H, N)."""
    B, N, H, _ = q.shape
    dq, dk, dv = (np.zeros(x.shape, dtype=ORACLE_DTYPE) for x in (q, k, v))
    delta = np.zeros((B, H, N), dtype=ORACLE_DTYPE)
    for b in range(B):
        for h in range(H):
            dq[b, :, h], dk[b, :, h], dv[b, :, h], delta[b, h] = attention_local_backward(
                q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], scale, n_global, map_w,
                win_rows, win_cols, causal)
    return dq, dk, dv, delta
