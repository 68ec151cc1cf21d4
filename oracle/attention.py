"""Plain float64 attention: the definition, written out.

TEST INFRASTRUCTURE ONLY (see the package docstring). Parity: every function
here is pinned by the CPU tests (brute force, closed forms, invariances, a
library cross-check and hand-derived golden cases).

Sources (page titles and sections; the pages are the authority on what is
computed):
  * "FlashAttention/zh" (marovi.ai wiki), section 為何標準注意力運行緩慢
    (why standard attention is slow): Attention(Q,K,V) = softmax(Q K^T / sqrt(d)) V
    with Q, K, V in R^{N x d}; the naive method builds S = Q K^T / sqrt(d),
    applies a row-wise softmax to get P, then multiplies by V.
  * same page, section 在線 softmax 技巧 (online softmax): the stable softmax
    softmax(x)_i = e^{x_i - m} / l with m = max_i x_i and l = sum_i e^{x_i - m}.
  * same page, section FlashAttention 算法 (the algorithm), last step: the
    forward also stores the log-sum-exp L_i = m_i + log l_i. "log" is read as
    the natural logarithm, matching the e^x of the softmax above.
  * "YOLOv12官版镜像集成Flash Attention v2，提速原理浅析", section 2.2: the safe
    softmax subtracts each row's maximum before exponentiating.
  * "InternViT-6B-448px-V1-2 如何加速注意力计算", section
    FlashAttention 封装类三条执行路径 (变长路径): packed variable-length batches
    described by cumulative sequence lengths; each sequence attends only to
    itself.
  * "FlashAttention/zh", section 變體與後續版本 (variants): the fused kernel
    composes with banded masks; "YOLOv12官版镜像集成Flash Attention v2，提速原理浅析",
    section 4.2 (dynamic sparse attention): each token attends only a local
    window of neighbours, and window attention restricts the range of key
    blocks, skipping the others.

Readings where the pages are silent:
  * The scale is a parameter (the definition's 1/sqrt(d) is the default the
    callers pass); L is computed on the scaled scores.
  * Causal masking (the variants section says the fused kernel supports a
    causal mask) is the lower-triangular mask of self-attention: query i sees
    keys j <= i, and requires as many queries as keys.
  * A banded mask is a band over the token order: with window = (left,
    right), query i sees key j iff i + off - left <= j <= i + off + right,
    where off = Nk - Nq places the last query on the last key (so Nq == Nk
    gives off = 0) and None means no bound on that side. (None, 0) is causal
    attention with that alignment. A two-dimensional image window is not a
    single band; local.py covers it (with the page's global anchors).
  * A row that sees no key (possible only with a band) has the empty sum
    l = 0: its output is 0 and L = ln 0 = -inf.
"""
from __future__ import annotations

import numpy as np

ORACLE_DTYPE = np.float64


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=ORACLE_DTYPE)


def _scores(q, k, scale, causal, rows, window=None):
    """S = scale * q k^T for the requested query rows, masked keys as -inf."""
    Nq, Nk = q.shape[0], k.shape[0]
    if causal and Nq != Nk:
        raise ValueError("causal attention is defined here only for Nq == Nk")
    if causal and window is not None:
        raise ValueError("causal and window are exclusive; causal is window (None, 0)")
    row_idx = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    S = scale * (q[row_idx] @ k.T)
    key_idx = np.arange(Nk)[None, :]
    if causal:
        S = np.where(key_idx > row_idx[:, None], -np.inf, S)
    if window is not None:
        left, right = window
        pos = row_idx[:, None] + (Nk - Nq)   # the query's aligned key position
        visible = np.ones(S.shape, dtype=bool)
        if left is not None:
            visible &= key_idx >= pos - left
        if right is not None:
            visible &= key_idx <= pos + right
        S = np.where(visible, S, -np.inf)
    return S


def _softmax_parts(S):
    """Row max m, exponentials e and sums l; a row with no visible key has m = -inf,
    e = 0 and l = 0 (instead of the NaN of -inf - -inf)."""
    m = np.max(S, axis=1, keepdims=True)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(S - m_safe)
    return m, e, np.sum(e, axis=1, keepdims=True)


def attention_probs(q, k, scale: float, causal: bool = False, rows=None,
                    window=None) -> np.ndarray:
    """P = row-softmax(S), materialised (N_rows x Nk), float64 (rows seeing no key: 0)."""
    q, k = _as64(q), _as64(k)
    _, e, l = _softmax_parts(_scores(q, k, scale, causal, rows, window))
    return e / np.where(l > 0, l, 1.0)


def attention(q, k, v, scale: float, causal: bool = False, rows=None, window=None):
    """One head: q (Nq,d), k (Nk,d), v (Nk,dv) -> (O (rows,dv), L (rows,)) in float64.

    O = softmax(scale * q k^T) v and L_i = m_i + ln l_i, with m_i the row max
    of the (masked) scores and l_i the sum of e^{S_ij - m_i}. `rows` restricts
    the output to a subset of query rows (the mask still uses each row's own
    index); None means all rows. `window` = (left, right) applies the banded
    mask (module docstring); rows that see no key give O = 0 and L = -inf.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    if q.shape[0] == 0:
        return np.zeros((0, v.shape[1])), np.zeros((0,))
    m, e, l = _softmax_parts(_scores(q, k, scale, causal, rows, window))
    P = e / np.where(l > 0, l, 1.0)
    O = P @ v
    with np.errstate(divide="ignore"):
        L = np.where(l[:, 0] > 0, m[:, 0] + np.log(np.where(l[:, 0] > 0, l[:, 0], 1.0)), -np.inf)
    return O, L


def attention_dense(q, k, v, scale: float, causal: bool = False,
                    batches=None, heads=None, rows=None, window=None):
    """Equal-length batch. q (B,Nq,H,d), k/v (B,Nk,H,d) (any real dtype).

    Returns O (nb, nrows, nh, d) and L (nb, nh, nrows) for the selected
    batches / heads / query rows (None = all), looping over (b, h).
    """
    B, Nq, H, _ = q.shape
    bs = range(B) if batches is None else list(batches)
    hs = range(H) if heads is None else list(heads)
    nrows = Nq if rows is None else len(rows)
    O = np.empty((len(bs), nrows, len(hs), v.shape[3]), dtype=ORACLE_DTYPE)
    L = np.empty((len(bs), len(hs), nrows), dtype=ORACLE_DTYPE)
    for bi, b in enumerate(bs):
        for hi, h in enumerate(hs):
            o, lse = attention(q[b, :, h, :], k[b, :, h, :], v[b, :, h, :],
                               scale, causal, rows, window)
            O[bi, :, hi, :] = o
            L[bi, hi, :] = lse
    return O, L


def attention_varlen(q, k, v, cu_seqlens, scale: float, causal: bool = False,
                     seqs=None, heads=None, window=None):
    """Packed batch. q/k/v (total,H,d); cu_seqlens (num_seqs+1,) prefix sums.

    Each sequence s occupies rows [cu[s], cu[s+1]) and attends only to itself.
    Returns O (total,H,d) and L (H,total); rows of sequences not selected in
    `seqs` (and heads not in `heads`) are left as NaN.
    """
    total, H, _ = q.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    O = np.full((total, H, v.shape[2]), np.nan, dtype=ORACLE_DTYPE)
    L = np.full((H, total), np.nan, dtype=ORACLE_DTYPE)
    ss = range(len(cu) - 1) if seqs is None else list(seqs)
    hs = range(H) if heads is None else list(heads)
    for s in ss:
        a, b = int(cu[s]), int(cu[s + 1])
        if b <= a:
            continue
        for h in hs:
            o, lse = attention(q[a:b, h, :], k[a:b, h, :], v[a:b, h, :], scale, causal,
                               window=window)
            O[a:b, h, :] = o
            L[h, a:b] = lse
    return O, L
