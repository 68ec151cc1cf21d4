"""Pins of the local-window + global-anchor oracle (oracle/local.py).

Each pin takes fn(q, k, v, scale, n_global, map_w, win_rows, win_cols, causal)
-> (O, L) for one head and raises on a mismatch. They fix the pattern from
outside the oracle: a pure-Python brute force that lays the tokens out on
the map by walking it, reductions to the (separately pinned) banded and
plain oracles, closed forms and the symmetry of the pattern.
"""
import math

import numpy as np

from oracle import attention


def _rand(N, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.standard_normal((N, d))


def _brute(q, k, v, scale, G, W, wr, wc, causal):
    """Pure Python: tokens G.. are placed on the map one by one, row by row."""
    N = len(q)
    place = {}
    r = c = 0
    for t in range(G, N):
        place[t] = (r, c)
        c += 1
        if c == W:
            r, c = r + 1, 0
    O, L = [], []
    for i in range(N):
        ws, idx = [], []
        for j in range(N):
            if causal and j > i:
                continue
            if i < G or j < G:
                ok = True
            else:
                (ri, ci), (rj, cj) = place[i], place[j]
                ok = -wr <= ri - rj <= wr and -wc <= ci - cj <= wc
            if ok:
                s = scale * math.fsum(q[i][e] * k[j][e] for e in range(len(q[i])))
                ws.append(math.exp(s))   # small scores: no max subtraction needed
                idx.append(j)
        tot = math.fsum(ws)
        O.append([math.fsum(w * v[j][e] for w, j in zip(ws, idx)) / tot for e in range(len(v[0]))])
        L.append(math.log(tot))
    return np.array(O), np.array(L)


CASES = [  # N, G, W, wr, wc, causal
    (1, 0, 1, 0, 0, False), (7, 0, 3, 1, 1, False), (9, 2, 3, 0, 1, False), (11, 3, 4, 1, 0, True),
    (12, 1, 5, 2, 2, False), (10, 4, 2, 0, 0, False), (13, 0, 4, 1, 2, True), (6, 6, 2, 1, 1, False),
    (8, 2, 100, 0, 1, False), (9, 0, 1, 2, 0, True),
]


def pin_brute_force(fn):
    for n, (N, G, W, wr, wc, causal) in enumerate(CASES):
        q, k, v = _rand(N, 3, 700 + n)
        O, L = fn(q, k, v, 0.6, G, W, wr, wc, causal)
        Ob, Lb = _brute(q.tolist(), k.tolist(), v.tolist(), 0.6, G, W, wr, wc, causal)
        np.testing.assert_allclose(O, Ob, atol=1e-12, err_msg=str(CASES[n]))
        np.testing.assert_allclose(L, Lb, atol=1e-12, err_msg=str(CASES[n]))


def pin_one_column_map_is_a_band(fn):
    """No anchors and a map one token wide: the window is the band (wr, wr) of
    the token order ((wr, 0) when causal)."""
    for causal in (False, True):
        for wr in (0, 1, 3):
            q, k, v = _rand(10, 4, 710 + wr)
            O, L = fn(q, k, v, 0.5, 0, 1, wr, 5, causal)
            Ob, Lb = attention(q, k, v, 0.5, window=(wr, 0 if causal else wr))
            np.testing.assert_allclose(O, Ob, atol=1e-12)
            np.testing.assert_allclose(L, Lb, atol=1e-12)


def pin_one_row_map_is_a_band(fn):
    """No anchors and a map one row long: the window is the band (wc, wc)."""
    q, k, v = _rand(9, 4, 720)
    O, L = fn(q, k, v, 0.5, 0, 9, 0, 2, False)
    Ob, Lb = attention(q, k, v, 0.5, window=(2, 2))
    np.testing.assert_allclose(O, Ob, atol=1e-12)
    np.testing.assert_allclose(L, Lb, atol=1e-12)


def pin_full_window_or_all_anchors_is_plain(fn):
    """A window wider than the map, or every token an anchor: plain attention."""
    for causal in (False, True):
        q, k, v = _rand(11, 3, 730 + causal)
        for G, W, wr, wc in ((2, 3, 5, 5), (11, 2, 0, 0), (0, 4, 10, 3)):
            O, L = fn(q, k, v, 0.7, G, W, wr, wc, causal)
            Ob, Lb = attention(q, k, v, 0.7, causal)
            np.testing.assert_allclose(O, Ob, atol=1e-12)
            np.testing.assert_allclose(L, Lb, atol=1e-12)


def pin_diagonal_closed_form(fn):
    """No anchors, window (0, 0): each token sees only itself, O_i = v_i and
    L_i = scale q_i . k_i."""
    q, k, v = _rand(8, 3, 740)
    O, L = fn(q, k, v, 0.9, 0, 3, 0, 0, False)
    np.testing.assert_allclose(O, v, atol=1e-12)
    np.testing.assert_allclose(L, 0.9 * np.sum(q * k, axis=1), atol=1e-12)


def pin_anchors_plus_self_closed_form(fn):
    """Window (0, 0) with G anchors: a map query sees the anchors and itself;
    an anchor query sees every key."""
    N, G = 9, 3
    q, k, v = _rand(N, 3, 750)
    O, L = fn(q, k, v, 0.8, G, 2, 0, 0, False)
    for i in range(N):
        keys = list(range(N)) if i < G else list(range(G)) + [i]
        s = 0.8 * k[keys] @ q[i]
        w = np.exp(s - s.max())
        np.testing.assert_allclose(O[i], (w / w.sum()) @ v[keys], atol=1e-12)
        np.testing.assert_allclose(L[i], s.max() + np.log(w.sum()), atol=1e-12)


def pin_zero_scores_closed_form(fn):
    """Keys that a query sees can be told apart only through their scores: with
    all scores zero (q = 0), O_i is the mean of the visible V rows and L_i =
    ln(count), where the count comes from a closed form on a full map (no
    anchors): (rows in reach) x (columns in reach)."""
    h, W, wr, wc = 4, 5, 1, 2
    N = h * W
    q = np.zeros((N, 2))
    _, k, v = _rand(N, 2, 760)
    O, L = fn(q, k, v, 1.0, 0, W, wr, wc, False)
    for i in range(N):
        r, c = divmod(i, W)
        rows = range(max(0, r - wr), min(h - 1, r + wr) + 1)
        cols = range(max(0, c - wc), min(W - 1, c + wc) + 1)
        keys = [rr * W + cc for rr in rows for cc in cols]
        np.testing.assert_allclose(L[i], math.log(len(keys)), atol=1e-12)
        np.testing.assert_allclose(O[i], v[keys].mean(axis=0), atol=1e-12)


def pin_symmetry(fn):
    """Non-causal, the pattern is symmetric: swapping the roles of q and k
    gives the transposed score mask, so with v = I the probabilities
    P(q, k) and P(k, q) share their zero pattern transposed."""
    N = 10
    q, k, _ = _rand(N, 3, 770)
    v = np.eye(N)
    P1, _ = fn(q, k, v, 0.4, 2, 3, 1, 0, False)
    P2, _ = fn(k, q, v, 0.4, 2, 3, 1, 0, False)
    assert np.array_equal(P1 > 0, (P2 > 0).T)


LOCAL_PINS = [pin_brute_force, pin_one_column_map_is_a_band, pin_one_row_map_is_a_band,
              pin_full_window_or_all_anchors_is_plain, pin_diagonal_closed_form,
              pin_anchors_plus_self_closed_form, pin_zero_scores_closed_form,
              pin_symmetry]
