"""Pins for a single-head attention function fn(q, k, v, scale, causal) -> (O, L).

Each pin checks fn against something other than itself: a brute-force
evaluation of the definition by a different route, closed forms, invariances
that the mathematics fixes, a library routine, or hand-derived cases. A pin
raises AssertionError (or any exception) when fn is wrong.

test_oracle.py runs every pin on the oracle (all must pass);
test_oracle_mutants.py runs them on planted mistakes in copies of the oracle
(each mistake must fail at least one pin).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


# ---------------------------------------------------------------------------
# 1. Brute force: pure-Python sums with math.fsum and no max subtraction,
#    i.e. O_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij}, L_i = ln sum_j e^{s_ij}.
# ---------------------------------------------------------------------------

def brute_force(q, k, v, scale, causal):
    Nq, Nk = len(q), len(k)
    O, L = [], []
    for i in range(Nq):
        w = []
        for j in range(Nk):
            if causal and j > i:
                continue
            s = scale * math.fsum(q[i][t] * k[j][t] for t in range(len(q[i])))
            w.append((math.exp(s), j))
        Z = math.fsum(e for e, _ in w)
        O.append([math.fsum(e * v[j][c] for e, j in w) / Z for c in range(len(v[0]))])
        L.append(math.log(Z))
    return O, L


def pin_brute_force(fn):
    rng = _rng(101)
    for Nq in (1, 2, 3, 5, 8):
        for Nk in (1, 2, 3, 5, 8):
            for d in (1, 2, 4):
                for causal in (False, True):
                    if causal and Nq != Nk:
                        continue
                    q = rng.standard_normal((Nq, d))
                    k = rng.standard_normal((Nk, d))
                    v = rng.standard_normal((Nk, 3))
                    scale = float(rng.uniform(0.2, 1.5))
                    O, L = fn(q, k, v, scale, causal)
                    Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), scale, causal)
                    _close(O, Ob, 1e-12, f"O brute force Nq={Nq} Nk={Nk} d={d} causal={causal}")
                    _close(L, Lb, 1e-12, f"L brute force Nq={Nq} Nk={Nk} d={d} causal={causal}")


# ---------------------------------------------------------------------------
# 2. The blockwise online-softmax route (any grouping of key blocks) gives the same O and L.
# ---------------------------------------------------------------------------

def pin_tiled_agrees(fn):
    from oracle.tiled import attention_tiled
    rng = _rng(102)
    for (N, d, causal) in [(37, 8, False), (37, 8, True), (64, 16, True), (20, 4, False)]:
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((N, d))
        v = rng.standard_normal((N, d))
        scale = 1 / math.sqrt(d)
        O, L = fn(q, k, v, scale, causal)
        for br, bc in [(1, 1), (3, 16), (16, 3), (16, 16), (64, 7)]:
            for form in ("local", "tree", "running"):
                Ot, Lt = attention_tiled(q, k, v, scale, causal, br, bc, form)
                _close(O, Ot, 1e-12, f"O tiled br={br} bc={bc} {form}")
                _close(L, Lt, 1e-12, f"L tiled br={br} bc={bc} {form}")


# ---------------------------------------------------------------------------
# 3. P = O(q, k, I): rows are non-negative, sum to 1, vanish above the diagonal.
# ---------------------------------------------------------------------------

def pin_probability_rows(fn):
    rng = _rng(103)
    for causal in (False, True):
        N, d = 9, 5
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((N, d))
        P, _ = fn(q, k, np.eye(N), 0.7, causal)
        P = np.asarray(P)
        assert np.all(P >= 0), "P has negative entries"
        _close(P.sum(axis=1), np.ones(N), 1e-12, "row sums of P")
        if causal:
            assert np.all(P[np.triu_indices(N, 1)] == 0), "P nonzero above the diagonal"
        else:
            assert np.all(P > 0), "non-causal P must be strictly positive"


# ---------------------------------------------------------------------------
# 4. Q = 0 (and scale = 0): uniform weights over the visible keys.
#    L_i = ln(#visible), O_i = mean of the visible V rows.
# ---------------------------------------------------------------------------

def pin_zero_query(fn):
    rng = _rng(104)
    N, d = 11, 6
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    for causal in (False, True):
        for q, scale in [(np.zeros((N, d)), 0.37), (rng.standard_normal((N, d)), 0.0)]:
            O, L = fn(q, k, v, scale, causal)
            if causal:
                cnt = np.arange(1, N + 1)
                Oexp = np.cumsum(v, axis=0) / cnt[:, None]
            else:
                cnt = np.full(N, N)
                Oexp = np.broadcast_to(v.mean(axis=0), (N, d))
            _close(L, np.log(cnt), 1e-12, f"L for uniform weights causal={causal}")
            _close(O, Oexp, 1e-12, f"O for uniform weights causal={causal}")


# ---------------------------------------------------------------------------
# 5. Constant V: every output row equals that constant row.
# ---------------------------------------------------------------------------

def pin_constant_v(fn):
    rng = _rng(105)
    N, d = 13, 4
    c = rng.standard_normal(d)
    for causal in (False, True):
        q = rng.standard_normal((N, d)) * 3
        k = rng.standard_normal((N, d))
        O, _ = fn(q, k, np.tile(c, (N, 1)), 0.5, causal)
        _close(O, np.tile(c, (N, 1)), 1e-12, "O for constant V")


# ---------------------------------------------------------------------------
# 6. Single visible key: causal row 0, and Nk = 1.  O = v_0, L = scale q.k_0.
# ---------------------------------------------------------------------------

def pin_single_key(fn):
    rng = _rng(106)
    N, d = 7, 5
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    O, L = fn(q, k, v, 0.9, True)
    _close(O[0], v[0], 1e-12, "causal row 0 O")
    _close(L[0], 0.9 * q[0] @ k[0], 1e-12, "causal row 0 L")
    O, L = fn(q, k[:1], v[:1], 0.9, False)
    _close(O, np.tile(v[0], (N, 1)), 1e-12, "Nk=1 O")
    _close(L, 0.9 * q @ k[0], 1e-12, "Nk=1 L")


# ---------------------------------------------------------------------------
# 7. Permuting key/value rows together changes nothing (non-causal).
# ---------------------------------------------------------------------------

def pin_key_permutation(fn):
    rng = _rng(107)
    Nq, Nk, d = 6, 10, 4
    q = rng.standard_normal((Nq, d))
    k = rng.standard_normal((Nk, d))
    v = rng.standard_normal((Nk, d))
    perm = rng.permutation(Nk)
    O1, L1 = fn(q, k, v, 0.6, False)
    O2, L2 = fn(q, k[perm], v[perm], 0.6, False)
    _close(O1, O2, 1e-12, "O under key permutation")
    _close(L1, L2, 1e-12, "L under key permutation")


# ---------------------------------------------------------------------------
# 8. Shifting every key by u shifts row i's scores by scale q_i.u:
#    O is unchanged and L_i grows by exactly scale q_i.u.
# ---------------------------------------------------------------------------

def pin_key_shift(fn):
    rng = _rng(108)
    N, d = 8, 3
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, d))
    u = rng.standard_normal(d) * 4
    for causal in (False, True):
        O1, L1 = fn(q, k, v, 0.8, causal)
        O2, L2 = fn(q, k + u, v, 0.8, causal)
        _close(O2, O1, 1e-11, "O under key shift")
        _close(L2, np.asarray(L1) + 0.8 * (q @ u), 1e-11, "L under key shift")


# ---------------------------------------------------------------------------
# 9. Library routine: torch's scaled_dot_product_attention and logsumexp on
#    the CPU in float64 (a textbook routine, used only to check the oracle).
# ---------------------------------------------------------------------------

def pin_library(fn):
    import torch
    rng = _rng(109)
    for (Nq, Nk, d, causal) in [(17, 17, 8, False), (17, 17, 8, True), (5, 23, 16, False)]:
        q = rng.standard_normal((Nq, d))
        k = rng.standard_normal((Nk, d))
        v = rng.standard_normal((Nk, d))
        scale = 1 / math.sqrt(d) * 1.3
        O, L = fn(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        Ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                              scale=scale)[0, 0].numpy()
        S = scale * (torch.from_numpy(q) @ torch.from_numpy(k).T)
        if causal:
            S = S.masked_fill(torch.triu(torch.ones(Nq, Nk, dtype=torch.bool), 1), float("-inf"))
        Lt = torch.logsumexp(S, dim=1).numpy()
        _close(O, Ot, 1e-12, "O vs torch sdpa")
        _close(L, Lt, 1e-12, "L vs torch logsumexp")


# ---------------------------------------------------------------------------
# 10. Hand-derived golden cases (tests/golden/hand_cases.json).
# ---------------------------------------------------------------------------

def pin_golden(fn):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        O, L = fn(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]), c["scale"], c["causal"])
        _close(O, c["O"], 1e-9, f"golden {c['name']} O")
        _close(L, c["L"], 1e-9, f"golden {c['name']} L")


ALL_PINS = [pin_brute_force, pin_tiled_agrees, pin_probability_rows, pin_zero_query,
            pin_constant_v, pin_single_key, pin_key_permutation, pin_key_shift,
            pin_library, pin_golden]


# ---------------------------------------------------------------------------
# Banded mask. fn(q, k, v, scale, window) -> (O, L), window = (left, right),
# None = unbounded; query i sees key j iff i+off-left <= j <= i+off+right with
# off = Nk - Nq; a row that sees no key gives O = 0 and L = -inf.
# ---------------------------------------------------------------------------

def _close_inf(a, b, tol, what):
    """Like _close, but -inf entries must match exactly (position and sign)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert not np.any(np.isnan(a)), f"{what}: NaN values"
    ia, ib = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(ia, ib), f"{what}: -inf pattern differs"
    assert np.all(np.isfinite(a[~ia])), f"{what}: non-finite values"
    err = np.max(np.abs(a[~ia] - b[~ib])) if np.any(~ia) else 0.0
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


def brute_force_band(q, k, v, scale, window):
    """Pure-Python loops: the band test written out per (i, j) pair."""
    Nq, Nk = len(q), len(k)
    left, right = window
    off = Nk - Nq
    O, L = [], []
    for i in range(Nq):
        w = []
        for j in range(Nk):
            if left is not None and j - (i + off) < -left:
                continue
            if right is not None and j - (i + off) > right:
                continue
            s = scale * math.fsum(q[i][t] * k[j][t] for t in range(len(q[i])))
            w.append((math.exp(s), j))
        if not w:
            O.append([0.0] * len(v[0]))
            L.append(-math.inf)
            continue
        Z = math.fsum(e for e, _ in w)
        O.append([math.fsum(e * v[j][c] for e, j in w) / Z for c in range(len(v[0]))])
        L.append(math.log(Z))
    return O, L


_WINDOWS = [(None, None), (None, 0), (0, 0), (1, 0), (0, 2), (2, 1), (3, None), (None, 1), (5, 5)]


def pin_band_brute_force(fn):
    rng = _rng(131)
    for Nq in (1, 3, 5, 8):
        for Nk in (1, 2, 5, 8):
            for window in _WINDOWS:
                q = rng.standard_normal((Nq, 3))
                k = rng.standard_normal((Nk, 3))
                v = rng.standard_normal((Nk, 2))
                scale = float(rng.uniform(0.2, 1.5))
                O, L = fn(q, k, v, scale, window)
                Ob, Lb = brute_force_band(q.tolist(), k.tolist(), v.tolist(), scale, window)
                what = f"band {window} Nq={Nq} Nk={Nk}"
                _close(O, Ob, 1e-12, "O " + what)
                _close_inf(L, Lb, 1e-12, "L " + what)


def pin_band_reduces(fn):
    """(None, None) is unmasked attention and (None, 0) with Nq == Nk is causal
    attention, both checked against the plain brute force above."""
    rng = _rng(137)
    for N in (1, 4, 9):
        for Nk in (N, 6):
            q = rng.standard_normal((N, 4))
            k = rng.standard_normal((Nk, 4))
            v = rng.standard_normal((Nk, 3))
            O, L = fn(q, k, v, 0.7, (None, None))
            Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.7, False)
            _close(O, Ob, 1e-12, f"O unbounded band N={N} Nk={Nk}")
            _close(L, Lb, 1e-12, f"L unbounded band N={N} Nk={Nk}")
        k = rng.standard_normal((N, 4))
        v = rng.standard_normal((N, 3))
        O, L = fn(q, k, v, 0.7, (None, 0))
        Ob, Lb = brute_force(q.tolist(), k.tolist(), v.tolist(), 0.7, True)
        _close(O, Ob, 1e-12, f"O causal band N={N}")
        _close(L, Lb, 1e-12, f"L causal band N={N}")


def pin_band_diagonal(fn):
    """Band (0, 0): query i sees only key i + off, so O_i = v_{i+off} and
    L_i = scale q_i . k_{i+off}; outside [0, Nk) the row is empty."""
    rng = _rng(139)
    for Nq, Nk in ((5, 5), (3, 7), (7, 3)):
        q = rng.standard_normal((Nq, 4))
        k = rng.standard_normal((Nk, 4))
        v = rng.standard_normal((Nk, 2))
        O, L = fn(q, k, v, 0.9, (0, 0))
        off = Nk - Nq
        for i in range(Nq):
            j = i + off
            if 0 <= j < Nk:
                _close(O[i], v[j], 1e-12, f"O diagonal band row {i}")
                _close([L[i]], [0.9 * float(q[i] @ k[j])], 1e-12, f"L diagonal band row {i}")
            else:
                _close(O[i], np.zeros(2), 0.0, f"O empty row {i}")
                assert L[i] == -math.inf, f"L empty row {i}: {L[i]}"


def pin_band_tiled_agrees(fn):
    from oracle.tiled import attention_tiled
    rng = _rng(149)
    for Nq, Nk in ((20, 20), (13, 29), (29, 13)):
        q = rng.standard_normal((Nq, 5))
        k = rng.standard_normal((Nk, 5))
        v = rng.standard_normal((Nk, 3))
        for window in ((None, 0), (4, 3), (0, 6), (7, None)):
            O, L = fn(q, k, v, 0.6, window)
            for br, bc, form in ((1, 1, "local"), (4, 3, "local"), (3, 2, "tree"),
                                 (16, 16, "running")):
                Ot, Lt = attention_tiled(q, k, v, 0.6, False, br, bc, form, window=window)
                _close(O, Ot, 1e-12, f"O tiled band {window} {br}x{bc} {form}")
                _close_inf(L, Lt, 1e-12, f"L tiled band {window} {br}x{bc} {form}")


BAND_PINS = [pin_band_brute_force, pin_band_reduces, pin_band_diagonal, pin_band_tiled_agrees]
