"""The CPU oracle against its pins (no GPU)."""
import math

import numpy as np
import pytest

from oracle import attention, attention_dense, attention_probs, attention_tiled, attention_varlen
from tests.oracle_pins import ALL_PINS, BAND_PINS


def _tiled_fn(q, k, v, scale, causal):
    return attention_tiled(q, k, v, scale, causal, block_rows=4, block_cols=3)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_definition_pins(pin):
    pin(attention)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_tiled_pins(pin):
    """The blockwise algorithm meets the same pins on its own."""
    pin(_tiled_fn)


@pytest.mark.parametrize("pin", BAND_PINS, ids=lambda p: p.__name__)
def test_oracle_band_pins(pin):
    pin(lambda q, k, v, scale, window: attention(q, k, v, scale, window=window))


@pytest.mark.parametrize("pin", BAND_PINS, ids=lambda p: p.__name__)
def test_oracle_tiled_band_pins(pin):
    pin(lambda q, k, v, scale, window: attention_tiled(q, k, v, scale, False, 4, 3, window=window))


def test_band_probs_rows_sum_to_one_or_zero():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((7, 4))
    k = rng.standard_normal((11, 4))
    P = attention_probs(q, k, 0.5, window=(1, 0))
    sums = P.sum(1)
    assert np.all((np.abs(sums - 1.0) < 1e-14) | (sums == 0.0))
    assert np.all(P >= 0)


def test_probs_match_attention_weights():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((9, 4))
    k = rng.standard_normal((9, 4))
    for causal in (False, True):
        P = attention_probs(q, k, 0.5, causal)
        O, _ = attention(q, k, np.eye(9), 0.5, causal)
        np.testing.assert_allclose(P, O, atol=1e-14)
        np.testing.assert_allclose(P.sum(1), 1.0, atol=1e-14)


def test_rows_subset_is_a_slice():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((40, 8)) for _ in range(3))
    rows = [0, 3, 17, 39]
    for causal in (False, True):
        O, L = attention(q, k, v, 0.3, causal)
        Os, Ls = attention(q, k, v, 0.3, causal, rows=rows)
        np.testing.assert_array_equal(Os, O[rows])
        np.testing.assert_array_equal(Ls, L[rows])


def test_dense_loops_heads_and_batches():
    rng = np.random.default_rng(7)
    B, N, H, d = 2, 12, 3, 4
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    O, L = attention_dense(q, k, v, 0.5, True)
    assert O.shape == (B, N, H, d) and L.shape == (B, H, N)
    for b in range(B):
        for h in range(H):
            o, l = attention(q[b, :, h], k[b, :, h], v[b, :, h], 0.5, True)
            np.testing.assert_array_equal(O[b, :, h], o)
            np.testing.assert_array_equal(L[b, h], l)
    Os, Ls = attention_dense(q, k, v, 0.5, True, batches=[1], heads=[2], rows=[0, 5])
    np.testing.assert_array_equal(Os[0, :, 0], O[1, [0, 5], 2])
    np.testing.assert_array_equal(Ls[0, 0], L[1, 2, [0, 5]])


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_per_sequence(causal):
    """Packing sequences gives the same O and L as running each one alone."""
    rng = np.random.default_rng(8)
    lengths = [5, 0, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 4
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    O, L = attention_varlen(q, k, v, cu, 0.6, causal)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    for s, n in enumerate(lengths):
        a = int(cu[s])
        if n == 0:
            continue
        for h in range(H):
            o, l = attention(q[a:a + n, h], k[a:a + n, h], v[a:a + n, h], 0.6, causal)
            np.testing.assert_array_equal(O[a:a + n, h], o)
            np.testing.assert_array_equal(L[h, a:a + n], l)
    # and no attention across the boundary: changing another sequence changes nothing
    k2 = k.copy()
    k2[cu[3]:cu[4]] += 10.0
    O2, L2 = attention_varlen(q, k2, v, cu, 0.6, causal)
    np.testing.assert_array_equal(O2[: cu[3]], O[: cu[3]])
    np.testing.assert_array_equal(L2[:, : cu[3]], L[:, : cu[3]])


def test_causal_requires_square():
    with pytest.raises(ValueError):
        attention(np.zeros((3, 2)), np.zeros((4, 2)), np.zeros((4, 2)), 1.0, True)


def test_empty_query():
    O, L = attention(np.zeros((0, 4)), np.zeros((3, 4)), np.zeros((3, 4)), 1.0, False)
    assert O.shape == (0, 4) and L.shape == (0,)


# ---------------------------------------------------------------------------
# Backward (gradients of the definition)
# ---------------------------------------------------------------------------

from oracle import (attention_backward, attention_backward_dense,  # noqa: E402
                    attention_backward_varlen)
from tests.oracle_bwd_pins import BWD_PINS  # noqa: E402


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda p: p.__name__)
def test_oracle_backward_pins(pin):
    pin(attention_backward)


def test_backward_p_recomputed_from_l():
    """The pages' recomputation: with L from the forward, exp(S - L) is the
    softmax P the backward uses."""
    rng = np.random.default_rng(31)
    q, k = rng.standard_normal((6, 4)), rng.standard_normal((6, 4))
    for causal in (False, True):
        _, L = attention(q, k, rng.standard_normal((6, 2)), 0.8, causal)
        S = 0.8 * q @ k.T
        if causal:
            S = np.where(np.triu(np.ones((6, 6), dtype=bool), 1), -np.inf, S)
        np.testing.assert_allclose(np.exp(S - L[:, None]), attention_probs(q, k, 0.8, causal),
                                   rtol=0, atol=1e-14)


def test_backward_wrappers_match_single_head():
    rng = np.random.default_rng(32)
    q, k, v, do = (rng.standard_normal((2, 7, 3, 4)) for _ in range(4))
    dq, dk, dv, delta = attention_backward_dense(q, k, v, do, 0.5, True)
    for b in range(2):
        for h in range(3):
            g = attention_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], 0.5, True)
            for got, want in zip((dq[b, :, h], dk[b, :, h], dv[b, :, h], delta[b, h]), g):
                np.testing.assert_array_equal(got, want)
    lengths = [3, 0, 5]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    qv, kv, vv, dov = (rng.standard_normal((8, 2, 4)) for _ in range(4))
    dq, dk, dv, delta = attention_backward_varlen(qv, kv, vv, dov, cu, 0.5, False)
    g = attention_backward(qv[3:8, 1], kv[3:8, 1], vv[3:8, 1], dov[3:8, 1], 0.5, False)
    np.testing.assert_array_equal(dk[3:8, 1], g[1])
    np.testing.assert_array_equal(delta[1, 3:8], g[3])


# ---------------------------------------------------------------------------
# Key padding mask (remove the padding, attend, put back)
# ---------------------------------------------------------------------------

from oracle import attention_padded  # noqa: E402
from tests.oracle_pins import _close, _close_inf, brute_force  # noqa: E402


def _brute_force_masked(q, k, v, valid, scale, causal):
    """Pure Python: scores of padding keys (and, when causal, of later keys) left
    out of the sums in the padded positions, no removal of rows; padding rows
    give 0 and -inf."""
    N = len(q)
    O, L = [], []
    for i in range(N):
        if not valid[i]:
            O.append([0.0] * len(v[0]))
            L.append(-math.inf)
            continue
        w = [(math.exp(scale * math.fsum(a * b for a, b in zip(q[i], k[j]))), j)
             for j in range(N) if valid[j] and (not causal or j <= i)]
        Z = math.fsum(e for e, _ in w)
        O.append([math.fsum(e * v[j][c] for e, j in w) / Z for c in range(len(v[0]))])
        L.append(math.log(Z))
    return O, L


@pytest.mark.parametrize("causal", [False, True])
def test_padded_matches_masked_brute_force(causal):
    rng = np.random.default_rng(41)
    B, S, H, d = 3, 7, 2, 3
    q, k, v = (rng.standard_normal((B, S, H, d)) for _ in range(3))
    mask = np.array([[1, 1, 1, 1, 0, 0, 0], [0, 1, 0, 1, 1, 0, 1], [0] * 7], dtype=np.uint8)
    O, L = attention_padded(q, k, v, mask, 0.8, causal)
    for b in range(B):
        for h in range(H):
            Ob, Lb = _brute_force_masked(q[b, :, h].tolist(), k[b, :, h].tolist(),
                                         v[b, :, h].tolist(), mask[b].tolist(), 0.8, causal)
            _close(O[b, :, h], Ob, 1e-12, f"padded O b={b} h={h}")
            _close_inf(L[b, h], Lb, 1e-12, f"padded L b={b} h={h}")


def test_padded_all_valid_is_plain_attention():
    rng = np.random.default_rng(42)
    q, k, v = (rng.standard_normal((2, 9, 3, 4)) for _ in range(3))
    for causal in (False, True):
        O, L = attention_padded(q, k, v, np.ones((2, 9), dtype=np.uint8), 0.6, causal)
        Od, Ld = attention_dense(q, k, v, 0.6, causal)
        np.testing.assert_array_equal(O, Od)
        np.testing.assert_array_equal(L, Ld)


def test_padded_right_padding_is_varlen():
    """Right padding (first n_b tokens valid) is the packed varlen batch of those lengths."""
    rng = np.random.default_rng(43)
    B, S, H, d = 3, 8, 2, 4
    lengths = [8, 3, 5]
    q, k, v = (rng.standard_normal((B, S, H, d)) for _ in range(3))
    mask = np.array([[1] * n + [0] * (S - n) for n in lengths], dtype=np.uint8)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    pack = lambda x: np.concatenate([x[b, :n] for b, n in enumerate(lengths)])  # noqa: E731
    for causal in (False, True):
        O, L = attention_padded(q, k, v, mask, 0.5, causal)
        Ov, Lv = attention_varlen(pack(q), pack(k), pack(v), cu, 0.5, causal)
        for b, n in enumerate(lengths):
            a = int(cu[b])
            _close(O[b, :n], Ov[a:a + n], 1e-13, "right padding O")
            _close(L[b, :, :n], Lv[:, a:a + n], 1e-13, "right padding L")
            assert np.all(O[b, n:] == 0) and np.all(np.isneginf(L[b, :, n:]))


def test_padded_keys_ignore_padding_content():
    """Changing q, k, v at padding positions changes nothing (non-causal and causal)."""
    rng = np.random.default_rng(44)
    q, k, v = (rng.standard_normal((1, 10, 1, 4)) for _ in range(3))
    mask = np.array([[1, 0, 1, 1, 0, 1, 1, 1, 0, 1]], dtype=np.uint8)
    for causal in (False, True):
        O1, L1 = attention_padded(q, k, v, mask, 0.7, causal)
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        for x in (q2, k2, v2):
            x[0, mask[0] == 0] = 50.0
        O2, L2 = attention_padded(q2, k2, v2, mask, 0.7, causal)
        np.testing.assert_array_equal(O1, O2)
        np.testing.assert_array_equal(L1, L2)


def test_lse_merge_of_key_chunks_is_attention():
    """Attention over all keys equals the merge of attention over disjoint key
    chunks through their log-sum-exps: L = ln sum_s e^{L_s}, O = sum_s e^{L_s - L} O_s
    (the use of L beyond the backward; the split decode relies on it)."""
    rng = np.random.default_rng(45)
    q = rng.standard_normal((1, 8))
    k, v = rng.standard_normal((37, 8)), rng.standard_normal((37, 5))
    O, L = attention(q, k, v, 0.4)
    for bounds in ([0, 37], [0, 10, 37], [0, 1, 2, 30, 37], [0, 5, 5, 37]):
        parts = [attention(q, k[a:b], v[a:b], 0.4) for a, b in zip(bounds, bounds[1:]) if b > a]
        Ls = np.array([p[1][0] for p in parts])
        Lm = np.log(np.sum(np.exp(Ls - Ls.max()))) + Ls.max()
        Om = sum(np.exp(p[1][0] - Lm) * p[0][0] for p in parts)
        np.testing.assert_allclose(Om, O[0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(Lm, L[0], rtol=0, atol=1e-13)


# ---------------------------------------------------------------------------
# Backward with a band and with a key padding mask
# ---------------------------------------------------------------------------

from oracle import attention_backward_padded  # noqa: E402


def _fd_grads(loss, arrays, h=1e-6):
    grads = []
    for which in range(len(arrays)):
        g = np.zeros_like(arrays[which])
        for idx in np.ndindex(*g.shape):
            plus = [a.copy() for a in arrays]
            minus = [a.copy() for a in arrays]
            plus[which][idx] += h
            minus[which][idx] -= h
            g[idx] = (loss(*plus) - loss(*minus)) / (2 * h)
        grads.append(g)
    return grads


@pytest.mark.parametrize("window", [(None, 0), (1, 0), (0, 2), (2, 1), (0, 0), (1, None)])
@pytest.mark.parametrize("Nq,Nk", [(4, 4), (3, 6), (6, 3)])
def test_backward_band_finite_differences(window, Nq, Nk):
    """Gradients with a band against central differences of the (pinned) band
    forward; rows that see no key have zero gradients."""
    rng = np.random.default_rng(51 + Nq + 7 * Nk)
    q, k, v = rng.standard_normal((Nq, 3)), rng.standard_normal((Nk, 3)), rng.standard_normal((Nk, 2))
    do = rng.standard_normal((Nq, 2))

    def loss(q_, k_, v_):
        O, _ = attention(q_, k_, v_, 0.7, window=window)
        return float(np.sum(O * do))
    dq, dk, dv, delta = attention_backward(q, k, v, do, 0.7, window=window)
    fq, fk, fv = _fd_grads(loss, [q, k, v])
    np.testing.assert_allclose(dq, fq, atol=1e-7)
    np.testing.assert_allclose(dk, fk, atol=1e-7)
    np.testing.assert_allclose(dv, fv, atol=1e-7)
    O, _ = attention(q, k, v, 0.7, window=window)
    np.testing.assert_allclose(delta, np.sum(do * O, axis=1), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_padded_finite_differences(causal):
    """Gradients with a key padding mask against central differences of the
    (pinned) padded forward: zero at padding positions, and padding content
    never matters."""
    rng = np.random.default_rng(61 + causal)
    B, S, H, d = 2, 6, 1, 2
    q, k, v, do = (rng.standard_normal((B, S, H, d)) for _ in range(4))
    mask = np.array([[1, 0, 1, 1, 0, 1], [1, 1, 1, 0, 0, 0]], dtype=np.uint8)

    def loss(q_, k_, v_):
        O, _ = attention_padded(q_, k_, v_, mask, 0.9, causal)
        return float(np.sum(O * do))
    dq, dk, dv, delta = attention_backward_padded(q, k, v, do, mask, 0.9, causal)
    fq, fk, fv = _fd_grads(loss, [q, k, v])
    np.testing.assert_allclose(dq, fq, atol=1e-7)
    np.testing.assert_allclose(dk, fk, atol=1e-7)
    np.testing.assert_allclose(dv, fv, atol=1e-7)
    pad = mask == 0
    assert np.all(dq[pad] == 0) and np.all(dk[pad] == 0) and np.all(dv[pad] == 0)
    assert np.all(delta.transpose(0, 2, 1)[pad] == 0)
