"""The local-window + global-anchor oracle against its pins, and planted
mistakes in a copy of it that the pins must catch."""
import numpy as np
import pytest

from oracle.local import attention_local, local_pairs, local_visible
from tests.oracle_local_pins import LOCAL_PINS


@pytest.mark.parametrize("pin", LOCAL_PINS, ids=lambda p: p.__name__)
def test_local_oracle_pin(pin):
    pin(attention_local)


def test_local_pair_count_closed_form():
    """Visible pairs on a full map with G anchors: G N (anchor rows) + (N - G) G
    (anchor keys of map rows) + the product of the row and column reaches."""
    h, W, wr, wc, G = 6, 7, 2, 1, 3
    N = G + h * W
    reach = lambda n, w: sum(min(n - 1, x + w) - max(0, x - w) + 1 for x in range(n))  # noqa: E731
    expect = G * N + (N - G) * G + reach(h, wr) * reach(W, wc)
    assert local_pairs(N, G, W, wr, wc) == expect
    vis = local_visible(N, G, W, wr, wc)
    assert np.array_equal(local_visible(N, G, W, wr, wc, True), vis & np.tri(N, dtype=bool))


def _make_local(mutation):
    def fn(q, k, v, scale, G, W, wr, wc, causal):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        N = q.shape[0]
        t = np.arange(N)
        anc = t < G
        pos = np.maximum(t - (0 if mutation == "map_not_offset_by_anchors" else G), 0)
        row, col = pos // W, pos % W
        if mutation == "rows_cols_swapped":
            row, col = col, row
        lim_r = wr - (1 if mutation == "window_off_by_one" else 0)
        near = (np.abs(row[:, None] - row[None, :]) <= lim_r) & \
               (np.abs(col[:, None] - col[None, :]) <= wc)
        vis = near.copy()
        if mutation != "anchor_queries_not_global":
            vis |= anc[:, None]
        if mutation != "anchor_keys_hidden":
            vis |= anc[None, :]
        if causal and mutation != "causal_dropped":
            vis &= t[None, :] <= t[:, None]
        if mutation == "causal_reversed" and causal:
            vis = near & (t[None, :] >= t[:, None])
        S = np.where(vis, scale * (q @ k.T), -np.inf)
        m = S.max(axis=1, keepdims=True)
        e = np.exp(S - m)
        l = e.sum(axis=1, keepdims=True)
        return (e / l) @ v, m[:, 0] + np.log(l[:, 0])
    return fn


LOCAL_MUTATIONS = ["map_not_offset_by_anchors", "rows_cols_swapped", "window_off_by_one",
                   "anchor_queries_not_global", "anchor_keys_hidden", "causal_dropped",
                   "causal_reversed"]


def test_local_reference_copy_passes():
    fn = _make_local("none")
    for pin in LOCAL_PINS:
        pin(fn)


@pytest.mark.parametrize("mutation", LOCAL_MUTATIONS)
def test_local_mutant_is_caught(mutation):
    fn = _make_local(mutation)
    failed = []
    for pin in LOCAL_PINS:
        try:
            pin(fn)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"local mutation {mutation!r} passed every local pin"


@pytest.mark.parametrize("G,Wd,wr,wc,causal", [(2, 3, 1, 0, False), (0, 4, 0, 1, True),
                                               (3, 2, 1, 1, True), (1, 5, 0, 0, False)])
def test_local_backward_finite_differences(G, Wd, wr, wc, causal):
    """Gradients against central differences of the (pinned) local forward."""
    from oracle.local import attention_local_backward
    rng = np.random.default_rng(91 + G + 7 * Wd)
    N = 9
    q, k, v, do = (rng.standard_normal((N, 3)) for _ in range(4))

    def loss(q_, k_, v_):
        O, _ = attention_local(q_, k_, v_, 0.7, G, Wd, wr, wc, causal)
        return float(np.sum(O * do))
    dq, dk, dv, delta = attention_local_backward(q, k, v, do, 0.7, G, Wd, wr, wc, causal)
    h = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            up = loss(q, k, v)
            x[idx] = x0 - h
            dn = loss(q, k, v)
            x[idx] = x0
            fd[idx] = (up - dn) / (2 * h)
        np.testing.assert_allclose(g, fd, atol=1e-7)
    O, _ = attention_local(q, k, v, 0.7, G, Wd, wr, wc, causal)
    np.testing.assert_allclose(delta, np.sum(do * O, axis=1), atol=1e-12)


def test_local_backward_one_wide_map_is_the_band_backward():
    from oracle import attention_backward
    from oracle.local import attention_local_backward
    rng = np.random.default_rng(95)
    q, k, v, do = (rng.standard_normal((12, 4)) for _ in range(4))
    for causal in (False, True):
        got = attention_local_backward(q, k, v, do, 0.5, 0, 1, 2, 7, causal)
        ref = attention_backward(q, k, v, do, 0.5, window=(2, 0 if causal else 2))
        for a, b in zip(got, ref):
            np.testing.assert_allclose(a, b, atol=1e-12)


# ---------------------------------------------------------------------------
# The (B, N, H, d) wrappers that the GPU tests compare against: each (batch,
# head) slice must be exactly the single-head result, in the documented
# layouts (O (nb, N, nh, d), L (nb, nh, N); gradients in the input layouts,
# delta (B, H, N)). B = 2 and H = 3 differ, so a swapped index or a
# transposed output lands on the wrong slice and fails.
# ---------------------------------------------------------------------------

_PATTERN = (2, 4, 1, 1)   # n_global, map_w, win_rows, win_cols


def _wrapper_inputs(seed):
    rng = np.random.default_rng(seed)
    B, N, H, d = 2, 14, 3, 4
    return [rng.standard_normal((B, N, H, d)) for _ in range(4)]


def _local_dense_wrapper_pin(wrapper):
    q, k, v, _ = _wrapper_inputs(301)
    for causal in (False, True):
        O, L = wrapper(q, k, v, 0.6, *_PATTERN, causal)
        assert O.shape == (2, 14, 3, 4) and L.shape == (2, 3, 14)
        for b in range(2):
            for h in range(3):
                o, l = attention_local(q[b, :, h], k[b, :, h], v[b, :, h], 0.6, *_PATTERN, causal)
                np.testing.assert_array_equal(O[b, :, h], o)
                np.testing.assert_array_equal(L[b, h], l)
        Os, Ls = wrapper(q, k, v, 0.6, *_PATTERN, causal, batches=[1], heads=[2, 0])
        np.testing.assert_array_equal(Os[0, :, 0], O[1, :, 2])
        np.testing.assert_array_equal(Os[0, :, 1], O[1, :, 0])
        np.testing.assert_array_equal(Ls[0], L[1, [2, 0]])


def _local_backward_dense_wrapper_pin(wrapper):
    from oracle.local import attention_local_backward
    q, k, v, do = _wrapper_inputs(302)
    for causal in (False, True):
        dq, dk, dv, delta = wrapper(q, k, v, do, 0.6, *_PATTERN, causal)
        assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
        assert delta.shape == (2, 3, 14)
        for b in range(2):
            for h in range(3):
                g = attention_local_backward(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h],
                                             0.6, *_PATTERN, causal)
                for got, want in zip((dq[b, :, h], dk[b, :, h], dv[b, :, h], delta[b, h]), g):
                    np.testing.assert_array_equal(got, want)


def test_local_dense_wrapper_is_per_head():
    from oracle.local import attention_local_dense
    _local_dense_wrapper_pin(attention_local_dense)


def test_local_backward_dense_wrapper_is_per_head():
    from oracle.local import attention_local_backward_dense
    _local_backward_dense_wrapper_pin(attention_local_backward_dense)


def _mutant_local_dense(mutation):
    def fn(q, k, v, scale, G, Wd, wr, wc, causal=False, batches=None, heads=None):
        B, N, H, _ = q.shape
        bs = list(range(B)) if batches is None else list(batches)
        hs = list(range(H)) if heads is None else list(heads)
        O = np.zeros((len(bs), N, len(hs), v.shape[3]))
        L = np.zeros((len(bs), len(hs), N))
        for bi, b in enumerate(bs):
            for hi, h in enumerate(hs):
                if mutation == "batch_head_swapped":   # reads slice (h mod B, b mod H)
                    src = (h % B, b % H)
                elif mutation == "head_off_by_one":
                    src = (b, (h + 1) % H)
                else:
                    src = (b, h)
                o, l = attention_local(q[src[0], :, src[1]], k[src[0], :, src[1]],
                                       v[src[0], :, src[1]], scale, G, Wd, wr, wc, causal)
                if mutation == "lse_rows_reversed":
                    l = l[::-1]
                O[bi, :, hi], L[bi, hi] = o, l
        if mutation == "output_heads_reversed":
            O = O[:, :, ::-1]
        return O, L
    return fn


def _mutant_local_backward_dense(mutation):
    from oracle.local import attention_local_backward

    def fn(q, k, v, do, scale, G, Wd, wr, wc, causal=False):
        B, N, H, _ = q.shape
        dq, dk, dv = (np.zeros(x.shape) for x in (q, k, v))
        delta = np.zeros((B, H, N))
        for b in range(B):
            for h in range(H):
                src_h = (h + 1) % H if mutation == "head_off_by_one" else h
                g = attention_local_backward(q[b, :, src_h], k[b, :, src_h], v[b, :, src_h],
                                             do[b, :, src_h], scale, G, Wd, wr, wc, causal)
                if mutation == "dq_dk_swapped":
                    g = (g[1], g[0], g[2], g[3])
                dq[b, :, h], dk[b, :, h], dv[b, :, h], delta[b, h] = g
        if mutation == "delta_transposed":
            delta = np.ascontiguousarray(delta.transpose(1, 0, 2)).reshape(B, H, N)
        return dq, dk, dv, delta
    return fn


@pytest.mark.parametrize("mutation", ["batch_head_swapped", "head_off_by_one",
                                      "lse_rows_reversed", "output_heads_reversed"])
def test_local_dense_wrapper_mutant_is_caught(mutation):
    _local_dense_wrapper_pin(_mutant_local_dense("none"))
    with pytest.raises(AssertionError):
        _local_dense_wrapper_pin(_mutant_local_dense(mutation))


@pytest.mark.parametrize("mutation", ["head_off_by_one", "dq_dk_swapped", "delta_transposed"])
def test_local_backward_dense_wrapper_mutant_is_caught(mutation):
    _local_backward_dense_wrapper_pin(_mutant_local_backward_dense("none"))
    with pytest.raises(AssertionError):
        _local_backward_dense_wrapper_pin(_mutant_local_backward_dense(mutation))
