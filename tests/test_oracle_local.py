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
