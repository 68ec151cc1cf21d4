"""Planted mistakes in copies of the oracle must each fail at least one pin.

This shows the pins are strong enough that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, a wrong axis or
log base) cannot pass unnoticed. The mistakes live only in this file, on the
CPU; the oracle itself is untouched.
"""
import numpy as np
import pytest

from tests.oracle_pins import ALL_PINS


def _make(mutation):
    def fn(q, k, v, scale, causal):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        Nq, Nk = q.shape[0], k.shape[0]
        sc = 1.0 if mutation == "scale_dropped" else scale
        if mutation == "scores_transposed":
            S = sc * (k @ q.T)
        else:
            S = sc * (q @ k.T)
        if causal:
            i = np.arange(Nq)[:, None]
            j = np.arange(Nk)[None, :]
            if mutation == "mask_off_by_one":
                masked = j >= i
            elif mutation == "mask_flipped":
                masked = j < i
            else:
                masked = j > i
            S = np.where(masked, -np.inf, S)
        m = S.max(axis=0 if mutation == "softmax_axis0" else 1,
                  keepdims=True)
        if mutation == "no_max_subtraction":
            m = np.zeros_like(m)
        sign = -1.0 if mutation == "exp_sign" else 1.0
        e = np.exp(sign * (S - m))
        l = e.sum(axis=0 if mutation == "softmax_axis0" else 1, keepdims=True)
        P = e if mutation == "unnormalised" else e / l
        vv = v[::-1] if mutation == "v_reversed" else v
        O = P @ vv
        mm = m if mutation != "softmax_axis0" else m.T
        ll = l if mutation != "softmax_axis0" else l.T
        if mutation == "lse_missing_max":
            L = np.log(ll[:, 0])
        elif mutation == "lse_log2":
            L = mm[:, 0] + np.log2(ll[:, 0])
        elif mutation == "lse_unscaled_max":
            L = (mm[:, 0] / sc if sc != 0 else mm[:, 0]) + np.log(ll[:, 0])
        elif mutation == "lse_is_max":
            L = mm[:, 0]
        else:
            L = mm[:, 0] + np.log(ll[:, 0])
        if mutation == "o_off_by_one_row":
            O = np.roll(O, 1, axis=0)
        return O, L
    return fn


MUTATIONS = ["scale_dropped", "scores_transposed", "mask_off_by_one", "mask_flipped",
             "softmax_axis0", "no_max_subtraction", "exp_sign", "unnormalised",
             "v_reversed", "lse_missing_max", "lse_log2", "lse_unscaled_max",
             "lse_is_max", "o_off_by_one_row"]


def test_unmutated_copy_passes_every_pin():
    fn = _make("none")
    for pin in ALL_PINS:
        pin(fn)


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutation_is_caught(mutation):
    fn = _make(mutation)
    caught = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mutation!r}"


# ---------------------------------------------------------------------------
# Banded mask: planted mistakes in a copy of the band logic must each fail at
# least one of the band pins.
# ---------------------------------------------------------------------------

from tests.oracle_pins import BAND_PINS  # noqa: E402

BAND_MUTATIONS = ["left_off_by_one", "right_off_by_one", "alignment_flipped",
                  "alignment_ignored", "empty_row_nan", "empty_row_l_zero",
                  "window_sides_swapped"]


def _make_band(mutation):
    def fn(q, k, v, scale, window):
        q = np.asarray(q, dtype=np.float64)
        k = np.asarray(k, dtype=np.float64)
        v = np.asarray(v, dtype=np.float64)
        Nq, Nk = q.shape[0], k.shape[0]
        left, right = window
        if mutation == "window_sides_swapped":
            left, right = right, left
        off = Nk - Nq
        if mutation == "alignment_flipped":
            off = Nq - Nk
        elif mutation == "alignment_ignored":
            off = 0
        i = np.arange(Nq)[:, None] + off
        j = np.arange(Nk)[None, :]
        vis = np.ones((Nq, Nk), dtype=bool)
        if left is not None:
            vis &= j >= i - left + (1 if mutation == "left_off_by_one" else 0)
        if right is not None:
            vis &= j <= i + right - (1 if mutation == "right_off_by_one" else 0)
        S = np.where(vis, scale * (q @ k.T), -np.inf)
        m = S.max(axis=1, keepdims=True)
        if mutation != "empty_row_nan":
            m = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(S - m)
        l = e.sum(axis=1, keepdims=True)
        with np.errstate(invalid="ignore", divide="ignore"):
            if mutation == "empty_row_nan":
                O = (e / l) @ v
                L = m[:, 0] + np.log(l[:, 0])
            else:
                O = (e / np.where(l > 0, l, 1.0)) @ v
                L = np.where(l[:, 0] > 0, m[:, 0] + np.log(np.where(l > 0, l, 1.0)[:, 0]),
                             0.0 if mutation == "empty_row_l_zero" else -np.inf)
        return O, L
    return fn


def test_band_reference_copy_passes():
    """The unmutated copy passes every band pin (so the mutants fail for their mistake)."""
    fn = _make_band("none")
    for pin in BAND_PINS:
        pin(fn)


@pytest.mark.parametrize("mutation", BAND_MUTATIONS)
def test_band_mutant_is_caught(mutation):
    fn = _make_band(mutation)
    failed = []
    for pin in BAND_PINS:
        try:
            pin(fn)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"band mutation {mutation!r} passed every band pin"


# ---------------------------------------------------------------------------
# Backward: planted mistakes in a copy of the gradient formulas must each fail
# at least one backward pin.
# ---------------------------------------------------------------------------

from tests.oracle_bwd_pins import BWD_PINS  # noqa: E402

BWD_MUTATIONS = ["dq_no_scale", "dk_no_scale", "ds_sign_flipped", "delta_dropped",
                 "delta_from_p_only", "dk_from_ds_not_transposed", "dv_from_p_not_transposed",
                 "dq_uses_v", "causal_mask_dropped", "delta_from_unmasked_p"]


def _make_bwd(mutation):
    def fn(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        Nq, Nk = q.shape[0], k.shape[0]
        S = scale * (q @ k.T)
        mask = np.triu(np.ones((Nq, Nk), dtype=bool), 1) if causal else np.zeros((Nq, Nk), bool)
        Sm = S if mutation == "causal_mask_dropped" else np.where(mask, -np.inf, S)
        P = np.exp(Sm - Sm.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        dv = (P @ do[:Nk] if Nq >= Nk else P.T @ do) if mutation == "dv_from_p_not_transposed" \
            else P.T @ do
        dP = do @ v.T
        if mutation == "delta_from_unmasked_p":
            Pu = np.exp(S - S.max(axis=1, keepdims=True))
            Pu /= Pu.sum(axis=1, keepdims=True)
            delta = np.sum(Pu * dP, axis=1)
        elif mutation == "delta_from_p_only":
            delta = np.sum(P, axis=1)
        else:
            delta = np.sum(P * dP, axis=1)
        dS = P * (dP - (0.0 if mutation == "delta_dropped" else delta[:, None]))
        if mutation == "ds_sign_flipped":
            dS = -dS
        dq = (1.0 if mutation == "dq_no_scale" else scale) * (dS @ (v if mutation == "dq_uses_v" else k))
        if mutation == "dk_from_ds_not_transposed":
            dk = scale * (dS @ q[:Nk] if Nq >= Nk and dS.shape[1] == Nk else dS.T @ q)
            if Nq == Nk:
                dk = scale * (dS @ q)
        else:
            dk = (1.0 if mutation == "dk_no_scale" else scale) * (dS.T @ q)
        return dq, dk, dv, delta
    return fn


def test_bwd_reference_copy_passes():
    fn = _make_bwd("none")
    for pin in BWD_PINS:
        pin(fn)


@pytest.mark.parametrize("mutation", BWD_MUTATIONS)
def test_bwd_mutant_is_caught(mutation):
    fn = _make_bwd(mutation)
    failed = []
    for pin in BWD_PINS:
        try:
            pin(fn)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"backward mutation {mutation!r} passed every backward pin"


# ---------------------------------------------------------------------------
# Key padding mask: planted mistakes in a copy of the padded route must each
# fail the padded pins of test_oracle.py.
# ---------------------------------------------------------------------------

from oracle import attention  # noqa: E402

PAD_MUTATIONS = ["mask_inverted", "padding_rows_not_zeroed", "padding_l_zero",
                 "padding_keys_kept", "causal_over_compacted_reversed"]


def _make_padded(mutation):
    def fn(q, k, v, mask, scale, causal):
        B, S, H, _ = q.shape
        m = np.asarray(mask) != 0
        if mutation == "mask_inverted":
            m = ~m
        O = np.zeros((B, S, H, v.shape[3])) if mutation != "padding_rows_not_zeroed" \
            else np.ones((B, S, H, v.shape[3]))
        L = np.full((B, H, S), 0.0 if mutation == "padding_l_zero" else -np.inf)
        for b in range(B):
            idx = np.arange(S) if mutation == "padding_keys_kept" else np.nonzero(m[b])[0]
            if idx.size == 0:
                continue
            if mutation == "causal_over_compacted_reversed":
                idx = idx[::-1]
            for h in range(H):
                o, lse = attention(q[b, idx, h], k[b, idx, h], v[b, idx, h], scale, causal)
                rows = idx if mutation != "padding_keys_kept" else np.nonzero(m[b])[0]
                sel = slice(None) if mutation != "padding_keys_kept" else rows
                O[b, rows, h] = o[sel]
                L[b, h, rows] = lse[sel]
        return O, L
    return fn


def _padded_pins(fn):
    import tests.test_oracle as T
    orig = T.attention_padded
    T.attention_padded = fn
    try:
        T.test_padded_matches_masked_brute_force(False)
        T.test_padded_matches_masked_brute_force(True)
        T.test_padded_all_valid_is_plain_attention()
        T.test_padded_right_padding_is_varlen()
    finally:
        T.attention_padded = orig


def test_padded_reference_copy_passes():
    _padded_pins(_make_padded("none"))


@pytest.mark.parametrize("mutation", PAD_MUTATIONS)
def test_padded_mutant_is_caught(mutation):
    with pytest.raises(Exception):  # noqa: B017 - any failure counts as caught
        _padded_pins(_make_padded(mutation))
