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
