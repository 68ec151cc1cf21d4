"""The backward's GPU tolerance against a CPU model of the kernels' arithmetic.

The GPU tests accept a gradient element when it lies within the bar of
tests/test_gpu_backward.py (assert_grad_close with the D-rounding terms of
dense_terms). These CPU tests show that bar is neither too tight nor too
loose. A numpy model computes the gradients the way the dK/dV and dQ kernels
do ("FlashAttention/zh" (marovi.ai wiki), section 反向傳遞與重計算: S and P
recomputed from the saved L, dS = P (dP - D), D = dO . O):
  * Q, K, V, dO and the forward's O are 16-bit; L is fp32;
  * S = Q K^T and dP = dO V^T accumulate in fp32;
  * P = exp2(scale log2e S - log2e L) in fp32, D = sum dO O in fp32;
  * P and dS are rounded to 16 bits where they become matrix operands;
  * dV = P^T dO, dK = scale dS^T Q and dQ = scale dS K accumulate in fp32
    and are rounded to 16 bits once.
The model must sit well inside the bar (at most half of it), and every
planted kernel-side mistake below (a dropped term, a wrong sign or index, a
skipped tile, a transposed operand) must fail it. The model is test code of
its own: it shares nothing with the HIP kernels and is not the oracle, which
supplies the reference gradients in float64.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_backward_dense, attention_dense
from tests.gpu_util import to_f64
from tests.test_gpu_backward import EPS_O, assert_grad_close, dense_terms

LOG2E = np.float32(1.4426950408889634)
TILE = 64   # rows of a streamed query or key tile


def _r16(x, dtype):
    """fp32 values rounded to the 16-bit type (round to nearest even), as fp32."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
    return W.f16_bits_to_f32(W.f32_to_f16_bits(x))


def model_head(q, k, v, do, o, L, scale, causal, dtype, mistake=None):
    """One head (rows x d, fp32 holding 16-bit values; L fp32) -> dq, dk, dv, D in fp32."""
    Nq, Nk, d = q.shape[0], k.shape[0], q.shape[1]
    f32 = np.float32
    S = q @ k.T                                     # fp32 accumulate
    dP = do @ v.T
    D = np.sum(do * o, axis=1, dtype=f32)           # fp32
    if mistake == "d_wrong_row":
        D = np.roll(D, -1)
    L2 = L.astype(f32) * LOG2E
    if mistake == "l_not_base2":
        L2 = L.astype(f32)
    if mistake == "l_wrong_row":
        L2 = np.roll(L2, 1)
    sl2 = f32(scale) * LOG2E
    if mistake == "scale_missing_in_p":
        sl2 = LOG2E
    P = np.exp2(S * sl2 - L2[:, None]).astype(f32)
    qi = np.arange(Nq)[:, None]
    kj = np.arange(Nk)[None, :]
    if causal:
        off = Nk - Nq
        seen = kj <= qi + off
        if mistake == "diagonal_excluded":
            seen = kj < qi + off
        P = np.where(seen, P, f32(0))
    if mistake == "delta_dropped":
        dS = P * dP
    elif mistake == "delta_sign":
        dS = P * (dP + D[:, None])
    else:
        dS = P * (dP - D[:, None])
    P16, dS16 = _r16(P, dtype), _r16(dS, dtype)
    if mistake == "ds_for_p_in_dv":
        P16 = dS16
    # dK / dV: the key-stationary pass over query tiles.
    Pk, dSk, qk, dok = P16, dS16, q, do
    if mistake == "last_query_tile_skipped":
        last = (Nq - 1) // TILE * TILE
        Pk, dSk = P16.copy(), dS16.copy()
        Pk[last:] = 0
        dSk[last:] = 0
    if mistake == "query_rows_permuted_in_dv":
        # A transposing read of dO that hands rows {4..7} and {8..11} of every
        # 16-row step in swapped order while P keeps its own order.
        perm = np.arange(Nq)
        for base in range(0, Nq - 15, 16):
            perm[base + 4:base + 8], perm[base + 8:base + 12] = (
                np.arange(base + 8, base + 12), np.arange(base + 4, base + 8))
        dok = do[perm]
    dv = Pk.T @ dok
    dk = f32(scale) * (dSk.T @ qk)
    if mistake == "dk_scale_missing":
        dk = dSk.T @ qk
    if mistake == "dk_accumulated_in_16_bits":
        acc = np.zeros((Nk, d), dtype=f32)
        for t0 in range(0, Nq, TILE):
            acc = _r16(acc + dSk[t0:t0 + TILE].T @ qk[t0:t0 + TILE], dtype)
        dk = f32(scale) * acc
    # dQ: the query-stationary pass over key tiles.
    dSq, kq = dS16, k
    if mistake == "last_key_tile_skipped":
        last = (Nk - 1) // TILE * TILE
        dSq = dS16.copy()
        dSq[:, last:] = 0
    if mistake == "key_tile_shifted_in_dq":
        # K of the next key tile paired with the dS of this one (the last tile
        # takes the first).
        kq = np.roll(k, -TILE, axis=0)
    dq = f32(scale) * (dSq @ kq)
    if mistake == "dq_scale_missing":
        dq = dSq @ kq
    if mistake == "d256_halves_swapped" and d == 256:
        dk = np.concatenate([dk[:, 128:], dk[:, :128]], axis=1)
    return _r16(dq, dtype), _r16(dk, dtype), _r16(dv, dtype), D


CASES = [
    # (B, Nq, Nk, H, d, causal, dtype, seed): several 64-row tiles with ragged tails
    (1, 200, 200, 2, 64, False, "bf16", 21),
    (1, 200, 200, 2, 128, True, "bf16", 22),
    (1, 129, 300, 2, 128, False, "bf16", 23),
    (1, 300, 300, 1, 256, True, "bf16", 24),
    (1, 200, 200, 2, 128, True, "f16", 25),
]


def _setup(B, Nq, Nk, H, d, causal, dtype, seed):
    q, k, v = W.make_dense(B, Nq, H, d, seed, Nk=Nk, dtype=dtype)
    do, _, _ = W.make_dense(B, Nq, H, d, seed + 1, dtype=dtype)
    scale = 1 / np.sqrt(d)
    qf, kf, vf, dof = (to_f64(x, dtype) for x in (q, k, v, do))
    oref, lref = attention_dense(qf, kf, vf, scale, causal)
    o16 = _r16(oref, dtype)                          # the forward's 16-bit O
    l32 = lref.astype(np.float32)                    # and its fp32 L
    ref = attention_backward_dense(qf, kf, vf, dof, scale, causal)
    extra = dense_terms(qf, kf, vf, dof, scale, causal, EPS_O[dtype])
    return (qf, kf, vf, dof, o16, l32, scale), ref, extra


def _model(inputs, causal, dtype, mistake=None):
    qf, kf, vf, dof, o16, l32, scale = inputs
    B, Nq, H, d = qf.shape
    Nk = kf.shape[1]
    dq = np.zeros((B, Nq, H, d)); dk = np.zeros((B, Nk, H, d)); dv = np.zeros((B, Nk, H, d))
    D = np.zeros((B, H, Nq))
    f32 = np.float32
    for b in range(B):
        for h in range(H):
            with np.errstate(over="ignore", invalid="ignore"):   # planted mistakes may overflow
                g = model_head(qf[b, :, h].astype(f32), kf[b, :, h].astype(f32), vf[b, :, h].astype(f32),
                               dof[b, :, h].astype(f32), o16[b, :, h], l32[b, h], scale, causal,
                               dtype, mistake)
            dq[b, :, h], dk[b, :, h], dv[b, :, h], D[b, h] = g
    return dq, dk, dv, D


def _check(got, ref, extra, what, dtype, margin=1.0):
    """The GPU tests' bar; margin < 1 asks the error to fit in that fraction of it."""
    gq, gk, gv, gd = ref
    tq, tk, dD = extra
    dq, dk, dv, D = got
    for name, g, r, e, per_row in (("dq", dq, gq, tq, True), ("dk", dk, gk, tk, True),
                                   ("dv", dv, gv, 0.0, True), ("delta", D, gd, dD, False)):
        # err <= margin * (bound + extra)  <=>  r + (g - r) / margin passes the bar
        assert_grad_close(r + (g - r) / margin, r, f"{name} {what}", per_row=per_row, extra=e,
                          dtype=dtype)


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"N{c[1]}x{c[2]}_d{c[4]}_{'c' if c[5] else 'n'}_{c[6]}")
def test_kernel_model_within_half_the_bar(case):
    B, Nq, Nk, H, d, causal, dtype, seed = case
    inputs, ref, extra = _setup(*case)
    _check(_model(inputs, causal, dtype), ref, extra, f"model {case}", dtype, margin=0.5)


# Each of these is a structural mistake and fails the bar on some case. A
# precision mistake can pass it: dK partial sums rounded to 16 bits after
# every query tile ("dk_accumulated_in_16_bits" in model_head) use 0.2-0.3 of
# the bar at 200-300 rows and 0.6 at 1025; the bar is about three times the
# model's own error, so it catches an error growth of that order, not less.
MISTAKES = [
    "delta_dropped", "delta_sign", "d_wrong_row", "l_not_base2", "l_wrong_row",
    "scale_missing_in_p", "diagonal_excluded", "ds_for_p_in_dv", "last_query_tile_skipped",
    "query_rows_permuted_in_dv", "dk_scale_missing", "last_key_tile_skipped",
    "key_tile_shifted_in_dq", "dq_scale_missing", "d256_halves_swapped",
]


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_kernel_mistake_fails_the_bar(mistake):
    caught = []
    for case in CASES:
        B, Nq, Nk, H, d, causal, dtype, seed = case
        if mistake == "diagonal_excluded" and not causal:
            continue
        if mistake == "d256_halves_swapped" and d != 256:
            continue
        inputs, ref, extra = _setup(*case)
        try:
            _check(_model(inputs, causal, dtype, mistake), ref, extra, f"{mistake} {case}", dtype)
        except AssertionError:
            caught.append(case)
    assert caught, f"the bar accepts the planted mistake {mistake!r} on every case"
