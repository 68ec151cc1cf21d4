"""Backward (fa_bwd / fa_bwd_varlen): HIP path vs the float64 CPU oracle.

The kernels receive O and L computed by the oracle's forward (O rounded to
the input type, L to fp32), so these tests check the backward alone; one
test chains the HIP forward into the HIP backward.

Tolerance (no figure on the pages): a gradient row (one token, one head,
d values) is a sum of products of 16-bit P or dS with 16-bit dO, Q or K,
accumulated in fp32 and rounded to 16 bits once. The rounding of P and dS
(2^-9 relative for bf16) dominates, and its sum stays within a few 2^-9 of
that row's own RMS. Rows differ in scale by an order of magnitude: a causal
row that sees only a few keys has dS values of several units, and its dQ
row (and the dK rows of the keys it sees) are far above the tensor's RMS.
The bar is |gpu - ref| <= 2e-2 (rms_row(ref) + |ref|) + 1e-3 rms(ref) per
element for bf16 (the middle term covers rows that are exactly zero, such as
dQ of a row with one visible key). fp16 rounds 8 times finer (unit roundoff
2^-11 against 2^-8), so its bar is both terms divided by 8. A CPU model of
the kernels' arithmetic stays within a third of the bar, and planted kernel
mistakes fail it (tests/test_bwd_bar.py).

One more term, derived rather than tuned: the method forms D_i = dO_i . O_i
from the 16-bit O the forward returned, not from the exact O (the identity
D_i = sum_j P_ij dP_ij holds only for the exact one). Rounding O by a
relative eps moves D_i by at most dD_i = eps sum_e |dO_ie O_ie|, which moves
dS_ij by P_ij dD_i with the same sign across the row, so it does not cancel:
it adds up to scale dD_i sum_j P_ij |K_je| to dQ and scale sum_i P_ij dD_i
|Q_ie| to dK (dV does not depend on D). eps is 2^-8 for bf16 and 2^-10 for
fp16 (twice the unit roundoff), and 2^-6 where O comes from the HIP forward
(its own P and output rounding). D itself is one value per row:
|gpu - ref| <= 2e-2 (rms(ref) + |ref|) + dD.
"""
import numpy as np
import pytest

import workloads as W
from oracle import (attention_backward_dense, attention_backward_varlen, attention_dense,
                    attention_probs, attention_varlen)
from tests.gpu_util import say, to_dev, to_f64, torch_or_skip

pytestmark = pytest.mark.gpu
G_TOL = 2e-2
TOL_SCALE = {"bf16": 1.0, "f16": 1.0 / 8}    # the bar follows the type's unit roundoff
EPS_O = {"bf16": 2.0**-8, "f16": 2.0**-10}   # relative rounding of O, doubled
EPS_O_HIP = 2.0**-6                          # O from the HIP forward


def d_rounding_terms(qf, kf, vf, dof, scale, causal, eps, window=None, P=None):
    """One head: the dq, dk and D bounds of the D-from-16-bit-O rounding (module docstring)."""
    if P is None:
        P = attention_probs(qf, kf, scale, causal, window=window)
    O = P @ vf
    dD = eps * np.sum(np.abs(dof * O), axis=1)                       # (Nq,)
    # bounds on magnitudes: the scale enters with its absolute value
    tq = abs(scale) * dD[:, None] * (P @ np.abs(kf))                 # (Nq, d)
    tk = abs(scale) * (P.T @ (dD[:, None] * np.abs(qf)))             # (Nk, d)
    return tq, tk, dD


def dense_terms(qf, kf, vf, dof, scale, causal, eps, window=None, mask=None):
    """d_rounding_terms over (B, N, H, d) tensors: tq, tk in the tensors' layouts, dD (B, H, Nq).
    mask: key padding mask (B, S); P is then that of the valid tokens, zero elsewhere."""
    B, Nq, H, _ = qf.shape
    tq, tk = np.zeros_like(qf), np.zeros_like(kf)
    dD = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            P = None
            if mask is not None:
                idx = np.nonzero(mask[b])[0]
                P = np.zeros((Nq, kf.shape[1]))
                if idx.size:
                    P[np.ix_(idx, idx)] = attention_probs(qf[b, idx, h], kf[b, idx, h], scale, causal)
            tq[b, :, h], tk[b, :, h], dD[b, h] = d_rounding_terms(
                qf[b, :, h], kf[b, :, h], vf[b, :, h], dof[b, :, h], scale, causal, eps,
                window=window, P=P)
    return tq, tk, dD


def assert_grad_close(got, ref, what, per_row=True, extra=0.0, dtype="bf16"):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(got - ref)
    tol = G_TOL * TOL_SCALE[dtype]
    if per_row:
        row_rms = np.sqrt(np.mean(ref * ref, axis=-1, keepdims=True))
        bound = tol * (row_rms + np.abs(ref)) + tol / 20 * rms
    else:
        bound = tol * (rms + np.abs(ref))
    bad = err > bound + extra
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance, first {idx}: "
                             f"gpu {got[idx]} ref {ref[idx]} (rms {rms:.3e}, max err {err.max():.3e})")


def _round(x64, dtype):
    """float64 values -> 16-bit patterns of dtype."""
    x = np.asarray(x64, dtype=np.float32)
    return W.f32_to_bf16_bits(x) if dtype == "bf16" else W.f32_to_f16_bits(x)


def _np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def check_bwd_dense(B, Nq, Nk, H, d, causal, seed, dtype="bf16", scale=None):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say(f"bwd dense B={B} Nq={Nq} Nk={Nk} H={H} d={d} causal={causal} dtype={dtype} seed={seed}")
    q, k, v = W.make_dense(B, Nq, H, d, seed, Nk=Nk, dtype=dtype)
    do, _, _ = W.make_dense(B, Nq, H, d, seed + 1, dtype=dtype)
    scale = 1 / np.sqrt(d) if scale is None else scale
    qf, kf, vf, dof = (to_f64(x, dtype) for x in (q, k, v, do))
    oref, lref = attention_dense(qf, kf, vf, scale, causal)
    dq, dk, dv, delta = aa.fa_bwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype),
                                  to_dev(_round(oref, dtype), dtype),
                                  torch.from_numpy(lref.astype(np.float32)).cuda(),
                                  to_dev(do, dtype), softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    gq, gk, gv, gd = attention_backward_dense(qf, kf, vf, dof, scale, causal)
    tq, tk, dD = dense_terms(qf, kf, vf, dof, scale, causal, EPS_O[dtype])
    what = f"Nq={Nq} Nk={Nk} d={d} causal={causal} {dtype} scale={scale}"
    assert_grad_close(_np(dq), gq, "dq " + what, extra=tq, dtype=dtype)
    assert_grad_close(_np(dk), gk, "dk " + what, extra=tk, dtype=dtype)
    assert_grad_close(_np(dv), gv, "dv " + what, dtype=dtype)
    assert_grad_close(_np(delta), gd, "delta " + what, per_row=False, extra=dD, dtype=dtype)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 200])
def test_bwd_dense(d, causal, N):
    check_bwd_dense(2, N, N, 2, d, causal, seed=8000 + N + d)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("Nq,Nk", [(129, 300), (300, 129), (1, 77)])
def test_bwd_cross_lengths(d, Nq, Nk):
    check_bwd_dense(1, Nq, Nk, 2, d, False, seed=8100 + Nq + d)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_long_rows(causal):
    # 6 key tiles of 128 rows for dK/dV, 6 query tiles for dQ, 64-row streamed tiles.
    check_bwd_dense(1, 700, 700, 2, 128, causal, seed=8200)


@pytest.mark.parametrize("d", [32, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_f16(d, causal):
    check_bwd_dense(2, 333, 333, 2, d, causal, seed=8300 + d, dtype="f16")


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_varlen(causal, d):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [1, 127, 0, 200, 64, 300]
    H = 2
    say(f"bwd varlen lengths={lengths} causal={causal} d={d}")
    q, k, v, cu = W.make_varlen(lengths, H, d, seed=8400)
    do, _, _, _ = W.make_varlen(lengths, H, d, seed=8401)
    scale = 1 / np.sqrt(d)
    qf, kf, vf, dof = (to_f64(x) for x in (q, k, v, do))
    oref, lref = attention_varlen(qf, kf, vf, cu, scale, causal)
    dq, dk, dv, delta = aa.fa_bwd_varlen(to_dev(q), to_dev(k), to_dev(v), to_dev(_round(oref, "bf16")),
                                         torch.from_numpy(lref.astype(np.float32)).cuda(), to_dev(do),
                                         torch.from_numpy(cu).cuda(), max(lengths),
                                         softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    gq, gk, gv, gd = attention_backward_varlen(qf, kf, vf, dof, cu, scale, causal)
    tq, tk, dD = np.zeros_like(qf), np.zeros_like(kf), np.zeros((H, qf.shape[0]))
    for s_ in range(len(lengths)):
        a, b = int(cu[s_]), int(cu[s_ + 1])
        for h in range(H):
            if b > a:
                tq[a:b, h], tk[a:b, h], dD[h, a:b] = d_rounding_terms(
                    qf[a:b, h], kf[a:b, h], vf[a:b, h], dof[a:b, h], scale, causal, EPS_O["bf16"])
    assert_grad_close(_np(dq), gq, f"varlen dq causal={causal}", extra=tq)
    assert_grad_close(_np(dk), gk, f"varlen dk causal={causal}", extra=tk)
    assert_grad_close(_np(dv), gv, f"varlen dv causal={causal}")
    assert_grad_close(_np(delta), gd, f"varlen delta causal={causal}", per_row=False, extra=dD)


def test_bwd_single_key_closed_form():
    """One key: P = 1, so dq = dk = 0 and dv = the sum of dO over the queries."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("bwd single key")
    q, k, v = (to_dev(x) for x in W.make_dense(1, 300, 2, 64, seed=8500, Nk=1))
    do = to_dev(W.make_dense(1, 300, 2, 64, seed=8501)[0])
    o, lse = aa.fa_fwd(q, k, v)
    dq, dk, dv, _ = aa.fa_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    # dS = P (dP - D) is 0 up to D: here O = v0 exactly (one key), so dP and D are
    # two fp32 sums of the same 64 products
    assert float(dq.abs().max()) <= 1e-3 and float(dk.abs().max()) <= 1e-3
    want = do.double().sum(dim=1, keepdim=True)
    assert_grad_close(_np(dv), want.cpu().numpy(), "dv = sum of dO")


def test_bwd_chained_with_forward_and_autograd():
    """HIP forward -> HIP backward against the oracle, and the autograd wrapper
    gives the same gradients bit for bit."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, N, H, d = 2, 400, 2, 128
    say("bwd chained with the HIP forward, autograd wrapper")
    q, k, v = W.make_dense(B, N, H, d, seed=8600)
    do = W.make_dense(B, N, H, d, seed=8601)[0]
    qd, kd, vd, dod = (to_dev(x) for x in (q, k, v, do))
    o, lse = aa.fa_fwd(qd, kd, vd, causal=True)
    dq, dk, dv, _ = aa.fa_bwd(qd, kd, vd, o, lse, dod, causal=True)
    qa, ka, va = (x.clone().requires_grad_(True) for x in (qd, kd, vd))
    oa = aa.attention(qa, ka, va, causal=True)
    oa.backward(dod)
    torch.cuda.synchronize()
    for a, b, n in ((qa.grad, dq, "dq"), (ka.grad, dk, "dk"), (va.grad, dv, "dv")):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), n
    f = [to_f64(x) for x in (q, k, v, do)]
    gq, gk, gv, _ = attention_backward_dense(*f, 1 / np.sqrt(d), True)
    tq, tk, _ = dense_terms(*f, 1 / np.sqrt(d), True, EPS_O_HIP)
    assert_grad_close(_np(dq), gq, "chained dq", extra=tq)
    assert_grad_close(_np(dk), gk, "chained dk", extra=tk)
    assert_grad_close(_np(dv), gv, "chained dv")


def test_bwd_deterministic():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("bwd determinism")
    q, k, v = (to_dev(x) for x in W.make_dense(1, 600, 4, 64, seed=8700))
    do = to_dev(W.make_dense(1, 600, 4, 64, seed=8701)[0])
    o, lse = aa.fa_fwd(q, k, v)
    g1 = aa.fa_bwd(q, k, v, o, lse, do)
    g2 = aa.fa_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    for a, b in zip(g1[:3], g2[:3]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(g1[3], g2[3])


def test_bwd_full_size_prefill_sampled():
    """prefill2k's shape (B=4, H=32, N=2048, d=128, causal): whole (batch, head)
    pairs against the oracle, and at every head the key-shift invariant: the dK
    rows sum to zero (relative to their scale)."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS["prefill2k"]
    say(f"bwd full-size prefill2k B={w.B} N={w.N} H={w.H}")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed)
    do = W.make_dense(w.B, w.N, w.H, w.d, w.seed + 1)[0]
    qd, kd, vd, dod = (to_dev(x) for x in (q, k, v, do))
    o, lse = aa.fa_fwd(qd, kd, vd, causal=True)
    dq, dk, dv, delta = aa.fa_bwd(qd, kd, vd, o, lse, dod, causal=True)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (2, 13)]:
        sl = lambda x: to_f64(x[b:b + 1, :, h:h + 1])  # noqa: E731
        gq, gk, gv, _ = attention_backward_dense(sl(q), sl(k), sl(v), sl(do), w.scale, True)
        tq, tk, _ = dense_terms(sl(q), sl(k), sl(v), sl(do), w.scale, True, EPS_O_HIP)
        assert_grad_close(_np(dq[b:b + 1, :, h:h + 1]), gq, f"prefill2k dq b={b} h={h}", extra=tq)
        assert_grad_close(_np(dk[b:b + 1, :, h:h + 1]), gk, f"prefill2k dk b={b} h={h}", extra=tk)
        assert_grad_close(_np(dv[b:b + 1, :, h:h + 1]), gv, f"prefill2k dv b={b} h={h}")
    dkf = dk.double()
    colsum = dkf.sum(dim=1).abs()                            # (B, H, d)
    scale_ = dkf.abs().sum(dim=1)
    assert torch.isfinite(dkf).all() and torch.isfinite(dq.double()).all()
    assert bool((colsum <= 2e-2 * scale_ + 1e-3).all()), float((colsum / scale_).max())


# ---------------------------------------------------------------------------
# Backward of the banded and the padded forward
# ---------------------------------------------------------------------------

from oracle import attention_backward_padded, attention_padded  # noqa: E402


def check_bwd_band(B, Nq, Nk, H, d, window, seed):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say(f"bwd band B={B} Nq={Nq} Nk={Nk} H={H} d={d} window={window} seed={seed}")
    q, k, v = W.make_dense(B, Nq, H, d, seed, Nk=Nk)
    do = W.make_dense(B, Nq, H, d, seed + 1)[0]
    scale = 1 / np.sqrt(d)
    qf, kf, vf, dof = (to_f64(x) for x in (q, k, v, do))
    oref, lref = attention_dense(qf, kf, vf, scale, window=window)
    dq, dk, dv, delta = aa.fa_bwd(to_dev(q), to_dev(k), to_dev(v), to_dev(_round(oref, "bf16")),
                                  torch.from_numpy(lref.astype(np.float32)).cuda(), to_dev(do),
                                  softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    gq, gk, gv, gd = attention_backward_dense(qf, kf, vf, dof, scale, window=window)
    tq, tk, dD = dense_terms(qf, kf, vf, dof, scale, False, EPS_O["bf16"], window=window)
    what = f"band {window} Nq={Nq} Nk={Nk} d={d}"
    assert_grad_close(_np(dq), gq, "dq " + what, extra=tq)
    assert_grad_close(_np(dk), gk, "dk " + what, extra=tk)
    assert_grad_close(_np(dv), gv, "dv " + what)
    assert_grad_close(_np(delta), gd, "delta " + what, per_row=False, extra=dD)


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", [(None, 0), (16, 16), (100, 3), (0, None), (0, 0)])
@pytest.mark.parametrize("Nq,Nk", [(333, 333), (129, 300), (300, 129)])
def test_bwd_band(d, window, Nq, Nk):
    # (300, 129): off = -171, rows before it see no key with a bounded right side.
    check_bwd_band(1, Nq, Nk, 2, d, window, seed=8800 + Nq + Nk + d)


def test_bwd_band_long_rows():
    check_bwd_band(1, 1000, 1000, 2, 128, (300, 40), seed=8850)


def test_bwd_band_varlen():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [1, 127, 0, 300, 64]
    window = (20, 5)
    say(f"bwd band varlen lengths={lengths} window={window}")
    q, k, v, cu = W.make_varlen(lengths, 2, 64, seed=8870)
    do, _, _, _ = W.make_varlen(lengths, 2, 64, seed=8871)
    scale = 1 / 8.0
    qf, kf, vf, dof = (to_f64(x) for x in (q, k, v, do))
    oref, lref = attention_varlen(qf, kf, vf, cu, scale, window=window)
    dq, dk, dv, _ = aa.fa_bwd_varlen(to_dev(q), to_dev(k), to_dev(v), to_dev(_round(oref, "bf16")),
                                     torch.from_numpy(lref.astype(np.float32)).cuda(), to_dev(do),
                                     torch.from_numpy(cu).cuda(), max(lengths), softmax_scale=scale,
                                     window=window)
    torch.cuda.synchronize()
    gq, gk, gv, _ = attention_backward_varlen(qf, kf, vf, dof, cu, scale, window=window)
    tq, tk = np.zeros_like(qf), np.zeros_like(kf)
    for s_ in range(len(lengths)):
        a, b = int(cu[s_]), int(cu[s_ + 1])
        for h in range(2):
            if b > a:
                tq[a:b, h], tk[a:b, h], _ = d_rounding_terms(
                    qf[a:b, h], kf[a:b, h], vf[a:b, h], dof[a:b, h], scale, False, EPS_O["bf16"],
                    window=window)
    assert_grad_close(_np(dq), gq, "band varlen dq", extra=tq)
    assert_grad_close(_np(dk), gk, "band varlen dk", extra=tk)
    assert_grad_close(_np(dv), gv, "band varlen dv")


@pytest.mark.parametrize("d,S", [(64, 333), (128, 333), (128, 1025), (256, 333)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_padded(d, S, causal):
    # Masks: right padding, scattered holes, all valid, all padding, a middle
    # run (one batch row each); at S = 1025 whole workgroups lie outside the
    # span of valid tokens.
    import aware_attention_amd as aa
    from tests.test_gpu_padded import _masks
    torch = torch_or_skip()
    B, H = 5, 2
    say(f"bwd padded B={B} S={S} d={d} causal={causal}")
    q, k, v = W.make_dense(B, S, H, d, seed=8900 + d + S)
    do = W.make_dense(B, S, H, d, seed=8901 + d + S)[0]
    mask = _masks(B, S, 8900 + d + S)
    scale = 1 / np.sqrt(d)
    qf, kf, vf, dof = (to_f64(x) for x in (q, k, v, do))
    oref, lref = attention_padded(qf, kf, vf, mask, scale, causal)
    dq, dk, dv, delta = aa.fa_bwd(to_dev(q), to_dev(k), to_dev(v), to_dev(_round(oref, "bf16")),
                                  torch.from_numpy(lref.astype(np.float32)).cuda(), to_dev(do),
                                  softmax_scale=scale, causal=causal,
                                  key_padding_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    gq, gk, gv, gd = attention_backward_padded(qf, kf, vf, dof, mask, scale, causal)
    tq, tk, dD = dense_terms(qf, kf, vf, dof, scale, causal, EPS_O["bf16"], mask=mask)
    what = f"padded d={d} causal={causal}"
    assert_grad_close(_np(dq), gq, "dq " + what, extra=tq)
    assert_grad_close(_np(dk), gk, "dk " + what, extra=tk)
    assert_grad_close(_np(dv), gv, "dv " + what)
    pad = mask == 0
    for t, n in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert np.all(_np(t)[pad] == 0), f"{n} must be 0 at padding positions"


def test_autograd_with_band_and_padding_mask():
    """The autograd wrapper passes the band and the padding mask to both passes
    (bitwise equal to the direct calls)."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("autograd with band and padding mask")
    q, k, v = (to_dev(x) for x in W.make_dense(2, 300, 2, 64, seed=8950))
    do = to_dev(W.make_dense(2, 300, 2, 64, seed=8951)[0])
    mask = torch.from_numpy(np.array([[1] * 200 + [0] * 100, [1] * 300], dtype=np.uint8)).cuda()
    for kw in (dict(window=(30, 0)), dict(key_padding_mask=mask, causal=True)):
        o, lse = aa.fa_fwd(q, k, v, **kw)
        g = aa.fa_bwd(q, k, v, o, lse, do, **kw)
        qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
        aa.attention(qa, ka, va, **kw).backward(do)
        torch.cuda.synchronize()
        for a, b_ in zip((qa.grad, ka.grad, va.grad), g[:3]):
            assert torch.equal(a.view(torch.int16), b_.view(torch.int16)), str(kw.keys())


# ---------------------------------------------------------------------------
# Backward of the local window + global anchor pattern
# ---------------------------------------------------------------------------

from oracle import attention_local_backward_dense, attention_local_dense, local_visible  # noqa: E402


def _local_terms(qf, kf, vf, dof, scale, G, Wd, wr, wc, causal, eps):
    """D-rounding bounds (module docstring) with the local pattern's P."""
    B, N, H, _ = qf.shape
    vis = local_visible(N, G, Wd, wr, wc, causal)
    tq, tk = np.zeros_like(qf), np.zeros_like(kf)
    for b in range(B):
        for h in range(H):
            S = np.where(vis, scale * qf[b, :, h] @ kf[b, :, h].T, -np.inf)
            e = np.exp(S - S.max(axis=1, keepdims=True))
            P = e / e.sum(axis=1, keepdims=True)
            tq[b, :, h], tk[b, :, h], _ = d_rounding_terms(
                qf[b, :, h], kf[b, :, h], vf[b, :, h], dof[b, :, h], scale, causal, eps, P=P)
    return tq, tk


def check_bwd_local(B, N, H, d, G, Wd, win, causal, seed):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    wr, wc = win
    say(f"bwd local B={B} N={N} H={H} d={d} G={G} map_w={Wd} win={win} causal={causal} "
        f"seed={seed}")
    q, k, v = W.make_dense(B, N, H, d, seed)
    do = W.make_dense(B, N, H, d, seed + 1)[0]
    scale = 1 / np.sqrt(d)
    qf, kf, vf, dof = (to_f64(x) for x in (q, k, v, do))
    oref, lref = attention_local_dense(qf, kf, vf, scale, G, Wd, wr, wc, causal)
    dq, dk, dv, delta = aa.fa_bwd(to_dev(q), to_dev(k), to_dev(v), to_dev(_round(oref, "bf16")),
                                  torch.from_numpy(lref.astype(np.float32)).cuda(), to_dev(do),
                                  softmax_scale=scale, causal=causal, local=(G, Wd, wr, wc))
    torch.cuda.synchronize()
    gq, gk, gv, gd = attention_local_backward_dense(qf, kf, vf, dof, scale, G, Wd, wr, wc, causal)
    tq, tk = _local_terms(qf, kf, vf, dof, scale, G, Wd, wr, wc, causal, EPS_O["bf16"])
    what = f"local G={G} map_w={Wd} win={win} causal={causal} N={N} d={d}"
    assert_grad_close(_np(dq), gq, "dq " + what, extra=tq)
    assert_grad_close(_np(dk), gk, "dk " + what, extra=tk)
    assert_grad_close(_np(dv), gv, "dv " + what)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_local_detector_map(d, causal):
    # 8 anchors + a 20 x 20 map, 5 x 5 window.
    check_bwd_local(2, 8 + 400, 2, d, 8, 20, (2, 2), causal, seed=14000 + d + causal)


@pytest.mark.parametrize("G,Wd,win", [(0, 1, (3, 0)), (70, 13, (0, 0)), (3, 17, (3, 1)),
                                      (0, 40, (1, 1)), (5, 33, (100, 100))])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_local_patterns(G, Wd, win, causal):
    check_bwd_local(1, 333, 2, 64, G, Wd, win, causal, seed=14100 + G + Wd)


@pytest.mark.parametrize("N", [1, 65, 300])
def test_bwd_local_lengths(N):
    check_bwd_local(2, N, 2, 128, min(3, N), 9, (1, 2), N % 2 == 1, seed=14200 + N)


def test_autograd_with_local_pattern():
    """The autograd wrapper with local= runs fa_fwd_local and fa_bwd_local
    (bitwise equal to the direct calls)."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("autograd with the local pattern")
    q, k, v = (to_dev(x) for x in W.make_dense(2, 408, 2, 64, seed=14300))
    do = to_dev(W.make_dense(2, 408, 2, 64, seed=14301)[0])
    loc = (8, 20, 2, 2)
    o, lse = aa.fa_fwd_local(q, k, v, 8, 20, (2, 2))
    g = aa.fa_bwd(q, k, v, o, lse, do, local=loc)
    qa, ka, va = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = aa.attention(qa, ka, va, local=loc)
    out.backward(do)
    torch.cuda.synchronize()
    assert torch.equal(out.detach().view(torch.int16), o.view(torch.int16))
    for a, b_ in zip((qa.grad, ka.grad, va.grad), g[:3]):
        assert torch.equal(a.view(torch.int16), b_.view(torch.int16))


# ---------------------------------------------------------------------------
# Full-size backward of every timed workload, in the launch bench.py times
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["prefill8k", "vit", "det1600", "band8k", "vitpad", "detlocal",
                                  "prefill8k_d256", "band8k_d256"])
def test_bwd_full_size_workloads(name):
    """Whole (batch, head) pairs against the oracle's gradients (one pair at
    N = 8192, two elsewhere), and at every head the key-shift invariant (the
    dK columns sum to zero relative to their scale) and finite gradients."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS[name]
    wl = W.make_workload(name)
    say(f"bwd full-size {name} B={w.B} N={w.N} H={w.H} d={w.d}")
    q, k, v = wl["q"], wl["k"], wl["v"]
    do = W.make_dense(w.B, w.N, w.H, w.d, w.seed + 1)[0]
    qd, kd, vd, dod = (to_dev(x) for x in (q, k, v, do))
    mask = wl.get("mask")
    kpm = torch.from_numpy(mask).cuda() if mask is not None else None
    if w.local is not None:
        G, mw, wr, wc = w.local
        o, lse = aa.fa_fwd_local(qd, kd, vd, G, mw, (wr, wc), softmax_scale=w.scale,
                                 causal=w.causal)
    else:
        o, lse = aa.fa_fwd(qd, kd, vd, softmax_scale=w.scale, causal=w.causal, window=w.window,
                           key_padding_mask=kpm)
    dq, dk, dv, _ = aa.fa_bwd(qd, kd, vd, o, lse, dod, softmax_scale=w.scale, causal=w.causal,
                              window=w.window, key_padding_mask=kpm, local=w.local)
    torch.cuda.synchronize()
    pairs = [(0, w.H // 2)] if w.N > 4096 else [(0, 0), (w.B - 1, w.H - 1)]
    for b, h in pairs:
        sl = lambda x: to_f64(x[b:b + 1, :, h:h + 1])  # noqa: E731
        qf, kf, vf, dof = sl(q), sl(k), sl(v), sl(do)
        if w.local is not None:
            gq, gk, gv, _ = attention_local_backward_dense(qf, kf, vf, dof, w.scale, *w.local,
                                                           w.causal)
            tq, tk = _local_terms(qf, kf, vf, dof, w.scale, *w.local, w.causal, EPS_O_HIP)
        elif mask is not None:
            gq, gk, gv, _ = attention_backward_padded(qf, kf, vf, dof, mask[b:b + 1], w.scale,
                                                      w.causal)
            tq, tk, _ = dense_terms(qf, kf, vf, dof, w.scale, w.causal, EPS_O_HIP,
                                    mask=mask[b:b + 1])
        else:
            gq, gk, gv, _ = attention_backward_dense(qf, kf, vf, dof, w.scale, w.causal,
                                                     window=w.window)
            tq, tk, _ = dense_terms(qf, kf, vf, dof, w.scale, w.causal, EPS_O_HIP,
                                    window=w.window)
        what = f"{name} b={b} h={h}"
        assert_grad_close(_np(dq[b:b + 1, :, h:h + 1]), gq, "dq " + what, extra=tq)
        assert_grad_close(_np(dk[b:b + 1, :, h:h + 1]), gk, "dk " + what, extra=tk)
        assert_grad_close(_np(dv[b:b + 1, :, h:h + 1]), gv, "dv " + what)
    dkf = dk.double()
    colsum = dkf.sum(dim=1).abs()                            # (B, H, d)
    scale_ = dkf.abs().sum(dim=1)
    assert torch.isfinite(dkf).all() and torch.isfinite(dq.double()).all()
    assert torch.isfinite(dv.double()).all()
    assert bool((colsum <= 2e-2 * scale_ + 1e-3).all()), float((colsum / (scale_ + 1e-30)).max())
