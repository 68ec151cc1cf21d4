"""Backward on strided views (fa_bwd_strided / fa_bwd_varlen_strided) and the
packed-QKV autograd path (attention_qkvpacked).

The strided entry points run the kernels of the contiguous ones with other
addresses, so each case first requires the gradients to equal, bit for bit,
those of fa_bwd (fa_bwd_band, fa_bwd_varlen, ...) on contiguous copies of the
same values, and then checks them against the float64 oracle to the bar of
the backward tests (tolerance derivation in test_gpu_backward's docstring).
Outputs written into views of larger tensors must leave every other element
untouched.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_backward_dense, attention_backward_varlen
from tests.gpu_util import say, to_dev, to_f64, torch_or_skip
from tests.test_gpu_backward import EPS_O_HIP, _np, assert_grad_close, d_rounding_terms, dense_terms

pytestmark = pytest.mark.gpu


def _bits_equal(a, b, what):
    import torch
    assert torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16)), what


def _mask_kw(mask):
    return dict(causal=mask == "causal", window=(40, 3) if mask == "band" else None)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mask", ["none", "causal", "band"])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_bwd_packed_qkv_dense(dtype, mask, d):
    """q, k, v views of a (B, S, 3, H, d) tensor, dout a (B, H, S, d) tensor seen as
    (B, S, H, d), dq, dk, dv written into the views of a packed (B, S, 3, H, d)
    gradient: equal to the contiguous call, and to the oracle."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, S, H = 2, 333, 3
    kw = _mask_kw(mask)
    say(f"bwd packed qkv dense dtype={dtype} mask={mask} d={d}")
    bits = np.stack(W.make_dense(B, S, H, d, seed=9100 + d, dtype=dtype), axis=2)
    dobits = W.make_dense(B, S, H, d, seed=9101 + d, dtype=dtype)[0]
    qkv = to_dev(bits, dtype)
    q, k, v = qkv.unbind(2)
    do_c = to_dev(dobits, dtype)
    do_v = do_c.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)   # head stride S d
    assert do_v.stride(2) == S * d and q.stride(1) == 3 * H * d
    o, lse = aa.fa_fwd(q, k, v, **kw)
    dqkv = torch.full_like(qkv, float("nan"))
    dq, dk, dv = dqkv.unbind(2)
    _, _, _, delta = aa.fa_bwd(q, k, v, o, lse, do_v, dq=dq, dk=dk, dv=dv, **kw)
    qc, kc, vc = q.contiguous(), k.contiguous(), v.contiguous()
    rq, rk, rv, rdelta = aa.fa_bwd(qc, kc, vc, o, lse, do_c, **kw)
    torch.cuda.synchronize()
    for a, b, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        _bits_equal(a, b, f"packed vs contiguous {n}")
    assert torch.equal(delta, rdelta)
    f = [to_f64(x, dtype) for x in (bits[:, :, 0], bits[:, :, 1], bits[:, :, 2], dobits)]
    scale = 1 / np.sqrt(d)
    gq, gk, gv, _ = attention_backward_dense(*f, scale, kw["causal"], window=kw["window"])
    tq, tk, _ = dense_terms(*f, scale, kw["causal"], EPS_O_HIP, window=kw["window"])
    what = f"packed {dtype} {mask} d={d}"
    assert_grad_close(_np(dq), gq, "dq " + what, extra=tq, dtype=dtype)
    assert_grad_close(_np(dk), gk, "dk " + what, extra=tk, dtype=dtype)
    assert_grad_close(_np(dv), gv, "dv " + what, dtype=dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mask", ["none", "causal", "band"])
def test_bwd_packed_qkv_varlen(dtype, mask):
    """(total, 3, H, d) packed QKV and gradient for a varlen batch with empty,
    one-token and multi-tile sequences."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [129, 1, 0, 400, 64]
    H, d = 2, 128
    kw = dict(causal=mask == "causal", window=(17, 17) if mask == "band" else None)
    say(f"bwd packed qkv varlen dtype={dtype} mask={mask}")
    q, k, v, cu = W.make_varlen(lengths, H, d, seed=9200, dtype=dtype)
    dobits = W.make_varlen(lengths, H, d, seed=9201, dtype=dtype)[0]
    qkv = to_dev(np.stack([q, k, v], axis=1), dtype)
    qv, kv, vv = qkv.unbind(1)
    cu_t = torch.from_numpy(cu).cuda()
    do = to_dev(dobits, dtype)
    o, lse = aa.fa_fwd_varlen(qv, kv, vv, cu_t, max(lengths), **kw)
    dqkv = torch.full_like(qkv, float("nan"))
    dq, dk, dv = dqkv.unbind(1)
    _, _, _, delta = aa.fa_bwd_varlen(qv, kv, vv, o, lse, do, cu_t, max(lengths), dq=dq, dk=dk,
                                      dv=dv, **kw)
    rq, rk, rv, rdelta = aa.fa_bwd_varlen(qv.contiguous(), kv.contiguous(), vv.contiguous(), o,
                                          lse, do, cu_t, max(lengths), **kw)
    torch.cuda.synchronize()
    for a, b, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        _bits_equal(a, b, f"packed varlen vs contiguous {n}")
    assert torch.equal(delta, rdelta)
    qf, kf, vf, dof = (to_f64(x, dtype) for x in (q, k, v, dobits))
    scale = 1 / np.sqrt(d)
    gq, gk, gv, _ = attention_backward_varlen(qf, kf, vf, dof, cu, scale, kw["causal"],
                                              window=kw["window"])
    tq, tk = np.zeros_like(qf), np.zeros_like(kf)
    for s_ in range(len(lengths)):
        a, b = int(cu[s_]), int(cu[s_ + 1])
        for h in range(H):
            if b > a:
                tq[a:b, h], tk[a:b, h], _ = d_rounding_terms(
                    qf[a:b, h], kf[a:b, h], vf[a:b, h], dof[a:b, h], scale, kw["causal"],
                    EPS_O_HIP, window=kw["window"])
    what = f"packed varlen {dtype} {mask}"
    assert_grad_close(_np(dq), gq, "dq " + what, extra=tq, dtype=dtype)
    assert_grad_close(_np(dk), gk, "dk " + what, extra=tk, dtype=dtype)
    assert_grad_close(_np(dv), gv, "dv " + what, dtype=dtype)


def test_bwd_bhsd_layout_and_guarded_outputs():
    """Every tensor in (B, H, S, d) storage seen as (B, S, H, d), cross lengths;
    dq, dk, dv written into the left halves of (..., 2 d) tensors whose right
    halves must stay untouched."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, Nq, Nk, H, d = 2, 190, 300, 4, 64
    say("bwd BHSD layout, guarded outputs")
    q = to_dev(W.make_dense(B, Nq, H, d, seed=9300)[0])
    _, k, v = (to_dev(x) for x in W.make_dense(B, Nq, H, d, seed=9301, Nk=Nk))
    do = to_dev(W.make_dense(B, Nq, H, d, seed=9302)[0])
    bhsd = lambda x: x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)  # noqa: E731
    qh, kh, vh, doh = (bhsd(x) for x in (q, k, v, do))
    o, lse = aa.fa_fwd(q, k, v)
    oh = bhsd(o)
    guards = [torch.full((B, n, H, 2 * d), float("nan"), dtype=torch.bfloat16, device="cuda")
              for n in (Nq, Nk, Nk)]
    dq, dk, dv = (g[..., :d] for g in guards)
    aa.fa_bwd(qh, kh, vh, oh, lse, doh, dq=dq, dk=dk, dv=dv)
    rq, rk, rv, _ = aa.fa_bwd(q, k, v, o, lse, do)
    torch.cuda.synchronize()
    for a, b, n in ((dq, rq, "dq"), (dk, rk, "dk"), (dv, rv, "dv")):
        _bits_equal(a, b, f"BHSD vs contiguous {n}")
    for g in guards:
        assert torch.isnan(g[..., d:]).all()


@pytest.mark.parametrize("causal", [False, True])
def test_attention_qkvpacked_dense(causal):
    """Autograd from one packed tensor: the output and the packed gradient equal
    those of attention() on contiguous q, k, v, bit for bit."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, S, H, d = 2, 257, 4, 128
    say(f"attention_qkvpacked dense causal={causal}")
    bits = np.stack(W.make_dense(B, S, H, d, seed=9400), axis=2)
    do = to_dev(W.make_dense(B, S, H, d, seed=9401)[0])
    qkv = to_dev(bits).requires_grad_(True)
    o = aa.attention_qkvpacked(qkv, causal=causal)
    o.backward(do)
    q, k, v = (to_dev(bits[:, :, i]).requires_grad_(True) for i in range(3))
    oc = aa.attention(q, k, v, causal=causal)
    oc.backward(do)
    torch.cuda.synchronize()
    _bits_equal(o, oc, "O")
    for i, (g, n) in enumerate(((q.grad, "dq"), (k.grad, "dk"), (v.grad, "dv"))):
        _bits_equal(qkv.grad[:, :, i], g, f"packed gradient {n}")


def test_attention_qkvpacked_varlen():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [100, 0, 1, 300]
    H, d = 2, 64
    say("attention_qkvpacked varlen")
    q, k, v, cu = W.make_varlen(lengths, H, d, seed=9500)
    do = to_dev(W.make_varlen(lengths, H, d, seed=9501)[0])
    qkv = to_dev(np.stack([q, k, v], axis=1)).requires_grad_(True)
    cu_t = torch.from_numpy(cu).cuda()
    o = aa.attention_qkvpacked(qkv, causal=True, cu_seqlens=cu_t, max_seqlen=max(lengths))
    o.backward(do)
    oc, lc = aa.fa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), cu_t, max(lengths), causal=True)
    rq, rk, rv, _ = aa.fa_bwd_varlen(to_dev(q), to_dev(k), to_dev(v), oc, lc, do, cu_t,
                                     max(lengths), causal=True)
    torch.cuda.synchronize()
    _bits_equal(o, oc, "varlen O")
    for i, (g, n) in enumerate(((rq, "dq"), (rk, "dk"), (rv, "dv"))):
        _bits_equal(qkv.grad[:, i], g, f"packed varlen gradient {n}")


def test_attention_views_are_not_copied():
    """attention() keeps q, k, v views that the kernels read in place: the tensors
    saved for the backward share the packed tensor's storage."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, S, H, d = 1, 130, 2, 64
    say("attention() on packed views")
    qkv = to_dev(np.stack(W.make_dense(B, S, H, d, seed=9600), axis=2)).requires_grad_(True)
    q, k, v = qkv.unbind(2)
    o = aa.attention(q, k, v, causal=True)
    saved = o.grad_fn.saved_tensors
    assert saved[0].data_ptr() == qkv.data_ptr()
    assert saved[1].data_ptr() == qkv.data_ptr() + H * d * qkv.element_size()
    o.float().sum().backward()     # dout: an expanded tensor (zero strides), copied first
    g = qkv.grad.clone()
    qkv.grad = None
    o2 = aa.attention_qkvpacked(qkv, causal=True)
    o2.float().sum().backward()
    torch.cuda.synchronize()
    _bits_equal(qkv.grad, g, "packed vs views gradient")
