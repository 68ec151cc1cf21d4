"""fp16 inputs and strided views (fa_fwd_strided / fa_fwd_varlen_strided).

fp16 results are compared with the float64 oracle on the same fp16 inputs,
element by element, to the same bar as bf16. Strided views (the packed
(B, S, 3, H, d) QKV tensor, a (B, H, S, d) layout seen as (B, S, H, d), an
output written into part of a larger tensor) must give results bitwise
equal to the same call on contiguous copies: the strides only move where
rows are read and written, never what is computed.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_dense, attention_varlen
from tests.gpu_util import (L_ATOL, assert_l_close, assert_o_close, o_to_f64, say, to_dev,
                            to_f64, torch_or_skip)

pytestmark = pytest.mark.gpu


def _np(t):
    return t.cpu().numpy().astype(np.float64)


def assert_l_band(lg, lref, what):
    empty = np.isneginf(lref)
    assert np.all(np.isneginf(lg[empty])), f"{what}: rows with no visible key need L = -inf"
    if (~empty).any():
        err = float(np.abs(lg[~empty] - lref[~empty]).max())
        assert err <= L_ATOL, f"{what}: L max abs err {err}"


def check_f16_dense(B, Nq, Nk, H, d, causal, seed, window=None):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say(f"f16 dense B={B} Nq={Nq} Nk={Nk} H={H} d={d} causal={causal} window={window}")
    q, k, v = W.make_dense(B, Nq, H, d, seed, Nk=Nk, dtype="f16")
    scale = 1 / np.sqrt(d)
    o, lse = aa.fa_fwd(to_dev(q, "f16"), to_dev(k, "f16"), to_dev(v, "f16"), softmax_scale=scale,
                       causal=causal, window=window)
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    oref, lref = attention_dense(to_f64(q, "f16"), to_f64(k, "f16"), to_f64(v, "f16"), scale,
                                 causal, window=window)
    what = f"f16 Nq={Nq} Nk={Nk} d={d} causal={causal} window={window}"
    assert_o_close(o_to_f64(o), oref, what)
    assert_l_band(_np(lse), lref, what)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 333])
def test_f16_dense(d, causal, N):
    check_f16_dense(2, N, N, 3, d, causal, seed=7000 + N + d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Nq,Nk", [(129, 517), (517, 129)])
def test_f16_cross_lengths(d, Nq, Nk):
    check_f16_dense(1, Nq, Nk, 2, d, False, seed=7100 + Nq + d)


@pytest.mark.parametrize("window", [(None, 0), (30, 30), (0, None)])
def test_f16_band(window):
    check_f16_dense(1, 700, 600, 2, 128, False, seed=7200, window=window)


def test_f16_long_causal_rows():
    check_f16_dense(1, 1500, 1500, 2, 128, True, seed=7250)


@pytest.mark.parametrize("causal", [False, True])
def test_f16_varlen(causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [1, 127, 0, 300, 64, 600]
    say(f"f16 varlen lengths={lengths} causal={causal}")
    q, k, v, cu = W.make_varlen(lengths, 2, 128, seed=7300, dtype="f16")
    o, lse = aa.fa_fwd_varlen(to_dev(q, "f16"), to_dev(k, "f16"), to_dev(v, "f16"),
                              torch.from_numpy(cu).cuda(), max(lengths), causal=causal)
    torch.cuda.synchronize()
    oref, lref = attention_varlen(to_f64(q, "f16"), to_f64(k, "f16"), to_f64(v, "f16"), cu,
                                  1 / np.sqrt(128), causal)
    assert_o_close(o_to_f64(o), oref, "f16 varlen O")
    assert_l_close(_np(lse), lref, "f16 varlen L")


def _equal_bits(a, b, what):
    import torch
    assert torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16)), what


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mask", ["none", "causal", "band"])
def test_packed_qkv_dense(dtype, mask):
    """q, k, v as views of one (B, S, 3, H, d) tensor: token stride 3 H d, head stride d."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, S, H, d = 2, 333, 3, 64
    say(f"packed qkv dense dtype={dtype} mask={mask}")
    bits = np.stack(W.make_dense(B, S, H, d, seed=7400, dtype=dtype), axis=2)   # (B,S,3,H,d)
    qkv = to_dev(bits, dtype)
    q, k, v = qkv.unbind(2)
    assert not q.is_contiguous() and q.stride(1) == 3 * H * d
    kw = dict(causal=mask == "causal", window=(40, 3) if mask == "band" else None)
    o, lse = aa.fa_fwd(q, k, v, **kw)
    oc, lc = aa.fa_fwd(q.contiguous(), k.contiguous(), v.contiguous(), **kw)
    torch.cuda.synchronize()
    _equal_bits(o, oc, "packed vs contiguous O")
    assert torch.equal(lse, lc)
    oref, lref = attention_dense(to_f64(bits[:, :, 0], dtype), to_f64(bits[:, :, 1], dtype),
                                 to_f64(bits[:, :, 2], dtype), 1 / np.sqrt(d), kw["causal"],
                                 window=kw["window"])
    assert_o_close(o_to_f64(o), oref, "packed O")
    assert_l_band(_np(lse), lref, "packed L")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_bhsd_layout_in_and_out(dtype):
    """(B, H, S, d) storage seen as (B, S, H, d) views for q, k, v and o."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, S, H, d = 2, 300, 4, 128
    say(f"BHSD layout dtype={dtype}")
    q, k, v = (to_dev(x, dtype) for x in W.make_dense(B, S, H, d, seed=7500, dtype=dtype))
    qh, kh, vh = (x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for x in (q, k, v))
    assert qh.stride(1) == d and qh.stride(2) == S * d
    o_store = torch.full((B, H, S, d), float("nan"), dtype=q.dtype, device="cuda")
    o_view = o_store.permute(0, 2, 1, 3)
    o, lse = aa.fa_fwd(qh, kh, vh, causal=True, out=o_view)
    oc, lc = aa.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert o.data_ptr() == o_store.data_ptr()
    _equal_bits(o_view, oc, "BHSD vs contiguous O")
    assert torch.equal(lse, lc)


def test_output_into_part_of_a_larger_tensor():
    """o = big[..., :d] of a (B, S, H, 2d) tensor: the other half stays untouched."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, S, H, d = 1, 257, 2, 64
    say("output view with guard half")
    q, k, v = (to_dev(x) for x in W.make_dense(B, S, H, d, seed=7600))
    big = torch.full((B, S, H, 2 * d), float("nan"), dtype=torch.bfloat16, device="cuda")
    o, lse = aa.fa_fwd(q, k, v, out=big[..., :d])
    oc, _ = aa.fa_fwd(q, k, v)
    torch.cuda.synchronize()
    _equal_bits(big[..., :d], oc, "O in the left half")
    assert torch.isnan(big[..., d:]).all()


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mask", ["none", "causal", "band"])
def test_packed_qkv_varlen(dtype, mask):
    """Packed (total, 3, H, d) QKV for a varlen batch, as the unmasked page-2 path builds it."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [129, 1, 0, 400, 64]
    H, d = 2, 128
    say(f"packed qkv varlen dtype={dtype} mask={mask}")
    q, k, v, cu = W.make_varlen(lengths, H, d, seed=7700, dtype=dtype)
    bits = np.stack([q, k, v], axis=1)                        # (total, 3, H, d)
    qkv = to_dev(bits, dtype)
    qv, kv, vv = qkv.unbind(1)
    cu_t = torch.from_numpy(cu).cuda()
    kw = dict(causal=mask == "causal", window=(17, 17) if mask == "band" else None)
    o, lse = aa.fa_fwd_varlen(qv, kv, vv, cu_t, max(lengths), **kw)
    oc, lc = aa.fa_fwd_varlen(qv.contiguous(), kv.contiguous(), vv.contiguous(), cu_t,
                              max(lengths), **kw)
    torch.cuda.synchronize()
    _equal_bits(o, oc, "packed varlen vs contiguous O")
    assert torch.equal(lse, lc)
    oref, lref = attention_varlen(to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype), cu,
                                  1 / np.sqrt(d), kw["causal"], window=kw["window"])
    assert_o_close(o_to_f64(o), oref, "packed varlen O")
    assert_l_band(_np(lse), lref, "packed varlen L")


def test_f16_full_size_prefill_sampled():
    """prefill2k's shape (B=4, H=32, N=2048, d=128, causal) in fp16, sampled rows."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS["prefill2k"]
    say(f"f16 full-size prefill2k B={w.B} N={w.N} H={w.H}")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed, dtype="f16")
    o, lse = aa.fa_fwd(to_dev(q, "f16"), to_dev(k, "f16"), to_dev(v, "f16"), causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 200)
    for b, h in [(0, 0), (w.B - 1, w.H - 1), (1, 17)]:
        rows = sorted({0, 1, 255, 256, w.N - 1} | set(rng.integers(0, w.N, size=40).tolist()))
        oref, lref = attention_dense(to_f64(q[b:b + 1, :, h:h + 1], "f16"),
                                     to_f64(k[b:b + 1, :, h:h + 1], "f16"),
                                     to_f64(v[b:b + 1, :, h:h + 1], "f16"), w.scale, True,
                                     rows=rows)
        assert_o_close(o_to_f64(o[b, rows, h]), oref[0, :, 0], f"f16 prefill2k b={b} h={h}")
        assert_l_close(_np(lse[b, h, rows]), lref[0, 0], f"f16 prefill2k b={b} h={h}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
