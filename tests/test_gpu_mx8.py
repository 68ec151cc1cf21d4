"""FP8 (MX block-scaled) path against the float64 oracle.

Quantisers: the E4M3 bytes and E8M0 exponents the HIP quantisers write are
compared bit for bit with oracle.fp8 (byte work: exact).

Attention: fa_fwd_mx8 on those operands against the definition applied to
their dequantised values (oracle.fp8.attention_mx8). L must agree to 1e-3 as
in the other paths (the scores are exact products of the FP8 values summed in
fp32, and the row sums stay fp32). O additionally carries the kernel's
rounding of P~ to E4M3 before P V; its bar is derived from that format: with
|dP~| <= max(2^-4 P~, 2^-10) per element (3 mantissa bits, subnormal step
2^-9, P~ in units of the running offset, whose sum is at least l, the sum of
e^(s - max)),
    |o_gpu - o_ref| <= 2^-4 sum_j P_j |V_j| + 2^-10 sum_j |V_j| / l
                       + 2^-8 |o_ref| + 1e-4
(the last two: bf16 rounding of O and fp32 accumulation). A statistical
check adds the size of the typical error: the mean of err^2 / sigma^2 with
sigma^2 = sum_j (2^-4 P_j V_j)^2 + (2^-9 o_ref)^2 + 1e-8 must stay below 1
(RNE errors are at most 2^-4 relative and average well under it).
"""
import numpy as np
import pytest

import workloads as W
from oracle import fp8 as F
from oracle.attention import attention_probs
from tests.gpu_util import L_ATOL, say, to_dev, to_f64, torch_or_skip

pytestmark = pytest.mark.gpu


def _decode_e4m3(b: np.ndarray) -> np.ndarray:
    """E4M3 (fn) bytes -> float64 values (written from the format's fields)."""
    b = np.asarray(b, dtype=np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.ldexp(1.0, e - 7))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return s * v


def _np_u8(t):
    return t.cpu().numpy()


def _quantize_gpu(q, k, v, dtype="bf16"):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    qq, qe = aa.mx8_quantize_qk(to_dev(q, dtype))
    kq, ke = aa.mx8_quantize_qk(to_dev(k, dtype))
    vt, vte = aa.mx8_quantize_v(to_dev(v, dtype))
    torch.cuda.synchronize()
    return qq, qe, kq, ke, vt, vte


def _check_quantizers(q, k, v, dtype, tensors):
    qq, qe, kq, ke, vt, vte = tensors
    for name, x, xq, xe in (("q", q, qq, qe), ("k", k, kq, ke)):
        rq, re_ = F.quantize_qk(to_f64(x, dtype))
        np.testing.assert_array_equal(_decode_e4m3(_np_u8(xq)), rq, err_msg=f"{name} codes")
        np.testing.assert_array_equal(_np_u8(xe).astype(np.int64) - 127, re_, err_msg=f"{name} exps")
    rvt, rvte = F.quantize_v_transposed(to_f64(v, dtype))
    np.testing.assert_array_equal(_decode_e4m3(_np_u8(vt)), rvt, err_msg="vt codes")
    # the kernel's exponent layout (B, H, Np/32, d) is the oracle's (B, H, d, Np/32) transposed
    np.testing.assert_array_equal(_np_u8(vte).astype(np.int64) - 127, rvte.transpose(0, 1, 3, 2),
                                  err_msg="vt exps")


def _check_attention(tensors, scale, causal, what, heads=None):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    qq, qe, kq, ke, vt, vte = tensors
    o, lse = aa.fa_fwd_mx8(qq, qe, kq, ke, vt, vte, softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy().astype(np.float64)
    lg = lse.cpu().numpy().astype(np.float64)
    Q = F.mx_dequantize(_decode_e4m3(_np_u8(qq)), _np_u8(qe).astype(np.int64) - 127)
    K = F.mx_dequantize(_decode_e4m3(_np_u8(kq)), _np_u8(ke).astype(np.int64) - 127)
    VT = F.mx_dequantize(_decode_e4m3(_np_u8(vt)),
                         (_np_u8(vte).astype(np.int64) - 127).transpose(0, 1, 3, 2))
    B, Nq, H, d = Q.shape
    Nk = K.shape[1]
    ratios = []
    pairs = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    for b, h in pairs:
        V = VT[b, h, :, :Nk].T
        Pm = attention_probs(Q[b, :, h], K[b, :, h], scale, causal)
        oref = Pm @ V
        S = scale * (Q[b, :, h] @ K[b, :, h].T)
        if causal:
            S = np.where(np.triu(np.ones((Nq, Nk), dtype=bool), 1), -np.inf, S)
        m = S.max(axis=1, keepdims=True)
        ell = np.exp(S - m).sum(axis=1)
        lref = m[:, 0] + np.log(ell)
        err = np.abs(og[b, :, h] - oref)
        bound = 2.0 ** -4 * (Pm @ np.abs(V)) + 2.0 ** -10 * np.abs(V).sum(0)[None, :] / ell[:, None] \
            + 2.0 ** -8 * np.abs(oref) + 1e-4
        bad = err > bound
        assert not bad.any(), (f"{what} b={b} h={h}: {int(bad.sum())} O elements beyond the bound; "
                               f"max err {err.max():.3e}")
        sigma2 = (2.0 ** -4) ** 2 * ((Pm ** 2) @ (V ** 2)) + (2.0 ** -9 * oref) ** 2 + 1e-8
        ratios.append(float(np.mean(err ** 2 / sigma2)))
        lerr = float(np.abs(lg[b, h] - lref).max())
        assert lerr <= L_ATOL, f"{what} b={b} h={h}: L max abs err {lerr}"
    r = float(np.mean(ratios))
    print(f"[mx8] {what}: mean err^2/sigma^2 = {r:.3f}", flush=True)
    assert r < 1.0, f"{what}: mean err^2/sigma^2 = {r}"


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 64, 65, 200, 333])
def test_mx8_small(causal, N):
    torch_or_skip()
    say(f"mx8 N={N} causal={causal}")
    q, k, v = W.make_dense(2, N, 2, 128, seed=13000 + N)
    t = _quantize_gpu(q, k, v)
    _check_quantizers(q, k, v, "bf16", t)
    _check_attention(t, 1 / np.sqrt(128), causal, f"N={N} causal={causal}")


def test_mx8_multi_tile_and_cross_lengths():
    torch_or_skip()
    say("mx8 Nq=700 Nk=1000, Nq=600 causal")
    q, _, _ = W.make_dense(1, 700, 2, 128, seed=13100)
    _, k, v = W.make_dense(1, 1000, 2, 128, seed=13101)
    t = _quantize_gpu(q, k, v)
    _check_attention(t, 1 / np.sqrt(128), False, "Nq=700 Nk=1000")
    q, k, v = W.make_dense(1, 600, 3, 128, seed=13102)
    _check_attention(_quantize_gpu(q, k, v), 1 / np.sqrt(128), True, "N=600 causal")


def test_mx8_negative_and_zero_scale():
    torch_or_skip()
    q, k, v = W.make_dense(1, 300, 2, 128, seed=13200)
    t = _quantize_gpu(q, k, v)
    _check_attention(t, -0.3, True, "scale -0.3 causal")
    _check_attention(t, 0.0, False, "scale 0")


def test_mx8_quantizers_edge_values_and_f16():
    """Blocks of zeros, a huge and a tiny block, values beyond E4M3's range
    within a block, and fp16 sources: the quantisers stay bit-exact."""
    torch_or_skip()
    rng = np.random.default_rng(13300)
    B, N, H, d = 1, 96, 2, 128
    x = rng.standard_normal((B, N, H, d)).astype(np.float32)
    x[0, 0, 0, :32] = 0.0                      # an all-zero block
    x[0, 1, 0] *= 3e4                          # large values (some beyond fp16: infinite there)
    x[0, 2, 1] *= 1e-6                         # tiny (subnormal quotients)
    x[0, 3, 0, 5] = 6e4                        # one dominant element per block
    x[0, 4, 1, 70] = np.inf                    # non-finite blocks: NaN scale, zero codes
    x[0, 5, 0, 100] = np.nan
    for dtype in ("bf16", "f16"):
        say(f"mx8 quantizer edges {dtype}")
        bits = W.f32_to_bf16_bits(x) if dtype == "bf16" else W.f32_to_f16_bits(x)
        t = _quantize_gpu(bits, bits, bits, dtype)
        _check_quantizers(bits, bits, bits, dtype, t)


def test_mx8_zero_q_closed_forms():
    """Closed forms through the whole path: with Q = 0 every visible score is 0,
    so P~ = 1 exactly in E4M3 and O is the plain mean of the visible rows of the
    dequantised V, L = ln(#visible keys); with constant V rows that mean is the
    row itself."""
    torch_or_skip()
    import aware_attention_amd as aa
    torch = torch_or_skip()
    N = 257
    _, k, vr = W.make_dense(1, N, 2, 128, seed=13400)
    z = np.zeros_like(k)
    vc = np.zeros((1, N, 2, 128), dtype=np.float32)
    vc[...] = 2.0 ** np.arange(-3, 5, 1 / 16)[:128]
    vc = W.f32_to_bf16_bits(vc)
    for causal in (False, True):
        for v in (vr, vc):
            say(f"mx8 zero q causal={causal}")
            o, lse = aa.attention_mx8(to_dev(z), to_dev(k), to_dev(v), causal=causal)
            torch.cuda.synchronize()
            V = F.mx_dequantize(*F.quantize_v_transposed(to_f64(v)))[..., :N].transpose(0, 3, 1, 2)
            cnt = np.arange(1, N + 1) if causal else np.full(N, N)
            csum = np.cumsum(V, axis=1) if causal else np.broadcast_to(V.sum(1, keepdims=True), V.shape)
            expect = csum / cnt[None, :, None, None]
            og = o.float().cpu().numpy()
            assert np.all(np.abs(og - expect) <= 2.0 ** -8 * np.abs(expect) + 1e-5), "O mean"
            assert np.abs(lse.cpu().numpy() - np.log(cnt)[None, None, :]).max() <= 1e-5, "L"


def test_mx8_full_size_prefill8k_sampled_heads():
    """The prefill8k shape (B1 H32 N8192 d128 causal) in the launch the benchmark
    times, with its quantisers bit-exact on every element and attention checked
    on four whole heads."""
    torch_or_skip()
    w = W.WORKLOADS["prefill8k"]
    say("mx8 full-size prefill8k")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed)
    t = _quantize_gpu(q, k, v)
    _check_quantizers(q, k, v, "bf16", t)
    _check_attention(t, w.scale, True, "prefill8k", heads=[(0, 0), (0, 7), (0, 18), (0, 31)])
