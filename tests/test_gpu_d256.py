"""Head dimension 256 (its own kernel): HIP path vs the float64 CPU oracle.

The oracle is the same definition; d is only a parameter there. Cases span
several 128-row query tiles and 64-key tiles with ragged tails, causal and
not, cross lengths, varlen, fp16, a packed QKV view (bitwise equal to the
contiguous call) and sampled rows of a full-size causal prefill at d = 256.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_dense, attention_varlen
from tests.gpu_util import (assert_l_close, assert_o_close, o_to_f64, say, to_dev, to_f64,
                            torch_or_skip)

pytestmark = pytest.mark.gpu


def check_256(B, Nq, Nk, H, causal, seed, dtype="bf16", scale=1 / 16.0):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say(f"d256 B={B} Nq={Nq} Nk={Nk} H={H} causal={causal} {dtype} seed={seed}")
    q, k, v = W.make_dense(B, Nq, H, 256, seed, Nk=Nk, dtype=dtype)
    o, lse = aa.fa_fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), causal=causal,
                       softmax_scale=scale)
    torch.cuda.synchronize()
    oref, lref = attention_dense(to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype),
                                 scale, causal)
    assert_o_close(o_to_f64(o), oref, f"d256 O Nq={Nq} Nk={Nk} causal={causal}")
    assert_l_close(lse.cpu().numpy().astype(np.float64), lref, f"d256 L Nq={Nq} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 63, 129, 300, 700])
def test_d256_dense(causal, N):
    check_256(2, N, N, 2, causal, seed=9500 + N)


@pytest.mark.parametrize("Nq,Nk", [(100, 333), (333, 1), (129, 64)])
def test_d256_cross_lengths(Nq, Nk):
    check_256(1, Nq, Nk, 2, False, seed=9550 + Nq + Nk)


@pytest.mark.parametrize("causal", [False, True])
def test_d256_f16(causal):
    check_256(2, 333, 333, 2, causal, seed=9580, dtype="f16")


@pytest.mark.parametrize("causal", [False, True])
def test_d256_varlen(causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [1, 127, 0, 128, 129, 300, 64, 65]
    say(f"d256 varlen lengths={lengths} causal={causal}")
    q, k, v, cu = W.make_varlen(lengths, 2, 256, seed=9600)
    o, lse = aa.fa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).cuda(),
                              max(lengths), causal=causal)
    torch.cuda.synchronize()
    oref, lref = attention_varlen(to_f64(q), to_f64(k), to_f64(v), cu, 1 / 16.0, causal)
    assert_o_close(o_to_f64(o), oref, "d256 varlen O")
    assert_l_close(lse.cpu().numpy().astype(np.float64), lref, "d256 varlen L")


def test_d256_packed_qkv_bitwise():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("d256 packed qkv")
    bits = np.stack(W.make_dense(2, 300, 2, 256, seed=9650), axis=2)   # (B, S, 3, H, d)
    q, k, v = to_dev(bits).unbind(2)
    o, lse = aa.fa_fwd(q, k, v, causal=True)
    oc, lc = aa.fa_fwd(q.contiguous(), k.contiguous(), v.contiguous(), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), oc.view(torch.int16)) and torch.equal(lse, lc)


def test_d256_full_size_sampled():
    """prefill8k_d256 (B=1 H=16 N=8192 d=256 causal): sampled rows of sampled heads."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS["prefill8k_d256"]
    say(f"d256 full size B={w.B} N={w.N} H={w.H}")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed)
    o, lse = aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 100)
    for h in sorted({0, w.H - 1, int(rng.integers(w.H))}):
        rows = sorted({0, 1, 127, 128, w.N - 1} | set(rng.integers(0, w.N, size=40).tolist()))
        oref, lref = attention_dense(to_f64(q[:, :, h:h + 1]), to_f64(k[:, :, h:h + 1]),
                                     to_f64(v[:, :, h:h + 1]), w.scale, True, rows=rows)
        assert_o_close(o_to_f64(o[0, rows, h]), oref[0, :, 0], f"d256 full h={h}")
        assert_l_close(lse[0, h, rows].cpu().numpy().astype(np.float64), lref[0, 0],
                       f"d256 full h={h}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


# ---------------------------------------------------------------------------
# Banded mask and key padding mask at head dimension 256
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("window", [(None, 0), (0, 0), (16, 16), (100, 3), (0, None),
                                    (63, 64), (None, None), (5, 200)])
@pytest.mark.parametrize("Nq,Nk", [(333, 333), (129, 700), (700, 129)])
def test_d256_band(window, Nq, Nk):
    # (700, 129): off = -571, so with a bounded right side the first rows see no key.
    from tests.test_gpu_band import check_band
    check_band(2 if Nq == Nk else 1, Nq, Nk, 2, 256, window, seed=13000 + Nq + 3 * Nk)


def test_d256_band_long_rows():
    from tests.test_gpu_band import check_band
    check_band(1, 1500, 1500, 2, 256, (700, 100), seed=13100)


@pytest.mark.parametrize("window", [(None, 0), (7, 7), (0, 0), (200, None)])
def test_d256_band_varlen(window):
    import aware_attention_amd as aa
    from tests.test_gpu_band import assert_l_band
    torch = torch_or_skip()
    lengths = [1, 127, 0, 128, 129, 300, 64]
    say(f"d256 varlen band lengths={lengths} window={window}")
    q, k, v, cu = W.make_varlen(lengths, 2, 256, seed=13200)
    scale = 1 / 16.0
    o, lse = aa.fa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).cuda(),
                              max(lengths), softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    oref, lref = attention_varlen(to_f64(q), to_f64(k), to_f64(v), cu, scale, window=window)
    assert_o_close(o_to_f64(o), oref, f"d256 varlen window={window} O")
    assert_l_band(lse.cpu().numpy().astype(np.float64), lref, f"d256 varlen window={window} L")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 65, 333])
def test_d256_padded(causal, S):
    # Five mask kinds (right padding, scattered holes, all valid, all padding,
    # a middle run), one per batch row.
    from tests.test_gpu_padded import check_padded
    check_padded(5, S, 2, 256, causal, seed=13300 + S)


@pytest.mark.parametrize("causal", [False, True])
def test_d256_padded_long_rows_with_empty_tiles(causal):
    from tests.test_gpu_padded import check_padded
    B, S = 3, 1100
    m = np.ones((B, S), dtype=np.uint8)
    m[0, :300] = 0
    m[1, 600:] = 0
    m[2, ::3] = 0
    check_padded(B, S, 2, 256, causal, seed=13400, mask=m)


def test_d256_padded_f16():
    from tests.test_gpu_padded import check_padded
    check_padded(5, 300, 2, 256, True, seed=13500, dtype="f16")


def test_d256_full_size_band_sampled():
    """band8k_d256 (B=1 H=16 N=8192 d=256, band (2047, 0)), in the launch bench.py
    times: sampled rows (band edges, tile edges, random) of sampled heads, and
    every output finite and inside the range of V."""
    import aware_attention_amd as aa
    from tests.test_gpu_band import assert_l_band
    torch = torch_or_skip()
    w = W.WORKLOADS["band8k_d256"]
    say(f"full-size band8k_d256 B={w.B} N={w.N} H={w.H} d={w.d} window={w.window}")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o, lse = aa.fa_fwd(qd, kd, vd, softmax_scale=w.scale, window=w.window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 100)
    fixed = {0, 1, 63, 64, 127, 128, 2046, 2047, 2048, 2049, w.N // 2, w.N - 2, w.N - 1}
    for h in sorted({0, w.H - 1} | {int(rng.integers(w.H)) for _ in range(2)}):
        rows = sorted(fixed | set(rng.integers(0, w.N, size=40).tolist()))
        oref, lref = attention_dense(to_f64(q[:, :, h:h + 1]), to_f64(k[:, :, h:h + 1]),
                                     to_f64(v[:, :, h:h + 1]), w.scale, rows=rows,
                                     window=w.window)
        assert_o_close(o_to_f64(o[0, rows, h]), oref[0, :, 0], f"band8k_d256 h={h}")
        assert_l_band(lse[0, h, rows].cpu().numpy().astype(np.float64), lref[0, 0],
                      f"band8k_d256 h={h}")
    vmin = vd.float().amin(dim=1, keepdim=True)
    vmax = vd.float().amax(dim=1, keepdim=True)
    of = o.float()
    slack = 1e-2 * (vmax - vmin) + 1e-3
    assert torch.isfinite(of).all() and torch.isfinite(lse).all()
    assert bool(((of >= vmin - slack) & (of <= vmax + slack)).all())
