"""The online-softmax offset moving in the middle of a sequence, on the GPU.

The forward kernels exponentiate a steady tile against the current offset
and only take the row maximum and the rescale of the output accumulator
("FlashAttention/zh" (marovi.ai wiki), section FlashAttention 算法: the
running maximum and the rescaling of O and l) when a lane's sum of P~ for
the tile exceeds 2^8. With N(0,1) inputs that never happens after a row's
first tile, so these cases scale the key rows up along the sequence: the
row maxima keep growing, and later tiles exceed the running maximum by more
than 8 (base 2) on many rows. Each case first checks on the CPU that its
inputs do that in tiles the kernels run in their steady loops, then compares
the GPU result with the float64 oracle: dense, causal, bands, key padding
masks, varlen, head dimension 256 and the FP8 path.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads as W
from oracle import attention_dense, attention_padded, attention_varlen
from tests.gpu_util import (L_ATOL, assert_l_close, assert_o_close, o_to_f64, say, to_dev,
                            to_f64, torch_or_skip)

pytestmark = pytest.mark.gpu

BC = 64   # keys per tile of the kernels


def ramp_keys(k_bits: np.ndarray, growth: float, axis: int = 1) -> np.ndarray:
    """Key rows scaled by 1 + growth * j / N along the token axis, rounded to bf16."""
    k = W.bf16_bits_to_f32(k_bits)
    n = k.shape[axis]
    shape = [1] * k.ndim
    shape[axis] = n
    f = (1.0 + growth * np.arange(n, dtype=np.float32) / n).reshape(shape)
    return W.f32_to_bf16_bits(k * f)


def late_jumps(q: np.ndarray, k: np.ndarray, scale: float, causal: bool, left=None,
               steady_only: bool = False) -> int:
    """Rows x tiles (from tile 2 on) whose tile maximum exceeds the running
    maximum of all earlier tiles by more than 8 in base 2: a sufficient
    condition for the kernels' full path with a rescale. q (Nq, d), k (Nk, d)
    as float64 (self-attention); left bounds a band's reach to the left.
    steady_only counts only tiles of the d <= 128 kernel's steady loop (for a
    row in the 256-row query tile starting at q0: tiles left of the tile's
    diagonal block when causal, else all but the last full tile)."""
    s = (q @ k.T) * scale * np.log2(np.e)
    Nq, Nk = s.shape
    i, j = np.arange(Nq)[:, None], np.arange(Nk)[None, :]
    hide = np.zeros((Nq, Nk), dtype=bool)
    if causal:
        hide |= j > i
    if left is not None:
        hide |= j < i - left
    s = np.where(hide, -np.inf, s)
    n_t = (Nk + BC - 1) // BC
    tmax = np.stack([s[:, t * BC:(t + 1) * BC].max(axis=1) for t in range(n_t)], axis=1)
    run = np.maximum.accumulate(tmax, axis=1)
    jumps = np.zeros_like(tmax, dtype=bool)
    jumps[:, 2:] = tmax[:, 2:] > run[:, 1:-1] + 8.0
    if steady_only:
        q0 = (np.arange(Nq) // 256) * 256
        end = q0 // BC if causal else np.full(Nq, Nk // BC - 1)
        jumps &= np.arange(n_t)[None, :] < end[:, None]
    return int(jumps.sum())


def _dense_case(B, N, H, d, seed, growth):
    q, k, v = W.make_dense(B, N, H, d, seed)
    return q, ramp_keys(k, growth), v


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_offset_moves_in_steady_tiles(d, causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    N, H, scale = 1100, 2, 1.0 / np.sqrt(d)
    q, k, v = _dense_case(1, N, H, d, 31000 + d + int(causal), growth=7.0)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    jumps = sum(late_jumps(qf[0, :, h], kf[0, :, h], scale, causal, steady_only=d <= 128)
                for h in range(H))
    assert jumps >= 50, f"inputs move the offset in only {jumps} (row, tile) pairs"
    say(f"rescale dense d={d} causal={causal} N={N} late jumps={jumps}")
    o, lse = aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    oref, lref = attention_dense(qf, kf, vf, scale, causal)
    what = f"rescale d={d} causal={causal}"
    assert_o_close(o_to_f64(o), oref, what + " O")
    assert_l_close(lse.cpu().numpy().astype(np.float64), lref, what + " L")


@pytest.mark.parametrize("d", [128, 256])
def test_offset_moves_in_band(d):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    N, H, scale, window = 1100, 2, 1.0 / np.sqrt(d), (300, 0)
    q, k, v = _dense_case(1, N, H, d, 31100 + d, growth=7.0)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    assert sum(late_jumps(qf[0, :, h], kf[0, :, h], scale, True, left=window[0])
               for h in range(H)) >= 50
    say(f"rescale band d={d} window={window}")
    o, lse = aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    oref, lref = attention_dense(qf, kf, vf, scale, window=window)
    assert_o_close(o_to_f64(o), oref, f"rescale band d={d} O")
    assert_l_close(lse.cpu().numpy().astype(np.float64), lref, f"rescale band d={d} L")


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_offset_moves_with_padding_mask(d, causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, S, H, scale = 2, 1100, 2, 1.0 / np.sqrt(d)
    q, k, v = _dense_case(B, S, H, d, 31200 + d + int(causal), growth=7.0)
    mask = np.zeros((B, S), dtype=np.uint8)
    mask[0, :1000] = 1          # right padding: one run of valid tokens (steady tiles)
    mask[1, :] = 1
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    assert late_jumps(qf[0, :1000, 0], kf[0, :1000, 0], scale, causal, steady_only=d <= 128) >= 25
    say(f"rescale padded d={d} causal={causal}")
    o, lse = aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), softmax_scale=scale, causal=causal,
                       key_padding_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    oref, lref = attention_padded(qf, kf, vf, mask, scale, causal)
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    assert_o_close(og, oref, f"rescale padded d={d} O")
    pad = np.isneginf(lref)
    assert np.all(np.isneginf(lg[pad])) and np.all(og.transpose(0, 2, 1, 3)[pad] == 0)
    err = float(np.abs(lg[~pad] - lref[~pad]).max())
    assert err <= L_ATOL, f"rescale padded d={d}: L max abs err {err}"


@pytest.mark.parametrize("causal", [False, True])
def test_offset_moves_varlen(causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = np.array([1100, 5, 700, 0, 1025, 129], dtype=np.int64)
    H, d, scale = 2, 128, 1.0 / np.sqrt(128)
    q, k, v, cu = W.make_varlen(lengths, H, d, seed=31300 + int(causal))
    kf32 = W.bf16_bits_to_f32(k)
    for i in range(len(lengths)):   # each sequence's keys grow along that sequence
        a, b = int(cu[i]), int(cu[i + 1])
        kf32[a:b] *= (1.0 + 7.0 * np.arange(b - a, dtype=np.float32) / max(b - a, 1))[:, None, None]
    k = W.f32_to_bf16_bits(kf32)
    qf, kf, vf = to_f64(q), to_f64(k), to_f64(v)
    assert late_jumps(qf[:1100, 0], kf[:1100, 0], scale, causal, steady_only=True) >= 25
    say(f"rescale varlen causal={causal}")
    o, lse = aa.fa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).cuda(),
                              int(lengths.max()), softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    oref, lref = attention_varlen(qf, kf, vf, cu, scale, causal)
    assert_o_close(o_to_f64(o), oref, f"rescale varlen causal={causal} O")
    assert_l_close(lse.cpu().numpy().astype(np.float64), lref, f"rescale varlen causal={causal} L")


@pytest.mark.parametrize("causal", [False, True])
def test_offset_moves_fp8(causal):
    from tests.test_gpu_mx8 import _check_attention, _quantize_gpu
    torch_or_skip()
    N, scale = 1000, 1.0 / np.sqrt(128)
    q, k, v = _dense_case(1, N, 2, 128, 31400 + int(causal), growth=7.0)
    qf, kf = to_f64(q), to_f64(k)
    assert late_jumps(qf[0, :, 0], kf[0, :, 0], scale, causal, steady_only=True) >= 25
    say(f"rescale fp8 causal={causal}")
    _check_attention(_quantize_gpu(q, k, v), scale, causal, f"rescale fp8 causal={causal}")
