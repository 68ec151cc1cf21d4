"""Key padding mask (fa_fwd_padded): HIP path vs the float64 CPU oracle.

The oracle removes the padding positions, attends over the valid tokens and
puts the result back (zeros at padding, L = -inf there). The kernel works in
the padded layout and masks padding keys per 64-key tile. Masks cover right
padding, scattered holes, an all-padding row, all-valid rows, and padding
that leaves whole key tiles empty.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_padded, attention_varlen
from tests.gpu_util import (L_ATOL, assert_o_close, o_to_f64, say, to_dev, to_f64,
                            torch_or_skip)

pytestmark = pytest.mark.gpu


def _masks(B, S, seed):
    rng = np.random.default_rng(seed)
    m = np.zeros((B, S), dtype=np.uint8)
    for b in range(B):
        kind = b % 5
        if kind == 0:                                   # right padding
            m[b, :int(rng.integers(1, S + 1))] = 1
        elif kind == 1:                                 # scattered holes
            m[b] = rng.random(S) < 0.7
        elif kind == 2:                                 # all valid
            m[b] = 1
        elif kind == 3:                                 # all padding
            pass
        else:                                           # a valid run in the middle
            a = int(rng.integers(0, S))
            m[b, a:a + int(rng.integers(1, S - a + 1))] = 1
    return m


def run_padded(q, k, v, mask, scale, causal, dtype="bf16"):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    o, lse = aa.fa_fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), softmax_scale=scale,
                       causal=causal, key_padding_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def check_padded(B, S, H, d, causal, seed, dtype="bf16", mask=None, scale=None):
    torch_or_skip()
    say(f"padded B={B} S={S} H={H} d={d} causal={causal} dtype={dtype} seed={seed}")
    q, k, v = W.make_dense(B, S, H, d, seed, dtype=dtype)
    mask = _masks(B, S, seed) if mask is None else mask
    scale = 1 / np.sqrt(d) if scale is None else scale
    og, lg = run_padded(q, k, v, mask, scale, causal, dtype)
    oref, lref = attention_padded(to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype), mask,
                                  scale, causal)
    what = f"S={S} d={d} causal={causal} {dtype}"
    assert_o_close(og, oref, "O " + what)
    pad = np.isneginf(lref)
    assert np.all(np.isneginf(lg[pad])), "L must be -inf at padding positions"
    assert np.all(og.transpose(0, 2, 1, 3)[pad] == 0), "O must be 0 at padding positions"
    if (~pad).any():
        err = float(np.abs(lg[~pad] - lref[~pad]).max())
        assert err <= L_ATOL, f"L {what}: max abs err {err}"


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("S", [1, 65, 333])
def test_padded(d, causal, S):
    check_padded(5, S, 2, d, causal, seed=9000 + S + d)


@pytest.mark.parametrize("causal", [False, True])
def test_padded_f16(causal):
    check_padded(5, 300, 2, 128, causal, seed=9100, dtype="f16")


@pytest.mark.parametrize("causal", [False, True])
def test_padded_long_rows_with_empty_tiles(causal):
    # 1100 tokens: the first 300 and the last 500 are padding in two rows, so
    # whole 64-key tiles (and whole 256-query tiles) hold no valid token.
    B, S = 3, 1100
    m = np.ones((B, S), dtype=np.uint8)
    m[0, :300] = 0
    m[1, 600:] = 0
    m[2, ::3] = 0
    check_padded(B, S, 2, 128, causal, seed=9200, mask=m)


def test_padded_right_padding_matches_varlen_kernel():
    """Right padding through fa_fwd_padded equals the packed varlen kernel on the
    same tokens (both HIP, same per-row arithmetic up to the tile order)."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, S, H, d = 4, 700, 2, 128
    lengths = [700, 1, 300, 513]
    say(f"padded vs varlen lengths={lengths}")
    q, k, v = W.make_dense(B, S, H, d, seed=9300)
    m = np.array([[1] * n + [0] * (S - n) for n in lengths], dtype=np.uint8)
    og, lg = run_padded(q, k, v, m, 1 / np.sqrt(d), False)
    pack = lambda x: np.concatenate([x[b, :n] for b, n in enumerate(lengths)])  # noqa: E731
    cu = W.cu_seqlens_from_lengths(lengths)
    ov, lv = aa.fa_fwd_varlen(to_dev(pack(q)), to_dev(pack(k)), to_dev(pack(v)),
                              torch.from_numpy(cu).cuda(), max(lengths))
    torch.cuda.synchronize()
    oref, lref = attention_varlen(to_f64(pack(q)), to_f64(pack(k)), to_f64(pack(v)), cu,
                                  1 / np.sqrt(d))
    for b, n in enumerate(lengths):
        a = int(cu[b])
        assert_o_close(og[b, :n], o_to_f64(ov[a:a + n]), f"padded vs varlen b={b}")
        assert np.abs(lg[b, :, :n] - lv[:, a:a + n].cpu().numpy()).max() <= L_ATOL
        assert_o_close(og[b, :n], oref[a:a + n], f"padded vs oracle b={b}")


def test_padded_full_size_vit_sampled():
    """The ViT batch shape (B=32, S=1025, H=25, d=128, Q and K RMS-normalised)
    with right padding to lengths drawn like the varlen workload; sampled rows."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS["vit"]
    lengths = W.varlen_lengths(w.B, 256, 1025, seed=w.seed + 7)
    say(f"padded full-size vit lengths min={lengths.min()} max={lengths.max()}")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed, rms_qk=True)
    m = np.array([[1] * int(n) + [0] * (w.N - int(n)) for n in lengths], dtype=np.uint8)
    o, lse = aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), key_padding_mask=torch.from_numpy(m).cuda())
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 300)
    for b in sorted({0, w.B - 1} | set(rng.integers(0, w.B, size=3).tolist())):
        n = int(lengths[b])
        for h in (0, w.H - 1):
            sub = lambda x: to_f64(x[b:b + 1, :, h:h + 1])  # noqa: E731
            oref, lref = attention_padded(sub(q), sub(k), sub(v), m[b:b + 1], w.scale)
            assert_o_close(o_to_f64(o[b:b + 1, :, h:h + 1]), oref, f"vit padded b={b} h={h}")
            lg = lse[b, h].cpu().numpy().astype(np.float64)
            assert np.abs(lg[:n] - lref[0, 0, :n]).max() <= L_ATOL
            assert np.all(np.isneginf(lg[n:]))
