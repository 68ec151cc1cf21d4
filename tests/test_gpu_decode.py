"""Split-KV decode (fa_decode): HIP path vs the float64 CPU oracle.

One query per (batch, head) against a cache of Nk keys, of which batch b
uses its first len_b. The oracle is the plain definition on those keys (a
batch with no key: O = 0, L = -inf). Cases cover every head dimension, cache
lengths around the 64-key and chunk boundaries, per-batch lengths including
0, fp16, a 100k-key cache (many chunks) and the split plan's extremes.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention
from tests.gpu_util import (L_ATOL, assert_o_close, o_to_f64, say, to_dev, to_f64,
                            torch_or_skip)

pytestmark = pytest.mark.gpu


def check_decode(B, Nk, H, d, seed, lens=None, dtype="bf16", scale=None):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say(f"decode B={B} Nk={Nk} H={H} d={d} lens={lens} {dtype} seed={seed}")
    q = W.make_dense(B, 1, H, d, seed, dtype=dtype)[0]
    _, k, v = W.make_dense(B, Nk, H, d, seed + 1, dtype=dtype)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32).cuda()
    scale = 1 / np.sqrt(d) if scale is None else scale
    o, lse = aa.fa_decode(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), seqlens_k=sl,
                          softmax_scale=scale)
    torch.cuda.synchronize()
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    qf, kf, vf = to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype)
    for b in range(B):
        n = Nk if lens is None else max(0, min(lens[b], Nk))
        for h in range(H):
            if n == 0:
                assert np.all(og[b, 0, h] == 0) and np.isneginf(lg[b, h]), f"empty cache b={b}"
                continue
            oref, lref = attention(qf[b, :, h], kf[b, :n, h], vf[b, :n, h], scale)
            assert_o_close(og[b, 0, h][None], oref, f"decode O b={b} h={h} n={n}")
            assert abs(lg[b, h] - lref[0]) <= L_ATOL, f"decode L b={b} h={h}: {lg[b, h]} vs {lref[0]}"


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("Nk", [1, 63, 65, 1000, 5000])
def test_decode(d, Nk):
    check_decode(3, Nk, 4, d, seed=9700 + Nk + d)


@pytest.mark.parametrize("d", [64, 128])
def test_decode_per_batch_lengths(d):
    check_decode(5, 3000, 2, d, seed=9800 + d, lens=[0, 1, 3000, 1500, 4000])


def test_decode_f16():
    check_decode(2, 2000, 4, 128, seed=9850, dtype="f16", lens=[2000, 777])


def test_decode_long_cache_many_chunks():
    # 100k keys in one head: chunks of at most 4096 keys, merged through L.
    check_decode(1, 100000, 2, 128, seed=9900)


def test_decode_many_heads_one_chunk():
    # 64 x 32 heads already fill the chip: one chunk per head.
    check_decode(64, 300, 32, 64, seed=9950)


def test_decode_matches_forward_and_is_deterministic():
    """The decode and the forward kernel with one query row agree to the
    forward's bar, and repeated decodes are bitwise equal."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("decode vs forward, determinism")
    q = to_dev(W.make_dense(2, 1, 8, 128, seed=9960)[0])
    _, k, v = (to_dev(x) for x in W.make_dense(2, 4000, 8, 128, seed=9961))
    o1, l1 = aa.fa_decode(q, k, v)
    o2, l2 = aa.fa_decode(q, k, v)
    of, lf = aa.fa_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    assert_o_close(o_to_f64(o1), o_to_f64(of), "decode vs forward")
    assert float((l1 - lf[:, :, 0]).abs().max()) <= L_ATOL


@pytest.mark.parametrize("name", ["decode8k", "decode32k"])
def test_decode_full_size_workloads(name):
    """decode8k / decode32k in the launch bench.py times (caller workspace,
    preallocated outputs): every (batch, head) against the oracle."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS[name]
    say(f"decode full-size {name} B={w.B} Nk={w.Nk} H={w.H} d={w.d}")
    wl = W.make_workload(name)
    q, k, v = (to_dev(x) for x in (wl["q"], wl["k"], wl["v"]))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(aa._lib.decode_workspace_bytes(w.B, w.Nk, w.H, w.d), dtype=torch.uint8,
                     device="cuda")
    aa.fa_decode(q, k, v, softmax_scale=w.scale, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    qf, kf, vf = to_f64(wl["q"]), to_f64(wl["k"]), to_f64(wl["v"])
    for b in range(w.B):
        for h in range(w.H):
            oref, lref = attention(qf[b, :, h], kf[b, :, h], vf[b, :, h], w.scale)
            assert_o_close(og[b, 0, h][None], oref, f"{name} O b={b} h={h}")
            assert abs(lg[b, h] - lref[0]) <= L_ATOL, f"{name} L b={b} h={h}"
