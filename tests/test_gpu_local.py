"""Local window on a token map plus global anchors (fa_fwd_local): HIP path vs
the float64 CPU oracle (oracle/local.py), element by element.

Cases: the detector map (8 anchors + 40 x 40 tokens, 5 x 5 window) at every
head dimension; patterns that reduce to a band (one-wide or one-row maps),
to plain attention (a window wider than the map, every token an anchor) and
to the diagonal; many anchors spanning several key tiles; short maps whose
last row is partial; lengths around the 64-key and 128-query tiles; causal;
fp16. Cross-checks against the banded and plain forward entry points, and
determinism.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_local_dense
from tests.gpu_util import (L_ATOL, assert_o_close, o_to_f64, say, to_dev, to_f64,
                            torch_or_skip)

pytestmark = pytest.mark.gpu


def run_local(q, k, v, G, Wd, win, causal, dtype="bf16", scale=None):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    o, lse = aa.fa_fwd_local(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), G, Wd, win,
                             softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def check_local(B, N, H, d, G, Wd, win, causal, seed, dtype="bf16", scale=None):
    say(f"local B={B} N={N} H={H} d={d} G={G} map_w={Wd} win={win} causal={causal} {dtype} "
        f"seed={seed}")
    q, k, v = W.make_dense(B, N, H, d, seed, dtype=dtype)
    scale = 1 / np.sqrt(d) if scale is None else scale
    og, lg = run_local(q, k, v, G, Wd, win, causal, dtype, scale)
    qf, kf, vf = to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype)
    oref, lref = attention_local_dense(qf, kf, vf, scale, G, Wd, win[0], win[1], causal)
    what = f"G={G} map_w={Wd} win={win} causal={causal} N={N} d={d}"
    assert_o_close(og, oref, "local O " + what)
    err = np.max(np.abs(lg - lref))
    assert err <= L_ATOL, f"local L {what}: max err {err}"


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_local_detector_map(d, causal):
    # 8 anchors + a 40 x 40 map, 5 x 5 window (the page's example).
    check_local(2, 8 + 1600, 2, d, 8, 40, (2, 2), causal, seed=12000 + d + causal)


@pytest.mark.parametrize("G,Wd,win", [
    (0, 40, (2, 2)),        # no anchors
    (1, 7, (1, 3)),         # short rows, wide columns
    (70, 13, (0, 0)),       # anchors over two key tiles, diagonal window
    (200, 1, (5, 0)),       # one-wide map: a band of the token order
    (0, 1000, (0, 64)),     # one row: a band of +-64
    (5, 33, (100, 100)),    # the window covers the map: plain attention
    (3, 17, (3, 1)),        # partial last map row
])
@pytest.mark.parametrize("causal", [False, True])
def test_local_patterns(G, Wd, win, causal):
    check_local(1, 777, 2, 64, G, Wd, win, causal, seed=12100 + G + Wd)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 127, 128, 129, 300])
def test_local_lengths(N):
    check_local(2, N, 2, 128, min(3, N), 9, (1, 2), N % 2 == 1, seed=12200 + N)


def test_local_all_anchors():
    check_local(1, 300, 2, 64, 300, 5, (0, 0), False, seed=12300)
    check_local(1, 300, 2, 64, 5000, 5, (0, 0), True, seed=12301)


def test_local_f16():
    check_local(2, 8 + 1600, 2, 128, 8, 40, (2, 2), False, seed=12400, dtype="f16")


def test_local_many_heads_and_batches():
    check_local(3, 8 + 400, 5, 32, 8, 20, (2, 2), False, seed=12500)


def test_local_agrees_with_band_and_plain_entry_points():
    """A one-wide map without anchors is the band (w, w) (causal: (w, 0)); a
    window over the whole map is plain attention: the other forward entry
    points give the same result to the forward's bar."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("local vs band and plain forward")
    q, k, v = (to_dev(x) for x in W.make_dense(2, 700, 2, 128, seed=12600))
    o1, l1 = aa.fa_fwd_local(q, k, v, 0, 1, (9, 0))
    o2, l2 = aa.fa_fwd(q, k, v, window=(9, 9))
    o3, l3 = aa.fa_fwd_local(q, k, v, 0, 1, (9, 0), causal=True)
    o4, l4 = aa.fa_fwd(q, k, v, window=(9, 0))
    o5, l5 = aa.fa_fwd_local(q, k, v, 4, 25, (1000, 1000))
    o6, l6 = aa.fa_fwd(q, k, v)
    torch.cuda.synchronize()
    for a, b_, la, lb, n in ((o1, o2, l1, l2, "band"), (o3, o4, l3, l4, "causal band"),
                             (o5, o6, l5, l6, "plain")):
        assert_o_close(o_to_f64(a), o_to_f64(b_), "local vs " + n)
        assert float((la - lb).abs().max()) <= L_ATOL, "L local vs " + n


def test_local_deterministic():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("local determinism")
    q, k, v = (to_dev(x) for x in W.make_dense(2, 1608, 4, 32, seed=12700))
    o1, l1 = aa.fa_fwd_local(q, k, v, 8, 40, (2, 2))
    o2, l2 = aa.fa_fwd_local(q, k, v, 8, 40, (2, 2))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_local_full_size_detlocal():
    """detlocal (B=16 H=4, 8 anchors + 40 x 40 map, 5 x 5 window, d=32) in the
    launch bench.py times, every output of 16 (batch, head) pairs against the
    oracle and the rest finite."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS["detlocal"]
    G, Wd, wr, wc = w.local
    say(f"full-size detlocal B={w.B} N={w.N} H={w.H} d={w.d} local={w.local}")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed)
    o, lse = aa.fa_fwd_local(to_dev(q), to_dev(k), to_dev(v), G, Wd, (wr, wc),
                             softmax_scale=w.scale)
    torch.cuda.synchronize()
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    batches = [0, 5, 10, 15]
    oref, lref = attention_local_dense(to_f64(q), to_f64(k), to_f64(v), w.scale, G, Wd, wr, wc,
                                       batches=batches)
    assert_o_close(og[batches], oref, "detlocal O")
    assert float(np.max(np.abs(lg[batches] - lref))) <= L_ATOL, "detlocal L"
    assert np.isfinite(og).all() and np.isfinite(lg).all()
