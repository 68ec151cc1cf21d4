"""Banded (sliding-window) mask: HIP path vs the float64 CPU oracle.

Query i sees key j iff i + off - left <= j <= i + off + right, with off =
Nk - Nq for an equal-length batch and 0 inside a packed sequence; a side of
None is unbounded. Rows that see no key must come out as O = 0 and L = -inf,
as in the oracle. Small cases compare every output and span several query
and key tiles with ragged tails; wide bands on longer rows reach the
kernel's loop over tiles that every row sees in full; the full-size banded
prefill compares sampled rows.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_dense, attention_varlen
from tests.gpu_util import (L_ATOL, assert_o_close, o_to_f64, say, to_dev, to_f64,
                            torch_or_skip)

pytestmark = pytest.mark.gpu


def assert_l_band(lg: np.ndarray, lref: np.ndarray, what: str = ""):
    """L within L_ATOL on rows that see a key; exactly -inf on rows that see none."""
    assert lg.shape == lref.shape, (lg.shape, lref.shape)
    empty = np.isneginf(lref)
    assert np.all(np.isneginf(lg[empty])), f"{what}: a row with no visible key must give L = -inf"
    seen = ~empty
    assert np.all(np.isfinite(lg[seen])), f"{what}: non-finite L on a row that sees keys"
    err = float(np.abs(lg[seen] - lref[seen]).max()) if seen.any() else 0.0
    assert err <= L_ATOL, f"{what}: L max abs err {err} > {L_ATOL}"


def assert_empty_rows_zero(og: np.ndarray, lref: np.ndarray, what: str = ""):
    """O is exactly 0 on rows that see no key. og (B, Nq, H, d), lref (B, H, Nq)."""
    empty = np.isneginf(lref).transpose(0, 2, 1)            # (B, Nq, H)
    assert np.all(og[empty] == 0.0), f"{what}: O must be 0 on rows that see no key"


def run_band(q, k, v, scale, window):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    o, lse = aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def check_band(B, Nq, Nk, H, d, window, seed, scale=None):
    torch_or_skip()
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    say(f"band B={B} Nq={Nq} Nk={Nk} H={H} d={d} window={window} seed={seed}")
    q, k, v = W.make_dense(B, Nq, H, d, seed, Nk=Nk)
    og, lg = run_band(q, k, v, scale, window)
    oref, lref = attention_dense(to_f64(q), to_f64(k), to_f64(v), scale, window=window)
    what = f"window={window} Nq={Nq} Nk={Nk} d={d}"
    assert_o_close(og, oref, what + " O")
    assert_l_band(lg, lref, what + " L")
    assert_empty_rows_zero(og, lref, what)


WINDOWS = [(None, 0), (0, 0), (16, 16), (100, 3), (0, None), (300, None), (63, 64),
           (None, None), (5, 200), (1000, 1000)]


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("window", WINDOWS)
@pytest.mark.parametrize("Nq,Nk", [(333, 333), (129, 700), (700, 129)])
def test_band_small(d, window, Nq, Nk):
    # (700, 129): off = -571, so with a bounded right side the first rows see
    # no key at all.
    check_band(2 if Nq == Nk else 1, Nq, Nk, 2, d, window, seed=6000 + Nq + 3 * Nk + d)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [(None, 0), (512, 512), (1500, 0), (0, 1500), (255, 255),
                                    (700, 100)])
def test_band_long_rows(d, window):
    # 8 query tiles of 256 rows and 32 key tiles: bands much wider than a
    # query tile leave runs of key tiles that every row of a tile sees in full.
    check_band(1, 2000, 2000, 2, d, window, seed=6100 + d)


@pytest.mark.parametrize("window", [(700, 100), (None, 40), (64, None)])
def test_band_cross_lengths_long(window):
    check_band(1, 1500, 2600, 2, 128, window, seed=6150)


def test_band_single_rows_and_keys():
    for Nq, Nk in [(1, 1), (1, 517), (517, 1), (2, 3)]:
        for window in [(0, 0), (None, 0), (3, None)]:
            check_band(1, Nq, Nk, 2, 64, window, seed=6170 + Nq + Nk)


@pytest.mark.parametrize("d", [32, 128])
@pytest.mark.parametrize("window", [(64, 64), (None, 0), (0, None)])
def test_band_tile_order(d, window):
    # 2 batches x 4 heads = 8 units, 12 query tiles each: banded launches
    # dispatch the query tiles with the most key tiles first (middle-out for
    # a two-sided band, descending / ascending for one-sided ones).
    check_band(2, 3000, 3000, 4, d, window, seed=6200 + d)


def test_band_zero_query_closed_form():
    # Q = 0: every visible score is 0, so O is the mean of the visible V rows
    # and L = ln(number of visible keys); rows that see nothing give 0, -inf.
    torch_or_skip()
    Nq, Nk, H, d, (left, right) = 400, 300, 2, 128, (20, 5)
    say(f"band zero-Q closed form Nq={Nq} Nk={Nk} window={(left, right)}")
    _, k, v = W.make_dense(1, Nk, H, d, seed=6300)
    q = np.zeros((1, Nq, H, d), dtype=k.dtype)
    og, lg = run_band(q, k, v, 0.09, (left, right))
    vf = to_f64(v)[0]
    oexp = np.zeros((Nq, H, d))
    lexp = np.full((H, Nq), -np.inf)
    for i in range(Nq):
        lo, hi = max(0, i + Nk - Nq - left), min(Nk - 1, i + Nk - Nq + right)
        if hi >= lo:
            oexp[i] = vf[lo:hi + 1].mean(axis=0)
            lexp[:, i] = np.log(hi - lo + 1)
    assert_o_close(og[0], oexp, "O = mean of visible V")
    assert_l_band(lg[0], lexp, "L = ln(#visible)")
    assert_empty_rows_zero(og, lexp[None], "zero-Q")


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("window", [(None, 0), (7, 7), (0, 0), (200, None), (None, None)])
def test_band_varlen(d, window):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [1, 127, 0, 128, 129, 300, 64, 65, 600]
    say(f"varlen band lengths={lengths} d={d} window={window}")
    q, k, v, cu = W.make_varlen(lengths, 3, d, seed=6400 + d)
    scale = 1 / np.sqrt(d)
    o, lse = aa.fa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).cuda(),
                              max(lengths), softmax_scale=scale, window=window)
    torch.cuda.synchronize()
    oref, lref = attention_varlen(to_f64(q), to_f64(k), to_f64(v), cu, scale, window=window)
    assert_o_close(o_to_f64(o), oref, f"varlen window={window} O")
    assert_l_band(lse.cpu().numpy().astype(np.float64), lref, f"varlen window={window} L")


def test_band_varlen_equals_dense_per_sequence():
    """fa_fwd_varlen on a pack == fa_fwd on each sequence alone (GPU vs GPU, bitwise)."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    lengths = [129, 1, 64, 700]
    window = (50, 10)
    say(f"varlen band vs dense per sequence window={window}")
    q, k, v, cu = W.make_varlen(lengths, 2, 128, seed=6500)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ov, lv = aa.fa_fwd_varlen(qd, kd, vd, torch.from_numpy(cu).cuda(), max(lengths),
                              window=window)
    for s, n in enumerate(lengths):
        a = int(cu[s])
        od, ld = aa.fa_fwd(qd[a:a + n][None].contiguous(), kd[a:a + n][None].contiguous(),
                           vd[a:a + n][None].contiguous(), window=window)
        torch.cuda.synchronize()
        assert torch.equal(ov[a:a + n].view(torch.int16), od[0].view(torch.int16))
        assert torch.equal(lv[:, a:a + n], ld[0])


def test_band_outputs_fully_written_and_guards_untouched():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, Nq, Nk, H, d = 2, 333, 200, 3, 64
    say("band NaN-poison/guard")
    q, k, v = W.make_dense(B, Nq, H, d, seed=6600, Nk=Nk)
    n_o, n_l, g = B * Nq * H * d, B * H * Nq, 4096
    o_buf = torch.full((n_o + 2 * g,), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((n_l + 2 * g,), float("nan"), dtype=torch.float32, device="cuda")
    o_buf[:g] = 7.0
    o_buf[-g:] = 7.0
    l_buf[:g] = 5.0
    l_buf[-g:] = 5.0
    o = o_buf[g:g + n_o].view(B, Nq, H, d)
    lse = l_buf[g:g + n_l].view(B, H, Nq)
    aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), out=o, lse=lse, window=(10, 0))
    torch.cuda.synchronize()
    # off = -133: rows 0..132 see no key (L = -inf, O = 0); every value is written.
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    assert torch.isinf(lse[:, :, :133]).all() and torch.isfinite(lse[:, :, 133:]).all()
    assert (o[:, :133] == 0).all()
    assert (o_buf[:g] == 7.0).all() and (o_buf[-g:] == 7.0).all()
    assert (l_buf[:g] == 5.0).all() and (l_buf[-g:] == 5.0).all()


def test_band_deterministic():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("band determinism")
    q, k, v = (to_dev(x) for x in W.make_dense(2, 1000, 4, 128, seed=6700))
    o1, l1 = aa.fa_fwd(q, k, v, window=(300, 20))
    o2, l2 = aa.fa_fwd(q, k, v, window=(300, 20))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


def test_full_size_band_sampled():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS["band8k"]
    say(f"full-size band8k B={w.B} N={w.N} H={w.H} d={w.d} window={w.window}")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o, lse = aa.fa_fwd(qd, kd, vd, softmax_scale=w.scale, window=w.window)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 100)
    fixed = {0, 1, 63, 64, 255, 256, 2046, 2047, 2048, 2049, w.N // 2, w.N - 2, w.N - 1}
    for h in sorted({0, w.H - 1} | {int(rng.integers(w.H)) for _ in range(3)}):
        rows = sorted(fixed | set(rng.integers(0, w.N, size=48).tolist()))
        oref, lref = attention_dense(to_f64(q[:, :, h:h + 1]), to_f64(k[:, :, h:h + 1]),
                                     to_f64(v[:, :, h:h + 1]), w.scale, rows=rows,
                                     window=w.window)
        assert_o_close(o_to_f64(o[0, rows, h]), oref[0, :, 0], f"band8k h={h}")
        assert_l_band(lse[0, h, rows].cpu().numpy().astype(np.float64), lref[0, 0],
                      f"band8k h={h}")
    vmin = vd.float().amin(dim=1, keepdim=True)
    vmax = vd.float().amax(dim=1, keepdim=True)
    of = o.float()
    slack = 1e-2 * (vmax - vmin) + 1e-3
    assert torch.isfinite(of).all() and torch.isfinite(lse).all()
    assert bool(((of >= vmin - slack) & (of <= vmax + slack)).all())
