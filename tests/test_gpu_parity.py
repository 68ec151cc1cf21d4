"""HIP path vs the float64 CPU oracle, element by element, on seeded inputs.

Small cases compare every output; they span several 256-row query tiles and
64-key tiles and end on ragged tails. The full-size workloads compare sampled
(batch, head) pairs and rows that the oracle computes one by one, plus a
property that holds at any size (each output row is a convex combination of
V rows).
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_dense, attention_varlen
from tests.gpu_util import (assert_l_close, assert_o_close, o_to_f64, say, to_dev, to_f64,
                            torch_or_skip)

pytestmark = pytest.mark.gpu


def run_dense(q, k, v, scale, causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    o, lse = aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def run_varlen(q, k, v, cu, max_seqlen, scale, causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    cu_t = torch.from_numpy(np.asarray(cu, dtype=np.int32)).cuda()
    o, lse = aa.fa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), cu_t, max_seqlen,
                              softmax_scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def check_dense_full(B, Nq, Nk, H, d, causal, seed, scale=None, rms=False):
    torch_or_skip()
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    say(f"dense B={B} Nq={Nq} Nk={Nk} H={H} d={d} causal={causal} seed={seed} scale={scale}")
    q, k, v = W.make_dense(B, Nq, H, d, seed, rms_qk=rms, Nk=Nk)
    og, lg = run_dense(q, k, v, scale, causal)
    oref, lref = attention_dense(to_f64(q), to_f64(k), to_f64(v), scale, causal)
    assert_o_close(og, oref, "O")
    assert_l_close(lg, lref, "L")


# ---------------------------------------------------------------------------
# Full comparisons at sizes the oracle finishes in seconds
# ---------------------------------------------------------------------------

def test_tiny_workload():
    w = W.WORKLOADS["tiny"]
    check_dense_full(w.B, w.N, w.N, w.H, w.d, w.causal, w.seed)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 63, 65, 127, 129, 200, 333])
def test_dense_ragged(d, causal, N):
    check_dense_full(2, N, N, 3, d, causal, seed=1000 + N + d + 7 * causal)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("Nq,Nk", [(100, 300), (300, 1), (129, 64), (1, 517)])
def test_dense_cross_lengths(d, Nq, Nk):
    check_dense_full(1, Nq, Nk, 2, d, False, seed=2000 + Nq + Nk + d)


def test_detector_400_full():
    w = W.WORKLOADS["det400"]
    check_dense_full(w.B, w.N, w.N, w.H, w.d, w.causal, w.seed)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_long_rows_several_tiles(d, causal):
    check_dense_full(1, 700, 700, 2, d, causal, seed=3000 + d + causal)


@pytest.mark.parametrize("d", [32, 128])
def test_unit_grouped_order(d):
    # Unmasked with a unit count (batch x heads) that is a multiple of 8: the
    # kernel numbers query tiles unit by unit. Three query tiles per unit, the
    # last one ragged.
    check_dense_full(2, 600, 600, 4, d, False, seed=5000 + d)


def test_varlen_unit_grouped_order():
    # Unmasked varlen with 4 sequences x 2 heads = 8 units, one sequence longer
    # than two query tiles and one of a single row.
    torch_or_skip()
    lengths = [600, 1, 300, 257]
    say(f"varlen lengths={lengths} d=64 causal=False H=2")
    q, k, v, cu = W.make_varlen(lengths, 2, 64, seed=5100)
    og, lg = run_varlen(q, k, v, cu, max(lengths), 0.125, False)
    oref, lref = attention_varlen(to_f64(q), to_f64(k), to_f64(v), cu, 0.125, False)
    assert_o_close(og, oref, "O")
    assert_l_close(lg, lref, "L")


def test_rms_normalised_qk():
    check_dense_full(2, 257, 257, 3, 128, False, seed=3, rms=True)


@pytest.mark.parametrize("scale", [0.0, 0.01, 0.6])
def test_scales(scale):
    check_dense_full(1, 190, 190, 2, 64, True, seed=77, scale=scale)


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_small(d, causal):
    torch_or_skip()
    lengths = [1, 127, 0, 128, 129, 300, 64, 65]
    cu = W.cu_seqlens_from_lengths(lengths)
    say(f"varlen lengths={lengths} d={d} causal={causal}")
    q, k, v, cu = W.make_varlen(lengths, 3, d, seed=4000 + d)
    og, lg = run_varlen(q, k, v, cu, max(lengths), 1 / np.sqrt(d), causal)
    oref, lref = attention_varlen(to_f64(q), to_f64(k), to_f64(v), cu, 1 / np.sqrt(d), causal)
    assert_o_close(og, oref, "O")
    assert_l_close(lg, lref, "L")


# ---------------------------------------------------------------------------
# Closed forms on the GPU
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_uniform_weights(causal):
    torch_or_skip()
    N, H, d = 300, 2, 128
    say(f"zero-Q closed form causal={causal}")
    _, k, v = W.make_dense(1, N, H, d, seed=91)
    q = np.zeros_like(k)
    og, lg = run_dense(q, k, v, 0.088, causal)
    vf = to_f64(v)[0]                                  # (N, H, d)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    oexp = (np.cumsum(vf, axis=0) / cnt[:, None, None]) if causal else np.broadcast_to(vf.mean(0), vf.shape)
    assert_o_close(og[0], oexp, "O = mean of visible V")
    assert_l_close(lg[0], np.broadcast_to(np.log(cnt), (H, N)), "L = ln(#visible)")


def test_constant_v_and_single_key():
    torch_or_skip()
    say("constant V / Nk=1 closed forms")
    q, k, v = W.make_dense(1, 150, 2, 64, seed=92)
    vc = np.broadcast_to(v[:, :1], v.shape).copy()          # every key row equal
    og, _ = run_dense(q, k, vc, 0.125, False)
    assert_o_close(og, np.broadcast_to(to_f64(vc)[:, :1], og.shape), "constant V")
    og, lg = run_dense(q, k[:, :1], v[:, :1], 0.125, False)  # one key
    assert_o_close(og, np.broadcast_to(to_f64(v)[:, :1], og.shape), "Nk=1 O")
    lexp = 0.125 * np.einsum("bnhd,bhd->bhn", to_f64(q), to_f64(k)[:, 0])
    assert_l_close(lg, lexp, "Nk=1 L")


# ---------------------------------------------------------------------------
# Every output written, nothing else touched, repeatable
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_outputs_fully_written_and_guards_untouched(causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    B, N, H, d = 2, 333, 3, 128
    say(f"NaN-poison/guard causal={causal}")
    q, k, v = W.make_dense(B, N, H, d, seed=93)
    n_o, n_l, g = B * N * H * d, B * H * N, 4096
    o_buf = torch.full((n_o + 2 * g,), float("nan"), dtype=torch.bfloat16, device="cuda")
    l_buf = torch.full((n_l + 2 * g,), float("nan"), dtype=torch.float32, device="cuda")
    o_buf[:g] = 7.0
    o_buf[-g:] = 7.0
    l_buf[:g] = 5.0
    l_buf[-g:] = 5.0
    o = o_buf[g:g + n_o].view(B, N, H, d)
    lse = l_buf[g:g + n_l].view(B, H, N)
    aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert (o_buf[:g] == 7.0).all() and (o_buf[-g:] == 7.0).all()
    assert (l_buf[:g] == 5.0).all() and (l_buf[-g:] == 5.0).all()


def test_varlen_rows_outside_sequences_untouched():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say("varlen guard rows")
    lengths = [50, 0, 200]
    q, k, v, cu = W.make_varlen(lengths, 2, 64, seed=94)
    total = q.shape[0]
    o = torch.full((total, 2, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((2, total), float("nan"), dtype=torch.float32, device="cuda")
    cu_t = torch.from_numpy(cu).cuda()
    aa.fa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), cu_t, 200, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("causal", [False, True])
def test_deterministic(causal):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say(f"determinism causal={causal}")
    q, k, v = (to_dev(x) for x in W.make_dense(2, 1000, 4, 128, seed=95))
    o1, l1 = aa.fa_fwd(q, k, v, causal=causal)
    o2, l2 = aa.fa_fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equals_dense_per_sequence(causal):
    """fa_fwd_varlen on a pack == fa_fwd on each sequence alone (GPU vs GPU, bitwise)."""
    import aware_attention_amd as aa
    torch = torch_or_skip()
    say(f"varlen vs dense per sequence causal={causal}")
    lengths = [129, 1, 64, 257]
    q, k, v, cu = W.make_varlen(lengths, 2, 128, seed=96)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    ov, lv = aa.fa_fwd_varlen(qd, kd, vd, torch.from_numpy(cu).cuda(), max(lengths), causal=causal)
    for s, n in enumerate(lengths):
        a = int(cu[s])
        od, ld = aa.fa_fwd(qd[a:a + n][None].contiguous(), kd[a:a + n][None].contiguous(),
                           vd[a:a + n][None].contiguous(), causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(ov[a:a + n].view(torch.int16), od[0].view(torch.int16))
        assert torch.equal(lv[:, a:a + n], ld[0])


# ---------------------------------------------------------------------------
# Full-size workloads, sampled
# ---------------------------------------------------------------------------

def _sample_rows(N, rng, n=48):
    fixed = {0, 1, 63, 64, 127, 128, N // 2, N - 2, N - 1}
    rows = sorted({r for r in fixed if 0 <= r < N} | set(rng.integers(0, N, size=n).tolist()))
    return rows


@pytest.mark.parametrize("name", ["det1600", "vit", "prefill2k", "prefill8k"])
def test_full_size_dense_sampled(name):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS[name]
    say(f"full-size {name} B={w.B} N={w.N} H={w.H} d={w.d} causal={w.causal}")
    q, k, v = W.make_dense(w.B, w.N, w.H, w.d, w.seed, rms_qk=w.rms_qk)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    o, lse = aa.fa_fwd(qd, kd, vd, softmax_scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(w.seed + 100)
    pairs = {(0, 0), (w.B - 1, w.H - 1)} | {(int(rng.integers(w.B)), int(rng.integers(w.H))) for _ in range(3)}
    for b, h in sorted(pairs):
        rows = _sample_rows(w.N, rng)
        oref, lref = attention_dense(to_f64(q[b:b + 1, :, h:h + 1]), to_f64(k[b:b + 1, :, h:h + 1]),
                                     to_f64(v[b:b + 1, :, h:h + 1]), w.scale, w.causal, rows=rows)
        og = o_to_f64(o[b, rows, h])
        lg = lse[b, h, rows].cpu().numpy().astype(np.float64)
        assert_o_close(og, oref[0, :, 0], f"{name} b={b} h={h}")
        assert_l_close(lg, lref[0, 0], f"{name} b={b} h={h}")
    # property at full size: O rows are convex combinations of V rows
    vmin = vd.float().amin(dim=1, keepdim=True)
    vmax = vd.float().amax(dim=1, keepdim=True)
    of = o.float()
    slack = 1e-2 * (vmax - vmin) + 1e-3
    assert torch.isfinite(of).all() and torch.isfinite(lse).all()
    assert bool(((of >= vmin - slack) & (of <= vmax + slack)).all())


def test_full_size_varlen_sampled():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    wl = W.make_workload("varlen")
    w = wl["spec"]
    say(f"full-size varlen seqs={w.num_seqs} total={wl['q'].shape[0]} max={wl['max_seqlen']}")
    q, k, v, cu = wl["q"], wl["k"], wl["v"], wl["cu_seqlens"]
    o, lse = aa.fa_fwd_varlen(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).cuda(),
                              wl["max_seqlen"], softmax_scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    rng = np.random.default_rng(404)
    seqs = sorted({0, w.num_seqs - 1} | set(rng.integers(0, w.num_seqs, size=4).tolist()))
    heads = [0, w.H - 1, int(rng.integers(w.H))]
    oref, lref = attention_varlen(to_f64(q), to_f64(k), to_f64(v), cu, w.scale, w.causal,
                                  seqs=seqs, heads=heads)
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    for s in seqs:
        a, b = int(cu[s]), int(cu[s + 1])
        for h in heads:
            assert_o_close(og[a:b, h], oref[a:b, h], f"varlen seq={s} h={h}")
            assert_l_close(lg[h, a:b], lref[h, a:b], f"varlen seq={s} h={h}")
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
