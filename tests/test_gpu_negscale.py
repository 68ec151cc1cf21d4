"""Negative softmax scales against the float64 oracle (the definition holds
for any finite scale; the pages' 1/sqrt(d) is only the default). The d <= 128
and d = 256 forward kernels move the sign into their Q registers; the local,
decode and backward kernels scale every score before any maximum. Every
entry point runs at scale -0.3 (and -1/sqrt(d)), with the usual bars.
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention_dense, attention_varlen
from tests.gpu_util import assert_l_close, assert_o_close, say, to_f64, torch_or_skip
from tests.test_gpu_backward import check_bwd_dense
from tests.test_gpu_band import check_band
from tests.test_gpu_d256 import check_256
from tests.test_gpu_decode import check_decode
from tests.test_gpu_local import check_local
from tests.test_gpu_padded import check_padded
from tests.test_gpu_parity import check_dense_full, run_varlen

pytestmark = pytest.mark.gpu

NEG = -0.3


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [65, 333])
def test_negative_scale_dense(d, causal, N):
    check_dense_full(2, N, N, 2, d, causal, seed=12000 + N + d, scale=NEG)


@pytest.mark.parametrize("d", [64, 128])
def test_negative_scale_dense_minus_inverse_sqrt_d(d):
    check_dense_full(1, 700, 700, 2, d, True, seed=12100 + d, scale=-1 / np.sqrt(d))


def test_negative_scale_cross_lengths():
    check_dense_full(1, 129, 700, 3, 128, False, seed=12150, scale=NEG)


@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_varlen(causal):
    torch_or_skip()
    lengths = [1, 300, 0, 129, 257]
    say(f"negative scale varlen lengths={lengths} causal={causal}")
    q, k, v, cu = W.make_varlen(lengths, 3, 128, seed=12200)
    og, lg = run_varlen(q, k, v, cu, max(lengths), NEG, causal)
    oref, lref = attention_varlen(to_f64(q), to_f64(k), to_f64(v), cu, NEG, causal)
    assert_o_close(og, oref, "O")
    assert_l_close(lg, lref, "L")


@pytest.mark.parametrize("window", [(None, 0), (16, 16), (100, 3)])
def test_negative_scale_band(window):
    check_band(1, 333, 333, 2, 128, window, seed=12300, scale=NEG)


@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_padded(causal):
    check_padded(2, 333, 2, 64, causal, seed=12400, scale=NEG)


@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_d256(causal):
    check_256(1, 300, 300, 2, causal, seed=12500, scale=NEG)


@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_local(causal):
    check_local(1, 8 + 20 * 20, 2, 64, 8, 20, (2, 2), causal, seed=12600, scale=NEG)


def test_negative_scale_decode():
    check_decode(2, 3000, 4, 128, seed=12700, lens=[3000, 1234], scale=NEG)


@pytest.mark.parametrize("causal", [False, True])
def test_negative_scale_backward(causal):
    check_bwd_dense(2, 200, 200, 2, 64, causal, seed=12800, scale=NEG)


def test_negative_scale_flips_the_softmax():
    """Closed form at full precision: with K = Q (self-keys) and scale -s the
    weights favour the least similar keys; the result equals the oracle run
    with Q negated and scale +s (the identity the kernels rely on)."""
    torch_or_skip()
    q, k, v = W.make_dense(1, 200, 2, 128, seed=12900)
    og, lg = None, None
    import aware_attention_amd as aa
    from tests.gpu_util import o_to_f64, to_dev
    import torch
    o, lse = aa.fa_fwd(to_dev(q), to_dev(k), to_dev(v), softmax_scale=NEG, causal=True)
    torch.cuda.synchronize()
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    oref, lref = attention_dense(-to_f64(q), to_f64(k), to_f64(v), -NEG, True)
    assert_o_close(og, oref, "O")
    assert_l_close(lg, lref, "L")
