"""fa_decode_noalloc (the decode entry point that allocates nothing) against
fa_decode, its workspace-taking twin, called through the C ABI.

Two calls in a row share the library's scratch array: a large one, then a
smaller one whose partial results occupy a prefix of what the first left
behind. Each output must equal fa_decode's bit for bit (the same kernels and
split plan), and both are checked against the float64 oracle at the forward's
bar (O: 2e-2 + 2e-2 |ref| per element; L: max-abs 1e-3).
"""
import numpy as np
import pytest

import workloads as W
from oracle import attention
from tests.gpu_util import L_ATOL, assert_o_close, o_to_f64, say, to_dev, to_f64, torch_or_skip

pytestmark = pytest.mark.gpu


def _raw_pair(B, Nk, H, d, seed, lens, dtype="bf16"):
    """(fa_decode_noalloc outputs, fa_decode outputs, inputs) through the raw C ABI."""
    import aware_attention_amd._lib as L
    torch = torch_or_skip()
    q = W.make_dense(B, 1, H, d, seed, dtype=dtype)[0]
    _, k, v = W.make_dense(B, Nk, H, d, seed + 1, dtype=dtype)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    code = L.FA_DTYPE_BF16 if dtype == "bf16" else L.FA_DTYPE_F16
    scale = 1.0 / np.sqrt(d)
    stream = torch.cuda.current_stream().cuda_stream
    o1, o2 = torch.full_like(qd, float("nan")), torch.full_like(qd, float("nan"))
    l1 = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    l2 = torch.full_like(l1, float("nan"))
    need = L.decode_workspace_bytes(B, Nk, H, d)
    assert 0 < need <= L.FA_DECODE_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    st = L.raw_fa_decode_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o1.data_ptr(),
                                 l1.data_ptr(), sl.data_ptr(), B, Nk, H, d, code, scale, stream)
    assert st == L.FA_OK, L.load().fa_last_error()
    st = L.raw_fa_decode(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o2.data_ptr(),
                         l2.data_ptr(), sl.data_ptr(), B, Nk, H, d, code, scale, ws.data_ptr(),
                         need, stream)
    assert st == L.FA_OK, L.load().fa_last_error()
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2), (q, k, v)


def _check_oracle(o, lse, q, k, v, lens, d, dtype):
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    qf, kf, vf = to_f64(q, dtype), to_f64(k, dtype), to_f64(v, dtype)
    B, _, H, _ = q.shape
    for b in range(B):
        n = max(0, min(lens[b], k.shape[1]))
        for h in range(H):
            if n == 0:
                assert np.all(og[b, 0, h] == 0) and np.isneginf(lg[b, h])
                continue
            oref, lref = attention(qf[b, :, h], kf[b, :n, h], vf[b, :n, h], 1.0 / np.sqrt(d))
            assert_o_close(og[b, 0, h][None], oref, f"noalloc O b={b} h={h}")
            assert abs(lg[b, h] - lref[0]) <= L_ATOL


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_noalloc_decode_equals_workspace_decode_twice(dtype):
    torch = torch_or_skip()
    # first call: 16 (batch, head) pairs over a 20000-key cache (many chunks, most of
    # the scratch's partial results); second call: smaller in every size
    for B, Nk, H, d, lens, seed in ((4, 20000, 4, 128, [20000, 12345, 1, 0], 7100),
                                    (2, 700, 3, 64, [700, 350], 7200)):
        say(f"noalloc decode B={B} Nk={Nk} H={H} d={d} lens={lens} {dtype}")
        (o1, l1), (o2, l2), (q, k, v) = _raw_pair(B, Nk, H, d, seed, lens, dtype)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "O differs from fa_decode"
        assert torch.equal(l1, l2), "L differs from fa_decode"
        _check_oracle(o1, l1, q, k, v, lens, d, dtype)
