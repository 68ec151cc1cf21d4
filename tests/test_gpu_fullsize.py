"""Whole outputs at full size: every (batch or sequence, head, row) of O and
L from the HIP forward, called as the benchmark calls it, against the float64
oracle, for each timed workload shape (tiny, the two detector maps, the ViT
batch, the packed variable-length batch and both causal prefill shapes).

The oracle is the plain definition (oracle.attention), run once per
(batch or sequence, head) on the host; the heads run in a thread pool with
single-threaded BLAS, and each workload's reference is computed once per test
session (oracle time on 16 host cores: about a minute in all). Bar: the
element-wise O bound 2e-2 + 2e-2 |ref| and max-abs 1e-3 on L.
"""
import functools
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import workloads as W
from oracle import attention
from tests.gpu_util import (assert_l_close, assert_o_close, o_to_f64, say, to_dev, to_f64,
                            torch_or_skip)

pytestmark = pytest.mark.gpu

_WORKERS = min(16, os.cpu_count() or 1)


def _pool_map(fn, items):
    """fn over items in threads (numpy releases the GIL), BLAS single-threaded."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(_WORKERS) as ex:
        return list(ex.map(fn, items))


@functools.lru_cache(maxsize=None)
def _reference(name: str):
    """(inputs, O_ref, L_ref) of a workload in the kernel's layouts, float64."""
    wl = W.make_workload(name)
    spec = wl["spec"]
    q, k, v = (to_f64(wl[x]) for x in ("q", "k", "v"))
    if isinstance(spec, W.Dense):
        B, N, H, d = q.shape
        units = [(b, h) for b in range(B) for h in range(H)]

        def one(u):
            b, h = u
            return attention(q[b, :, h], k[b, :, h], v[b, :, h], spec.scale, spec.causal)
        res = _pool_map(one, units)
        O = np.empty_like(q)
        L = np.empty((B, H, N))
        for (b, h), (o, l) in zip(units, res):
            O[b, :, h], L[b, h] = o, l
    else:
        cu = wl["cu_seqlens"]
        total, H, d = q.shape
        units = [(s, h) for s in range(spec.num_seqs) for h in range(H)]

        def one(u):
            s, h = u
            a, e = int(cu[s]), int(cu[s + 1])
            return attention(q[a:e, h], k[a:e, h], v[a:e, h], spec.scale, spec.causal)
        res = _pool_map(one, units)
        O = np.empty_like(q)
        L = np.empty((H, total))
        for (s, h), (o, l) in zip(units, res):
            a, e = int(cu[s]), int(cu[s + 1])
            O[a:e, h], L[h, a:e] = o, l
    return wl, O, L


@pytest.mark.parametrize("name", ["tiny", "det1600", "det400", "vit", "prefill2k", "prefill8k"])
def test_full_size_dense_every_output(name):
    import aware_attention_amd as aa
    torch = torch_or_skip()
    w = W.WORKLOADS[name]
    say(f"full-size every output {name} B={w.B} N={w.N} H={w.H} d={w.d} causal={w.causal}")
    wl, O_ref, L_ref = _reference(name)
    qd, kd, vd = to_dev(wl["q"]), to_dev(wl["k"]), to_dev(wl["v"])
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    aa.fa_fwd(qd, kd, vd, softmax_scale=w.scale, causal=w.causal, out=o, lse=lse)
    torch.cuda.synchronize()
    og = o_to_f64(o)
    lg = lse.cpu().numpy().astype(np.float64)
    for b in range(w.B):   # per batch, so a failure names where it is
        assert_o_close(og[b], O_ref[b], f"{name} b={b}")
        assert_l_close(lg[b], L_ref[b], f"{name} b={b}")


def test_full_size_varlen_every_output():
    import aware_attention_amd as aa
    torch = torch_or_skip()
    wl, O_ref, L_ref = _reference("varlen")
    spec, cu = wl["spec"], wl["cu_seqlens"]
    say(f"full-size every output varlen seqs={spec.num_seqs} total={wl['q'].shape[0]} "
        f"max={wl['max_seqlen']}")
    qd, kd, vd = to_dev(wl["q"]), to_dev(wl["k"]), to_dev(wl["v"])
    o = torch.empty_like(qd)
    lse = torch.empty((spec.H, qd.shape[0]), dtype=torch.float32, device="cuda")
    aa.fa_fwd_varlen(qd, kd, vd, torch.from_numpy(cu).cuda(), wl["max_seqlen"],
                     softmax_scale=spec.scale, causal=spec.causal, out=o, lse=lse)
    torch.cuda.synchronize()
    og, lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    for s in range(spec.num_seqs):
        a, e = int(cu[s]), int(cu[s + 1])
        assert_o_close(og[a:e], O_ref[a:e], f"varlen seq={s}")
        assert_l_close(lg[:, a:e], L_ref[:, a:e], f"varlen seq={s}")
