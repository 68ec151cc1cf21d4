"""MI355X (gfx950) FlashAttention-2 forward: thin Python binding over libfa.so.

Every step of the computation runs in the HIP kernels of libfa.so; this
module only checks and marshals arguments, allocates outputs through torch
and passes torch's current HIP stream. There is no fallback path: if the
library is missing or the device is not a gfx950, calls raise.

    o, lse = fa_fwd(q, k, v, softmax_scale=None, causal=False)
        q (B,Nq,H,d), k/v (B,Nk,H,d) bfloat16 CUDA tensors -> o (B,Nq,H,d) bf16,
        lse (B,H,Nq) float32.
    o, lse = fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, causal=False)
        q/k/v (total,H,d), cu_seqlens int32 (num_seqs+1,) on the device ->
        o (total,H,d), lse (H,total).
    Both take window=(left, right) instead of causal for a banded mask: query i
    sees key j iff i + (Nk - Nq) - left <= j <= i + (Nk - Nq) + right (varlen:
    offset 0), None meaning no bound on that side; rows that see no key get
    o = 0 and lse = -inf (entry points fa_fwd_band / fa_fwd_varlen_band).
    q, k, v (and out) may be float16 instead of bfloat16 (all the same type),
    and may be strided views whose last dimension is contiguous and whose other
    strides are multiples of 8 elements, such as q = qkv[:, :, 0] of a packed
    (B, S, 3, H, d) tensor; such calls go through fa_fwd_strided /
    fa_fwd_varlen_strided with no copy.
    dq, dk, dv, delta = fa_bwd(q, k, v, o, lse, dout, softmax_scale=None, causal=False)
    dq, dk, dv, delta = fa_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen, ...)
        the backward (contiguous tensors of one half-precision type): S and P are
        recomputed from lse; delta = rowsum(dout * o), laid out like lse.
    o = attention(q, k, v, softmax_scale=None, causal=False)
        forward with autograd: o.backward(...) runs fa_bwd.
    o, lse = fa_decode(q, k, v, seqlens_k=None, softmax_scale=None)
        one query per (batch, head), q (B,1,H,d), k/v (B,Nk,H,d) the cache, split
        over the cache and merged through the log-sum-exps (fa_decode).

The default scale is 1/sqrt(d), as in the definition on "FlashAttention/zh"
(marovi.ai wiki), section 為何標準注意力運行緩慢. Only half precision on the
device is accepted and no attention weights are returned, as in
"InternViT-6B-448px-V1-2 如何加速注意力计算", section
FlashAttention 封装类三条执行路径 (硬性约束).
"""
from __future__ import annotations

import math

from ._lib import (FA_DTYPE_BF16, FA_DTYPE_F16, FA_ERR_HIP, FA_ERR_INVALID_ARGUMENT,
                   FA_ERR_UNSUPPORTED, FA_OK, FaError, check, decode_workspace_bytes, load,
                   raw_fa_bwd, raw_fa_bwd_band, raw_fa_bwd_padded, raw_fa_bwd_varlen,
                   raw_fa_bwd_local, raw_fa_bwd_varlen_band, raw_fa_decode, raw_fa_fwd_local,
                   raw_fa_fwd, raw_fa_fwd_band, raw_fa_fwd_padded, raw_fa_fwd_strided,
                   raw_fa_fwd_varlen,
                   raw_fa_fwd_varlen_band, raw_fa_fwd_varlen_strided)

__all__ = ["fa_fwd", "fa_fwd_varlen", "fa_fwd_local", "fa_bwd", "fa_bwd_varlen", "fa_decode",
           "attention",
           "FaError", "load",
           "FA_OK", "FA_ERR_INVALID_ARGUMENT", "FA_ERR_UNSUPPORTED", "FA_ERR_HIP"]


def _torch():
    import torch
    return torch


def _dtype_code(dtype):
    torch = _torch()
    if dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if dtype == torch.float16:
        return FA_DTYPE_F16
    raise TypeError(f"q, k, v must be bfloat16 or float16 (got {dtype})")


def _check_tensor(t, name, ndim):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    _dtype_code(t.dtype)
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got shape {tuple(t.shape)})")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous last (head) dimension")


def _strides(t):
    """Element strides of every dimension but the last; 0 for dimensions of size 1,
    whose stride never matters."""
    return [t.stride(i) if t.shape[i] > 1 else 0 for i in range(t.dim() - 1)]


def _plain(*ts):
    """True when every tensor is contiguous bfloat16 (the entry points without strides)."""
    torch = _torch()
    return all(t.is_contiguous() and t.dtype == torch.bfloat16 for t in ts)


def _out(out, like, shape, name):
    torch = _torch()
    if out is None:
        return torch.empty(shape, dtype=like.dtype, device=like.device)
    _check_tensor(out, name, len(shape))
    if tuple(out.shape) != tuple(shape) or out.dtype != like.dtype:
        raise ValueError(f"{name} must have shape {tuple(shape)} and dtype {like.dtype}")
    return out


def _scale(softmax_scale, d):
    return 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)


def _window(window, causal):
    """(left, right) with None for unbounded -> the ABI's ints (-1 = unbounded)."""
    if causal:
        raise ValueError("pass either causal=True or window, not both (causal is window=(None, 0))")
    left, right = window
    sides = tuple(-1 if w is None else int(w) for w in (left, right))
    if any(w is not None and int(w) < 0 for w in (left, right)):
        raise ValueError("window sides must be >= 0, or None for unbounded")
    return tuple(min(w, 2**31 - 1) for w in sides)


def fa_fwd(q, k, v, softmax_scale=None, causal=False, out=None, lse=None, window=None,
           key_padding_mask=None):
    """Attention forward over an equal-length batch; returns (o, lse).

    key_padding_mask (B, S) bool or uint8 on q's device, nonzero = valid token:
    self-attention over the valid tokens of each batch row, padding positions
    returning o = 0 and lse = -inf (fa_fwd_padded)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n, 4)
    B, Nq, H, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != d:
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError(f"q, k and v must share one dtype (got {q.dtype}, {k.dtype}, {v.dtype})")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    Nk = k.shape[1]
    out = _out(out, q, (B, Nq, H, d), "out")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse.shape != (B, H, Nq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, H, Nq)")
    scale = _scale(softmax_scale, d)
    wl, wr = (-1, -1) if window is None else _window(window, causal)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr())
    if key_padding_mask is not None:
        m = key_padding_mask
        if window is not None:
            raise ValueError("key_padding_mask and window are exclusive")
        if Nk != Nq:
            raise ValueError("key_padding_mask is for self-attention (Nq == Nk)")
        if not all(t.is_contiguous() for t in (q, k, v, out)):
            raise ValueError("q, k, v and out must be contiguous with key_padding_mask")
        if not isinstance(m, torch.Tensor) or m.dtype not in (torch.bool, torch.uint8) \
                or tuple(m.shape) != (B, Nq) or m.device != q.device or not m.is_contiguous():
            raise ValueError("key_padding_mask must be a contiguous (B, S) bool or uint8 tensor "
                             "on q's device")
        m = m.view(torch.uint8)
        with torch.cuda.device(q.device):
            stream = torch.cuda.current_stream(q.device).cuda_stream
            check(raw_fa_fwd_padded(*ptrs, m.data_ptr(), B, Nq, H, d, _dtype_code(q.dtype), scale,
                                    int(bool(causal)), stream))
        return out, lse
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if not _plain(q, k, v, out):
            check(raw_fa_fwd_strided(*ptrs, B, Nq, Nk, H, d, _strides(q), _strides(k),
                                     _strides(v), _strides(out), _dtype_code(q.dtype), scale,
                                     int(bool(causal)), wl, wr, stream))
        elif window is None:
            check(raw_fa_fwd(*ptrs, B, Nq, Nk, H, d, scale, int(bool(causal)), stream))
        else:
            check(raw_fa_fwd_band(*ptrs, B, Nq, Nk, H, d, scale, wl, wr, stream))
    return out, lse


def fa_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, softmax_scale=None, causal=False,
                  out=None, lse=None, window=None):
    """Attention forward over a packed variable-length batch; returns (o, lse)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n, 3)
    total, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must share the packed shape (total, H, d)")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError(f"q, k and v must share one dtype (got {q.dtype}, {k.dtype}, {v.dtype})")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 \
            or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 1-D tensor on q's device")
    num_seqs = cu_seqlens.numel() - 1
    out = _out(out, q, (total, H, d), "out")
    if lse is None:
        lse = torch.empty((H, total), dtype=torch.float32, device=q.device)
    if lse.shape != (H, total) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape (H, total)")
    scale = _scale(softmax_scale, d)
    wl, wr = (-1, -1) if window is None else _window(window, causal)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            cu_seqlens.data_ptr())
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if not _plain(q, k, v, out):
            check(raw_fa_fwd_varlen_strided(*ptrs, num_seqs, int(max_seqlen), total, H, d,
                                            _strides(q), _strides(k), _strides(v),
                                            _strides(out), _dtype_code(q.dtype), scale,
                                            int(bool(causal)), wl, wr, stream))
        elif window is None:
            check(raw_fa_fwd_varlen(*ptrs, num_seqs, int(max_seqlen), total, H, d, scale,
                                    int(bool(causal)), stream))
        else:
            check(raw_fa_fwd_varlen_band(*ptrs, num_seqs, int(max_seqlen), total, H, d, scale,
                                         wl, wr, stream))
    return out, lse


def _check_contiguous(ts, names, dtype):
    for t, n in zip(ts, names):
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous for the backward")
        if t.dtype != dtype:
            raise TypeError(f"{n} must be {dtype} like q (got {t.dtype})")


def fa_bwd(q, k, v, o, lse, dout, softmax_scale=None, causal=False, dq=None, dk=None, dv=None,
           delta=None, window=None, key_padding_mask=None, local=None):
    """Backward over an equal-length batch; returns (dq, dk, dv, delta). window,
    key_padding_mask and local = (n_global, map_w, win_rows, win_cols) are those of
    the forward call (fa_bwd_band, fa_bwd_padded, fa_bwd_local)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check_tensor(t, n, 4)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != d \
            or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o and dout")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta is None:
        delta = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_contiguous((q, k, v, o, dout, dq, dk, dv), ("q", "k", "v", "o", "dout", "dq", "dk", "dv"),
                      q.dtype)
    if dq.shape != q.shape or dk.shape != k.shape or dv.shape != v.shape:
        raise ValueError("dq, dk and dv must be shaped like q, k and v")
    for t, n in ((lse, "lse"), (delta, "delta")):
        if t.shape != (B, H, Nq) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 tensor of shape (B, H, Nq)")
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr())
    dt, scale = _dtype_code(q.dtype), _scale(softmax_scale, d)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if local is not None:
            if window is not None or key_padding_mask is not None or Nk != Nq:
                raise ValueError("local: self-attention only, without a window or padding mask")
            clamp = lambda x: max(min(int(x), 2**31 - 1), -1)  # noqa: E731
            G, mw, wr, wc = (clamp(x) for x in local)
            check(raw_fa_bwd_local(*ptrs, B, Nq, H, d, dt, scale, int(bool(causal)), G, mw, wr,
                                   wc, stream))
        elif key_padding_mask is not None:
            m = key_padding_mask
            if window is not None or Nk != Nq:
                raise ValueError("key_padding_mask: self-attention only, and not with a window")
            if not isinstance(m, torch.Tensor) or m.dtype not in (torch.bool, torch.uint8) \
                    or tuple(m.shape) != (B, Nq) or m.device != q.device or not m.is_contiguous():
                raise ValueError("key_padding_mask must be a contiguous (B, S) bool or uint8 "
                                 "tensor on q's device")
            check(raw_fa_bwd_padded(*ptrs, m.view(torch.uint8).data_ptr(), B, Nq, H, d, dt, scale,
                                    int(bool(causal)), stream))
        elif window is not None:
            wl, wr = _window(window, causal)
            check(raw_fa_bwd_band(*ptrs, B, Nq, Nk, H, d, dt, scale, wl, wr, stream))
        else:
            check(raw_fa_bwd(*ptrs, B, Nq, Nk, H, d, dt, scale, int(bool(causal)), stream))
    return dq, dk, dv, delta


def fa_bwd_varlen(q, k, v, o, lse, dout, cu_seqlens, max_seqlen, softmax_scale=None,
                  causal=False, dq=None, dk=None, dv=None, delta=None, window=None):
    """Backward over a packed variable-length batch; returns (dq, dk, dv, delta)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check_tensor(t, n, 3)
    total, H, d = q.shape
    if any(t.shape != q.shape for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o and dout must share the packed shape (total, H, d)")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 \
            or cu_seqlens.dim() != 1 or cu_seqlens.device != q.device or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 1-D tensor on q's device")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if delta is None:
        delta = torch.empty((H, total), dtype=torch.float32, device=q.device)
    _check_contiguous((q, k, v, o, dout, dq, dk, dv), ("q", "k", "v", "o", "dout", "dq", "dk", "dv"),
                      q.dtype)
    if any(t.shape != q.shape for t in (dq, dk, dv)):
        raise ValueError("dq, dk and dv must be shaped like q")
    for t, n in ((lse, "lse"), (delta, "delta")):
        if t.shape != (H, total) or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous float32 tensor of shape (H, total)")
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), cu_seqlens.data_ptr())
    dt, scale = _dtype_code(q.dtype), _scale(softmax_scale, d)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if window is not None:
            wl, wr = _window(window, causal)
            check(raw_fa_bwd_varlen_band(*ptrs, cu_seqlens.numel() - 1, int(max_seqlen), total, H,
                                         d, dt, scale, wl, wr, stream))
        else:
            check(raw_fa_bwd_varlen(*ptrs, cu_seqlens.numel() - 1, int(max_seqlen), total, H, d,
                                    dt, scale, int(bool(causal)), stream))
    return dq, dk, dv, delta


def _autograd_function():
    torch = _torch()

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, softmax_scale, causal, window, key_padding_mask, local):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            if local is not None:
                if window is not None or key_padding_mask is not None:
                    raise ValueError("local excludes window and key_padding_mask")
                G, mw, wr, wc = local
                o, lse = fa_fwd_local(q, k, v, G, mw, (wr, wc), softmax_scale=softmax_scale,
                                      causal=causal)
            else:
                o, lse = fa_fwd(q, k, v, softmax_scale=softmax_scale, causal=causal,
                                window=window, key_padding_mask=key_padding_mask)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.softmax_scale, ctx.causal, ctx.window = softmax_scale, causal, window
            ctx.key_padding_mask, ctx.local = key_padding_mask, local
            return o

        @staticmethod
        def backward(ctx, dout):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv, _ = fa_bwd(q, k, v, o, lse, dout.contiguous(),
                                   softmax_scale=ctx.softmax_scale, causal=ctx.causal,
                                   window=ctx.window, key_padding_mask=ctx.key_padding_mask,
                                   local=ctx.local)
            return dq, dk, dv, None, None, None, None, None

    return _Attention


_ATTENTION_FN = None


def attention(q, k, v, softmax_scale=None, causal=False, window=None, key_padding_mask=None,
              local=None):
    """o = softmax(scale q k^T) v over (B, N, H, d) tensors, differentiable: the
    forward is fa_fwd (fa_fwd_local with local = (n_global, map_w, win_rows,
    win_cols)) and the backward fa_bwd (all HIP kernels), with the same causal
    flag, band, key padding mask or local pattern."""
    global _ATTENTION_FN
    if _ATTENTION_FN is None:
        _ATTENTION_FN = _autograd_function()
    return _ATTENTION_FN.apply(q, k, v, softmax_scale, causal, window, key_padding_mask, local)


def fa_fwd_local(q, k, v, n_global, map_w, window, softmax_scale=None, causal=False, out=None,
                 lse=None):
    """Local window on a token map plus global anchors: q, k, v (B, N, H, d) contiguous
    bf16 or fp16; tokens [0, n_global) are anchors, the rest a row-major map of map_w
    tokens per row; window = (win_rows, win_cols), e.g. (2, 2) for a 5 x 5 window.
    Query i sees key j iff i or j is an anchor or their map positions are within the
    window (and j <= i when causal). Returns (o (B, N, H, d), lse (B, H, N) float32)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n, 4)
    B, N, H, d = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one shape (B, N, H, d): q {tuple(q.shape)} "
                         f"k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if not all(t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k and v must be contiguous")
    win_rows, win_cols = (int(w) for w in window)
    out = _out(out, q, (B, N, H, d), "out")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if tuple(lse.shape) != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, H, N)")
    clamp = lambda x: max(min(int(x), 2**31 - 1), -1)  # noqa: E731 - sizes beyond int32 mean no bound
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        check(raw_fa_fwd_local(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, N, H, d, _dtype_code(q.dtype),
                               _scale(softmax_scale, d), int(bool(causal)), clamp(n_global),
                               clamp(map_w), clamp(win_rows), clamp(win_cols), stream))
    return out, lse


def fa_decode(q, k, v, seqlens_k=None, softmax_scale=None, out=None, lse=None, workspace=None):
    """Decode step: q (B, 1, H, d), k/v (B, Nk, H, d); returns (o (B, 1, H, d), lse (B, H)).
    seqlens_k: optional int32 (B,) on the device, the valid cache length per batch.
    workspace: optional uint8 device tensor of at least decode_workspace_bytes(...) bytes
    (allocated here through torch when None)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_tensor(t, n, 4)
    B, one, H, d = q.shape
    Nk = k.shape[1]
    if one != 1 or k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != d:
        raise ValueError(f"decode needs q (B,1,H,d) and k, v (B,Nk,H,d): q {tuple(q.shape)} "
                         f"k {tuple(k.shape)} v {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if not all(t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k and v must be contiguous for the decode")
    out = torch.empty_like(q) if out is None else out
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped like q")
    if lse.shape != (B, H) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor of shape (B, H)")
    sl = 0
    if seqlens_k is not None:
        if not isinstance(seqlens_k, torch.Tensor) or seqlens_k.dtype != torch.int32 \
                or tuple(seqlens_k.shape) != (B,) or seqlens_k.device != q.device:
            raise ValueError("seqlens_k must be an int32 tensor of shape (B,) on q's device")
        sl = seqlens_k.data_ptr()
    need = decode_workspace_bytes(B, Nk, H, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        check(raw_fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), sl or None, B, Nk, H, d, _dtype_code(q.dtype),
                            _scale(softmax_scale, d), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), stream))
    return out, lse
