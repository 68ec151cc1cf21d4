"""ctypes view of libfa.so (the C ABI declared in include/fa.h).

Loading fails loudly: there is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

# The library: libfa.so next to this file, or the build that the environment
# variable AWARE_ATTENTION_LIB names (the timing-perturbed libfa_stress.so of
# the race tests). Either way it must exist: there is no fallback.
LIB_PATH = os.environ.get("AWARE_ATTENTION_LIB") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARGUMENT = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3

FA_DTYPE_BF16 = 0
FA_DTYPE_F16 = 1

EXPORTED = ("fa_fwd", "fa_fwd_varlen", "fa_fwd_band", "fa_fwd_varlen_band", "fa_fwd_strided",
            "fa_fwd_varlen_strided", "fa_fwd_padded", "fa_bwd", "fa_bwd_varlen", "fa_bwd_band",
            "fa_bwd_varlen_band", "fa_bwd_padded", "fa_bwd_strided", "fa_bwd_varlen_strided",
            "fa_decode", "fa_fwd_local", "fa_bwd_local",
            "fa_decode_workspace_bytes", "fa_decode_noalloc", "fa_fwd_mx8",
            "fa_mx8_tokens_padded", "fa_mx8_quantize_qk", "fa_mx8_quantize_v", "fa_status_string",
            "fa_last_error", "fa_abi_version")

_lib = None


class FaError(RuntimeError):
    """A libfa call returned a status other than FA_OK."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load() -> ctypes.CDLL:
    """Load libfa.so once (raises OSError naming the path when it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"libfa.so is not built: {LIB_PATH} is missing "
                      f"(run `python -m aware_attention_amd.build`)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd.restype = i32
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd_varlen.restype = i32
    lib.fa_fwd_band.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    lib.fa_fwd_band.restype = i32
    lib.fa_fwd_varlen_band.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                       i32, vp]
    lib.fa_fwd_varlen_band.restype = i32
    p64 = ctypes.POINTER(ctypes.c_int64)
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, p64, p64, p64, p64,
                                   i32, f32, i32, i32, i32, vp]
    lib.fa_fwd_strided.restype = i32
    lib.fa_fwd_varlen_strided.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, p64, p64,
                                          p64, p64, i32, f32, i32, i32, i32, vp]
    lib.fa_fwd_varlen_strided.restype = i32
    lib.fa_fwd_padded.argtypes = [vp] * 6 + [i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_fwd_padded.restype = i32
    lib.fa_bwd_band.argtypes = [vp] * 10 + [i32] * 6 + [f32, i32, i32, vp]
    lib.fa_bwd_band.restype = i32
    lib.fa_bwd_varlen_band.argtypes = [vp] * 11 + [i32] * 6 + [f32, i32, i32, vp]
    lib.fa_bwd_varlen_band.restype = i32
    lib.fa_bwd_padded.argtypes = [vp] * 11 + [i32] * 5 + [f32, i32, vp]
    lib.fa_bwd_padded.restype = i32
    lib.fa_bwd_strided.argtypes = [vp] * 10 + [i32] * 5 + [p64, i32, f32, i32, i32, i32, vp]
    lib.fa_bwd_strided.restype = i32
    lib.fa_bwd_varlen_strided.argtypes = [vp] * 11 + [i32] * 5 + [p64, i32, f32, i32, i32, i32, vp]
    lib.fa_bwd_varlen_strided.restype = i32
    lib.fa_fwd_local.argtypes = [vp] * 5 + [i32] * 5 + [f32] + [i32] * 5 + [vp]
    lib.fa_fwd_local.restype = i32
    lib.fa_bwd_local.argtypes = [vp] * 10 + [i32] * 5 + [f32] + [i32] * 5 + [vp]
    lib.fa_bwd_local.restype = i32
    lib.fa_decode.argtypes = [vp] * 6 + [i32, i32, i32, i32, i32, f32, vp, ctypes.c_size_t, vp]
    lib.fa_decode.restype = i32
    lib.fa_fwd_mx8.argtypes = [vp] * 8 + [i32] * 5 + [f32, i32, vp]
    lib.fa_fwd_mx8.restype = i32
    lib.fa_mx8_tokens_padded.argtypes = [i32]
    lib.fa_mx8_tokens_padded.restype = i32
    lib.fa_mx8_quantize_qk.argtypes = [vp, i32, ctypes.c_int64, i32, vp, vp, vp]
    lib.fa_mx8_quantize_qk.restype = i32
    lib.fa_mx8_quantize_v.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.fa_mx8_quantize_v.restype = i32
    lib.fa_decode_noalloc.argtypes = [vp] * 6 + [i32, i32, i32, i32, i32, f32, vp]
    lib.fa_decode_noalloc.restype = i32
    lib.fa_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd.argtypes = [vp] * 10 + [i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_bwd.restype = i32
    lib.fa_bwd_varlen.argtypes = [vp] * 11 + [i32, i32, i32, i32, i32, i32, f32, i32, vp]
    lib.fa_bwd_varlen.restype = i32
    lib.fa_status_string.argtypes = [i32]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_error.argtypes = []
    lib.fa_last_error.restype = ctypes.c_char_p
    lib.fa_abi_version.argtypes = []
    lib.fa_abi_version.restype = i32
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != FA_OK:
        lib = load()
        msg = lib.fa_status_string(status).decode()
        detail = lib.fa_last_error().decode()
        raise FaError(status, f"libfa: {msg}: {detail}" if detail else f"libfa: {msg}")


def raw_fa_fwd(q, k, v, o, lse, B, Nq, Nk, H, d, scale, causal, stream) -> int:
    """Pointer-level call of fa_fwd; returns the status code."""
    return load().fa_fwd(q, k, v, o, lse, B, Nq, Nk, H, d, scale, causal, stream)


def raw_fa_fwd_varlen(q, k, v, o, lse, cu, num_seqs, max_seqlen, total, H, d, scale,
                      causal, stream) -> int:
    """Pointer-level call of fa_fwd_varlen; returns the status code."""
    return load().fa_fwd_varlen(q, k, v, o, lse, cu, num_seqs, max_seqlen, total, H, d,
                                scale, causal, stream)


def raw_fa_fwd_band(q, k, v, o, lse, B, Nq, Nk, H, d, scale, window_left, window_right,
                    stream) -> int:
    """Pointer-level call of fa_fwd_band; returns the status code."""
    return load().fa_fwd_band(q, k, v, o, lse, B, Nq, Nk, H, d, scale, window_left,
                              window_right, stream)


def raw_fa_fwd_varlen_band(q, k, v, o, lse, cu, num_seqs, max_seqlen, total, H, d, scale,
                           window_left, window_right, stream) -> int:
    """Pointer-level call of fa_fwd_varlen_band; returns the status code."""
    return load().fa_fwd_varlen_band(q, k, v, o, lse, cu, num_seqs, max_seqlen, total, H, d,
                                     scale, window_left, window_right, stream)


def _int64_array(x):
    """A host int64 array holding the sequence x (None passes a null pointer)."""
    return None if x is None else (ctypes.c_int64 * len(x))(*[int(e) for e in x])


def raw_fa_fwd_strided(q, k, v, o, lse, B, Nq, Nk, H, d, q_strides, k_strides, v_strides,
                       o_strides, dtype, scale, causal, window_left, window_right, stream) -> int:
    """Pointer-level call of fa_fwd_strided (strides: sequences of 3 ints); returns the status."""
    return load().fa_fwd_strided(q, k, v, o, lse, B, Nq, Nk, H, d, _int64_array(q_strides),
                                 _int64_array(k_strides), _int64_array(v_strides),
                                 _int64_array(o_strides), dtype, scale, causal, window_left,
                                 window_right, stream)


def raw_fa_fwd_varlen_strided(q, k, v, o, lse, cu, num_seqs, max_seqlen, total, H, d, q_strides,
                              k_strides, v_strides, o_strides, dtype, scale, causal, window_left,
                              window_right, stream) -> int:
    """Pointer-level call of fa_fwd_varlen_strided (strides: sequences of 2 ints)."""
    return load().fa_fwd_varlen_strided(q, k, v, o, lse, cu, num_seqs, max_seqlen, total, H, d,
                                        _int64_array(q_strides), _int64_array(k_strides),
                                        _int64_array(v_strides), _int64_array(o_strides), dtype,
                                        scale, causal, window_left, window_right, stream)


def raw_fa_bwd_strided(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d, strides, dtype,
                       scale, causal, window_left, window_right, stream) -> int:
    """Pointer-level call of fa_bwd_strided (strides: 24 ints, the (batch, token, head)
    strides of q, k, v, o, dout, dq, dk, dv); returns the status code."""
    return load().fa_bwd_strided(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d,
                                 _int64_array(strides), dtype, scale, causal, window_left,
                                 window_right, stream)


def raw_fa_bwd_varlen_strided(q, k, v, o, dout, lse, dq, dk, dv, delta, cu, num_seqs, max_seqlen,
                              total, H, d, strides, dtype, scale, causal, window_left,
                              window_right, stream) -> int:
    """Pointer-level call of fa_bwd_varlen_strided (strides: 16 ints, the (token, head)
    strides of q, k, v, o, dout, dq, dk, dv); returns the status code."""
    return load().fa_bwd_varlen_strided(q, k, v, o, dout, lse, dq, dk, dv, delta, cu, num_seqs,
                                        max_seqlen, total, H, d, _int64_array(strides), dtype,
                                        scale, causal, window_left, window_right, stream)


def raw_fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d, dtype, scale, causal,
               stream) -> int:
    """Pointer-level call of fa_bwd; returns the status code."""
    return load().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d, dtype, scale,
                         causal, stream)


def raw_fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, delta, cu, num_seqs, max_seqlen, total, H,
                      d, dtype, scale, causal, stream) -> int:
    """Pointer-level call of fa_bwd_varlen; returns the status code."""
    return load().fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, delta, cu, num_seqs,
                                max_seqlen, total, H, d, dtype, scale, causal, stream)


def raw_fa_fwd_padded(q, k, v, o, lse, mask, B, S, H, d, dtype, scale, causal, stream) -> int:
    """Pointer-level call of fa_fwd_padded; returns the status code."""
    return load().fa_fwd_padded(q, k, v, o, lse, mask, B, S, H, d, dtype, scale, causal, stream)


def raw_fa_decode(q, k, v, o, lse, seqlens_k, B, Nk, H, d, dtype, scale, workspace,
                  workspace_bytes, stream) -> int:
    """Pointer-level call of fa_decode; returns the status code."""
    return load().fa_decode(q, k, v, o, lse, seqlens_k, B, Nk, H, d, dtype, scale, workspace,
                            workspace_bytes, stream)


def raw_fa_fwd_local(q, k, v, o, lse, B, N, H, d, dtype, scale, causal, n_global, map_w,
                     win_rows, win_cols, stream) -> int:
    """Pointer-level call of fa_fwd_local; returns the status code."""
    return load().fa_fwd_local(q, k, v, o, lse, B, N, H, d, dtype, scale, causal, n_global,
                               map_w, win_rows, win_cols, stream)


def raw_fa_bwd_local(q, k, v, o, dout, lse, dq, dk, dv, delta, B, N, H, d, dtype, scale, causal,
                     n_global, map_w, win_rows, win_cols, stream) -> int:
    """Pointer-level call of fa_bwd_local; returns the status code."""
    return load().fa_bwd_local(q, k, v, o, dout, lse, dq, dk, dv, delta, B, N, H, d, dtype, scale,
                               causal, n_global, map_w, win_rows, win_cols, stream)


def raw_fa_fwd_mx8(q, qe, k, ke, vt, vte, o, lse, B, Nq, Nk, H, d, scale, causal, stream):
    """Pointer-level call of fa_fwd_mx8; returns the status code."""
    return load().fa_fwd_mx8(q, qe, k, ke, vt, vte, o, lse, B, Nq, Nk, H, d, scale, causal, stream)


def raw_fa_mx8_quantize_qk(x, dtype, rows, d, xq, xe, stream):
    """Pointer-level call of fa_mx8_quantize_qk; returns the status code."""
    return load().fa_mx8_quantize_qk(x, dtype, rows, d, xq, xe, stream)


def raw_fa_mx8_quantize_v(v, dtype, B, N, H, d, vt, vte, stream):
    """Pointer-level call of fa_mx8_quantize_v; returns the status code."""
    return load().fa_mx8_quantize_v(v, dtype, B, N, H, d, vt, vte, stream)


def mx8_tokens_padded(N) -> int:
    return int(load().fa_mx8_tokens_padded(N))


def raw_fa_decode_noalloc(q, k, v, o, lse, seqlens_k, B, Nk, H, d, dtype, scale, stream):
    """Pointer-level call of fa_decode_noalloc; returns the status code."""
    return load().fa_decode_noalloc(q, k, v, o, lse, seqlens_k, B, Nk, H, d, dtype, scale, stream)


FA_DECODE_NOALLOC_SCRATCH_BYTES = 8 << 20   # as include/fa.h


def decode_workspace_bytes(B, Nk, H, d) -> int:
    return int(load().fa_decode_workspace_bytes(B, Nk, H, d))


def raw_fa_bwd_band(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d, dtype, scale,
                    window_left, window_right, stream) -> int:
    """Pointer-level call of fa_bwd_band; returns the status code."""
    return load().fa_bwd_band(q, k, v, o, dout, lse, dq, dk, dv, delta, B, Nq, Nk, H, d, dtype,
                              scale, window_left, window_right, stream)


def raw_fa_bwd_varlen_band(q, k, v, o, dout, lse, dq, dk, dv, delta, cu, num_seqs, max_seqlen,
                           total, H, d, dtype, scale, window_left, window_right, stream) -> int:
    """Pointer-level call of fa_bwd_varlen_band; returns the status code."""
    return load().fa_bwd_varlen_band(q, k, v, o, dout, lse, dq, dk, dv, delta, cu, num_seqs,
                                     max_seqlen, total, H, d, dtype, scale, window_left,
                                     window_right, stream)


def raw_fa_bwd_padded(q, k, v, o, dout, lse, dq, dk, dv, delta, mask, B, S, H, d, dtype, scale,
                      causal, stream) -> int:
    """Pointer-level call of fa_bwd_padded; returns the status code."""
    return load().fa_bwd_padded(q, k, v, o, dout, lse, dq, dk, dv, delta, mask, B, S, H, d,
                                dtype, scale, causal, stream)
