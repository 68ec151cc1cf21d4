"""FP8 block-scaled attention forward, in float64: quantisation and definition.

TEST INFRASTRUCTURE ONLY (see the package docstring). Parity: pinned by the
CPU tests (E4M3 rounding against torch's float8_e4m3fn conversion and against
the format's own grid, closed forms of the block scaling, exact power-of-two
invariances, planted mistakes).

Sources (page titles and sections):
  * "FlashAttention/zh" (marovi.ai wiki), section 變體與後續版本: the
    FlashAttention-3 generation runs the attention in FP8 with block
    quantisation (block scaling) on the newest matrix units.
  * same page, section 局限性: low-precision formats such as FP8 need careful
    scaling to keep the accuracy.
  * same page, section 為何標準注意力運行緩慢: the attention itself,
    softmax(scale q k^T) v, and L = m + ln l (attention.py).

Readings where the pages are silent (they name FP8 and block scaling only):
  * The block-scaled format is the OCP microscaling (MX) one: blocks of 32
    consecutive elements share one power-of-two scale 2^e (an E8M0 exponent,
    e in [-127, 127]); the elements are FP8 E4M3 in its "fn" variant (1 sign,
    4 exponent bits with bias 7, 3 mantissa bits, no infinities, largest
    magnitude 448, subnormals down to 2^-9).
  * A block's exponent is floor(log2(amax)) - 8, 8 being the exponent of
    E4M3's largest power of two (clamped to [-127, 127]; an all-zero block
    gets -127). Elements are x / 2^e rounded to nearest-even on the E4M3 grid
    and saturated to +-448 (the quotient of the block maximum lies in
    [256, 512), so values above 448 are clamped rather than lost).
  * A block holding an infinity or a NaN has no finite scale: as in the OCP
    MX format, its exponent byte is the NaN code 0xFF (exponent 128 here) and
    its elements are stored as 0; it dequantises to NaN.
  * Q and K are blocked along the head dimension d (the contraction of
    Q K^T), V along the tokens (the contraction of P V), so V is held
    transposed, (d, tokens), with its token count padded with zeros to a
    multiple of 64.
  * What is computed from the quantised operands is the plain definition
    on their values: O and L are attention.attention applied to the
    dequantised Q, K and V. (A kernel also rounds P to FP8 before P V; that
    is an internal rounding like the 16-bit P of the other kernels, which
    the tests bound instead of modelling.)
"""
from __future__ import annotations

import numpy as np

from .attention import attention

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9
E4M3_EMAX = 8             # exponent of the largest power of two in E4M3
MX_BLOCK = 32             # elements per shared scale
E8M0_MIN, E8M0_MAX = -127, 127
E8M0_NAN = 128            # exponent of the NaN scale byte 0xFF
V_TOKEN_PAD = 64          # token padding of the transposed V


def _rne(x: np.ndarray) -> np.ndarray:
    """Round to the nearest integer, ties to even."""
    return np.rint(x)


def e4m3_round(x) -> np.ndarray:
    """Values of x rounded to nearest-even on the E4M3 (fn) grid, saturated to
    +-448. Returns float64 values (all exactly representable in E4M3)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # quantum of the binade of |x| (3 mantissa bits); subnormal range below 2^-6
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, -6, E4M3_EMAX)
    quantum = np.where(a < E4M3_MIN_NORMAL, E4M3_SUBNORMAL_STEP, 2.0 ** (e - 3))
    r = _rne(a / quantum) * quantum
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def e4m3_grid() -> np.ndarray:
    """Every finite E4M3 (fn) value, decoded from the bit fields."""
    vals = []
    for s in (0, 1):
        for e in range(16):
            for m in range(8):
                if e == 15 and m == 7:
                    continue                       # the NaN code
                v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
                vals.append(-v if s else v)
    return np.array(sorted(set(vals)))


def mx_exponent(amax) -> np.ndarray:
    """Shared E8M0 exponent of blocks with the given absolute maxima (NaN or
    infinite maxima give the NaN scale's exponent 128)."""
    amax = np.asarray(amax, dtype=np.float64)
    finite = np.isfinite(amax)
    safe = np.where(finite & (amax > 0), amax, 1.0)
    e = np.floor(np.log2(safe)) - E4M3_EMAX
    e = np.where(amax > 0, e, E8M0_MIN)
    e = np.clip(e, E8M0_MIN, E8M0_MAX)
    return np.where(finite, e, E8M0_NAN).astype(np.int64)


def mx_quantize(x, axis: int = -1):
    """Blocks of 32 consecutive elements along `axis` (its length a multiple of
    32): returns (values on the E4M3 grid, exponents), the exponents with the
    blocked axis shortened 32-fold. x equals about values * 2^exponent."""
    x = np.asarray(x, dtype=np.float64)
    xm = np.moveaxis(x, axis, -1)
    n = xm.shape[-1]
    if n % MX_BLOCK:
        raise ValueError("the blocked axis must be a multiple of 32 long")
    blocks = xm.reshape(*xm.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    bad = ~np.all(np.isfinite(blocks), axis=-1)
    amax = np.where(bad, np.inf, np.max(np.abs(np.where(np.isfinite(blocks), blocks, 0.0)), axis=-1))
    e = mx_exponent(amax)
    with np.errstate(over="ignore", invalid="ignore"):
        q = e4m3_round(blocks / np.ldexp(1.0, np.where(bad, 0, e))[..., None])
    q = np.where(bad[..., None], 0.0, q)
    return (np.moveaxis(q.reshape(xm.shape), -1, axis),
            np.moveaxis(e, -1, axis))


def mx_dequantize(q, e, axis: int = -1) -> np.ndarray:
    """Inverse of mx_quantize's layout: q * 2^e with each exponent over its 32 elements."""
    q = np.asarray(q, dtype=np.float64)
    e = np.asarray(e)
    scale = np.where(e == E8M0_NAN, np.nan, np.ldexp(1.0, np.where(e == E8M0_NAN, 0, e)))
    return q * np.repeat(scale, MX_BLOCK, axis=axis)


def quantize_qk(x):
    """Q or K (..., d) -> values and exponents (..., d / 32): blocks along d."""
    return mx_quantize(x, axis=-1)


def quantize_v_transposed(v):
    """V (B, N, H, d) -> V^T values (B, H, d, Np) and exponents (B, H, d, Np / 32),
    Np = N rounded up to a multiple of 64, the padding tokens zero."""
    v = np.asarray(v, dtype=np.float64)
    B, N, H, d = v.shape
    Np = -(-N // V_TOKEN_PAD) * V_TOKEN_PAD
    vt = np.zeros((B, H, d, Np))
    vt[..., :N] = v.transpose(0, 2, 3, 1)
    return mx_quantize(vt, axis=-1)


def attention_mx8(q8, qe, k8, ke, vt8, vte, scale: float, causal: bool = False):
    """Dense batch from MX-FP8 operands: q8/k8 (B, N, H, d) with exponents
    (B, N, H, d/32), vt8 (B, H, d, Np) with exponents (B, H, d, Np/32).
    Returns O (B, Nq, H, d) and L (B, H, Nq), float64: the definition on the
    dequantised values."""
    Q = mx_dequantize(q8, qe, axis=-1)
    K = mx_dequantize(k8, ke, axis=-1)
    VT = mx_dequantize(vt8, vte, axis=-1)
    B, Nq, H, d = Q.shape
    Nk = K.shape[1]
    O = np.empty((B, Nq, H, VT.shape[2]))
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            O[b, :, h], L[b, h] = attention(Q[b, :, h], K[b, :, h], VT[b, h, :, :Nk].T, scale,
                                            causal)
    return O, L
