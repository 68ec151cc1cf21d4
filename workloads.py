"""Seeded synthetic workloads for the attention forward pass.

This module only makes inputs. It holds none of the attention arithmetic, and
it is the one piece of code that both the CPU oracle's tests and the GPU path
read from. Everything is numpy, so importing it never touches a GPU.

Workloads (shapes follow the pages' models):
  tiny        B=1  H=2  N=128  d=64   non-causal            seed 1
  det1600     B=16 H=4  N=1600 d=32   non-causal (40x40 map) seed 2
  det400      B=16 H=4  N=400  d=32   non-causal (20x20 map) seed 22
  vit         B=32 H=25 N=1025 d=128  non-causal, Q,K RMS-normalised  seed 3
  varlen      64 sequences, lengths ~U{256..1025}, H=25 d=128, non-causal  seed 4
  prefill8k   B=1  H=32 N=8192 d=128  causal                 seed 5
  prefill2k   B=4  H=32 N=2048 d=128  causal                 seed 55
  band8k      B=1  H=32 N=8192 d=128  band (2047, 0): each query sees itself
              and the 2047 keys before it                    seed 6
  decode8k    B=16 H=32 d=128: one query per (batch, head), 8192-key cache   seed 8
  decode32k   B=4  H=32 d=128: one query per (batch, head), 32768-key cache  seed 9
              (q drawn first with the seed, then K and V of the cache)
  prefill8k_d256  B=1 H=16 N=8192 d=256 causal (prefill8k's FLOPs at head dim 256)  seed 7
  vitpad      the vit batch with a key padding mask: row b keeps its first
              n_b ~ U{256..1025} tokens (lengths seed 10), the rest is padding
  band8k_d256 B=1 H=16 N=8192 d=256 band (2047, 0)           seed 12
  detlocal    B=16 H=4 N=1608 d=32: 8 global anchor tokens + the 40x40 map,
              5x5 local window (the detector's local + global mix)  seed 11

The detector token counts (40x40, 20x20 and the 4-head, 32-wide head split)
come from "YOLOv12官版镜像集成Flash Attention v2，提速原理浅析" (sections 2.1 and
2.3). The ViT shape (448 px / 14 px patches = 32x32 patches + CLS = 1025
tokens, 25 heads of hidden 3200, bf16, RMSNorm on Q and K) comes from
"InternViT-6B-448px-V1-2 如何加速注意力计算" (sections 先认识模型 and
模型侧的启用与降级机制).

Recipe for every draw: numpy.random.default_rng(seed); float32
standard_normal in C order, drawn in the order lengths (varlen only) -> Q ->
K -> V; then rounded to bfloat16 with round-to-nearest-even. For "vit", Q and
K are RMS-normalised over d in float32 (eps 1e-6, unit weight) before the
rounding; V is not. fp16 inputs (dtype "f16") take the same float32 draws
rounded to IEEE binary16 (round to nearest, ties to even) instead.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


# ---------------------------------------------------------------------------
# bfloat16 <-> float32, as bit patterns (uint16), by integer arithmetic.
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaN inputs map to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = 0x7FC0
    return rounded


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rms_normalise(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(mean(x^2 over the last axis) + eps), in float32, weight 1."""
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(eps))).astype(np.float32)


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Dense:
    """Equal-length batch: Q,K,V,O laid out (B, N, H, d); L laid out (B, H, N)."""
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    rms_qk: bool = False
    window: tuple | None = None   # banded mask (left, right), None = unbounded side
    pad_seed: int | None = None   # key padding mask: right padding to lengths
                                  # drawn U{256..N} with this seed
    local: tuple | None = None    # (n_global, map_w, win_rows, win_cols): anchors
                                  # + a local window on the token map

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def pad_lengths(self) -> np.ndarray:
        """Valid tokens per batch row of a padded workload."""
        return varlen_lengths(self.B, 256, self.N, self.pad_seed)

    def flops(self) -> float:
        """Useful FLOPs: 4 d per (query, visible key) pair, the causal count
        taken as N^2 / 2, the band's as its exact pair count, a padded batch's
        over its valid tokens only."""
        if self.pad_seed is not None:
            n = self.pad_lengths().astype(np.float64)
            f = 4.0 * float(np.sum(n * n)) * self.d * self.H
            return f / 2 if self.causal else f
        if self.window is not None:
            return 4.0 * band_pairs(self.N, self.N, self.window) * self.d * self.H * self.B
        if self.local is not None:
            return 4.0 * local_pairs_count(self.N, *self.local, self.causal) * self.d * self.H * self.B
        f = 4.0 * self.N * self.N * self.d * self.H * self.B
        return f / 2 if self.causal else f

    def bytes_compulsory(self) -> int:
        qkvo = 4 * self.B * self.N * self.H * self.d * 2
        return qkvo + self.B * self.H * self.N * 4


@dataclasses.dataclass(frozen=True)
class Varlen:
    """Packed unpadded batch: Q,K,V,O laid out (total, H, d); L laid out (H, total)."""
    name: str
    num_seqs: int
    len_lo: int
    len_hi: int          # inclusive
    H: int
    d: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclasses.dataclass(frozen=True)
class Decode:
    """One query per (batch, head) against a KV cache: q, o (B, 1, H, d),
    k, v (B, Nk, H, d), every cache entry valid."""
    name: str
    B: int
    H: int
    Nk: int
    d: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def bytes_compulsory(self) -> int:
        """HBM bytes a decode step must move: K and V once, q and o, L."""
        return 2 * self.B * self.Nk * self.H * self.d * 2 + 2 * self.B * self.H * self.d * 2 \
            + self.B * self.H * 4

    def flops(self) -> float:
        return 4.0 * self.B * self.H * self.Nk * self.d


WORKLOADS = {
    "tiny": Dense("tiny", B=1, H=2, N=128, d=64, causal=False, seed=1),
    "det1600": Dense("det1600", B=16, H=4, N=1600, d=32, causal=False, seed=2),
    "det400": Dense("det400", B=16, H=4, N=400, d=32, causal=False, seed=22),
    "vit": Dense("vit", B=32, H=25, N=1025, d=128, causal=False, seed=3, rms_qk=True),
    "varlen": Varlen("varlen", num_seqs=64, len_lo=256, len_hi=1025, H=25, d=128,
                     causal=False, seed=4),
    "prefill8k": Dense("prefill8k", B=1, H=32, N=8192, d=128, causal=True, seed=5),
    "prefill2k": Dense("prefill2k", B=4, H=32, N=2048, d=128, causal=True, seed=55),
    "band8k": Dense("band8k", B=1, H=32, N=8192, d=128, causal=False, seed=6,
                    window=(2047, 0)),
    "detlocal": Dense("detlocal", B=16, H=4, N=1608, d=32, causal=False, seed=11,
                      local=(8, 40, 2, 2)),
    "band8k_d256": Dense("band8k_d256", B=1, H=16, N=8192, d=256, causal=False, seed=12,
                         window=(2047, 0)),
    "prefill8k_d256": Dense("prefill8k_d256", B=1, H=16, N=8192, d=256, causal=True, seed=7),
    "decode8k": Decode("decode8k", B=16, H=32, Nk=8192, d=128, seed=8),
    "decode32k": Decode("decode32k", B=4, H=32, Nk=32768, d=128, seed=9),
    "vitpad": Dense("vitpad", B=32, H=25, N=1025, d=128, causal=False, seed=3, rms_qk=True,
                    pad_seed=10),
}


def band_pairs(Nq: int, Nk: int, window) -> int:
    """Number of (query, key) pairs a banded mask leaves visible, for FLOP
    accounting: row i sees keys max(0, i + Nk - Nq - left) ..
    min(Nk - 1, i + Nk - Nq + right), None meaning no bound on that side."""
    left, right = window
    i = np.arange(Nq, dtype=np.int64) + (Nk - Nq)
    lo = np.zeros_like(i) if left is None else np.maximum(0, i - left)
    hi = np.full_like(i, Nk - 1) if right is None else np.minimum(Nk - 1, i + right)
    return int(np.maximum(0, hi - lo + 1).sum())


def local_pairs_count(N: int, n_global: int, map_w: int, win_rows: int, win_cols: int,
                      causal: bool = False) -> int:
    """Number of (query, key) pairs the local-window + anchor pattern leaves
    visible, for FLOP accounting: an anchor query sees every key (up to itself
    when causal); a map query sees the anchors and the map tokens within
    (win_rows, win_cols) of its own map position."""
    G = min(n_global, N)
    t = np.arange(N, dtype=np.int64)
    total = int(np.sum(t[:G] + 1)) if causal else G * N
    m = np.arange(N - G, dtype=np.int64)
    row, col = m // map_w, m % map_w
    for i in range(N - G):
        near = (np.abs(row - row[i]) <= win_rows) & (np.abs(col - col[i]) <= win_cols)
        if causal:
            near &= m <= i
        total += G + int(np.count_nonzero(near))
    return total


def _draw(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's conversion: round to
    nearest, ties to even); returns the 16-bit patterns as uint16."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen binary16 bit patterns (uint16) to float32 exactly."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    raise ValueError(f"dtype must be 'bf16' or 'f16' (got {dtype!r})")


def make_dense(B: int, N: int, H: int, d: int, seed: int, rms_qk: bool = False,
               Nk: int | None = None, dtype: str = "bf16"):
    """Return (q, k, v) as uint16 bit patterns of dtype ('bf16' or 'f16'),
    q (B,N,H,d), k/v (B,Nk,H,d)."""
    Nk = N if Nk is None else Nk
    rng = np.random.default_rng(seed)
    q = _draw(rng, (B, N, H, d))
    k = _draw(rng, (B, Nk, H, d))
    v = _draw(rng, (B, Nk, H, d))
    if rms_qk:
        q = _rms_normalise(q)
        k = _rms_normalise(k)
    return _round(q, dtype), _round(k, dtype), _round(v, dtype)


def varlen_lengths(num_seqs: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Integer lengths drawn uniformly from [lo, hi] inclusive (the first draw)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=num_seqs).astype(np.int64)


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    """Prefix sums [0, n0, n0+n1, ...] as int32."""
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    assert cu[-1] < 2**31
    return cu.astype(np.int32)


def make_varlen(lengths, H: int, d: int, seed: int, rng: np.random.Generator | None = None,
                dtype: str = "bf16"):
    """Return (q, k, v, cu_seqlens): q/k/v (total,H,d) bits of dtype, cu int32."""
    cu = cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    if rng is None:
        rng = np.random.default_rng(seed)
    q = _draw(rng, (total, H, d))
    k = _draw(rng, (total, H, d))
    v = _draw(rng, (total, H, d))
    return _round(q, dtype), _round(k, dtype), _round(v, dtype), cu


def make_workload(name: str):
    """Materialise a named workload.

    Dense -> dict(q, k, v, scale, causal, shape=(B,N,H,d)).
    Varlen -> dict(q, k, v, cu_seqlens, max_seqlen, scale, causal, lengths).
    """
    w = WORKLOADS[name]
    if isinstance(w, Decode):
        rng = np.random.default_rng(w.seed)
        q = _round(_draw(rng, (w.B, 1, w.H, w.d)), "bf16")
        k = _round(_draw(rng, (w.B, w.Nk, w.H, w.d)), "bf16")
        v = _round(_draw(rng, (w.B, w.Nk, w.H, w.d)), "bf16")
        return dict(q=q, k=k, v=v, scale=w.scale, spec=w)
    if isinstance(w, Dense):
        q, k, v = make_dense(w.B, w.N, w.H, w.d, w.seed, rms_qk=w.rms_qk)
        out = dict(q=q, k=k, v=v, scale=w.scale, causal=w.causal,
                   shape=(w.B, w.N, w.H, w.d), spec=w)
        if w.pad_seed is not None:
            n = w.pad_lengths()
            out["mask"] = (np.arange(w.N)[None, :] < n[:, None]).astype(np.uint8)
        return out
    rng = np.random.default_rng(w.seed)
    lengths = rng.integers(w.len_lo, w.len_hi + 1, size=w.num_seqs).astype(np.int64)
    q, k, v, cu = make_varlen(lengths, w.H, w.d, w.seed, rng=rng)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, max_seqlen=int(lengths.max()),
                scale=w.scale, causal=w.causal, lengths=lengths, spec=w)


def varlen_flops(lengths, H: int, d: int, causal: bool) -> float:
    """4 * d * H * sum(n_i^2), halved when causal."""
    s = float(np.sum(np.asarray(lengths, dtype=np.float64) ** 2))
    f = 4.0 * d * H * s
    return f / 2 if causal else f
