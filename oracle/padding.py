"""Attention over a padded batch with a key padding mask, float64.

TEST INFRASTRUCTURE ONLY (see the package docstring). Pinned by the CPU tests.

Source: "InternViT-6B-448px-V1-2 如何加速注意力计算", section
FlashAttention 封装类三条执行路径 (带掩码路径): with a key_padding_mask, the
padded positions are removed from the tensors (unpad_input), attention runs
on the valid tokens only, and the result is put back into the padded shape
(pad_input); padding takes no part in the computation.

Readings where the page is silent:
  * mask[b, s] != 0 marks a valid token, 0 a padding position; the mask is
    shared by queries and keys (self-attention over one padded sequence).
  * Causal attention applies to the sequence after the padding is removed,
    which is the same as query i seeing valid keys j <= i in the padded
    positions (removing positions keeps their order).
  * pad_input puts zeros at padding positions: O = 0 there. The page says
    nothing of L at padding positions; they see no key in the removed
    computation, so L = ln 0 = -inf, as for any row with no visible key.
"""
from __future__ import annotations

import numpy as np

from .attention import ORACLE_DTYPE, attention


def attention_padded(q, k, v, mask, scale: float, causal: bool = False):
    """q, k, v (B, S, H, d); mask (B, S). Returns O (B, S, H, d) and L (B, H, S)."""
    q, k, v = (np.asarray(x, dtype=ORACLE_DTYPE) for x in (q, k, v))
    mask = np.asarray(mask)
    B, S, H, _ = q.shape
    O = np.zeros((B, S, H, v.shape[3]), dtype=ORACLE_DTYPE)
    L = np.full((B, H, S), -np.inf, dtype=ORACLE_DTYPE)
    for b in range(B):
        idx = np.nonzero(mask[b])[0]            # unpad: the valid positions, in order
        if idx.size == 0:
            continue
        for h in range(H):
            o, lse = attention(q[b, idx, h], k[b, idx, h], v[b, idx, h], scale, causal)
            O[b, idx, h] = o                    # pad: scatter back, zeros elsewhere
            L[b, h, idx] = lse
    return O, L
