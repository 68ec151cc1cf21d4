"""CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check in the repository's
entry module and the CPU-baseline leg of the benchmark may import or call
anything here. The product path (the HIP library and its Python binding)
never imports this package, and this package imports nothing from the
product path.

Contents:
  attention.py  the plain definition of exact scaled-dot-product attention,
                with the score matrix materialised, in float64.
  tiled.py      a blockwise online-softmax route to the same result (partial
                summaries of key blocks, combined in any grouping), in
                float64, used only to cross-check the definition.
  backward.py   the gradients dQ, dK, dV of the definition (chain rule through
                the softmax), with P materialised, in float64.
  padding.py    attention over a padded batch with a key padding mask: remove
                the padding, attend, put the result back (zeros at padding).
  local.py      attention with a local window on a token map plus global
                anchor tokens, the score mask built from map coordinates, and
                its gradients.
  fp8.py        FP8 E4M3 rounding, MX block scaling (32 elements sharing a
                power-of-two scale) and attention on the dequantised values.
"""
from .attention import (attention, attention_probs, attention_dense,
                        attention_varlen, ORACLE_DTYPE)
from .backward import (attention_backward, attention_backward_dense,
                       attention_backward_padded, attention_backward_varlen)
from .local import (attention_local, attention_local_backward, attention_local_backward_dense,
                    attention_local_dense, local_pairs, local_visible)
from .padding import attention_padded
from .tiled import attention_tiled

__all__ = ["attention", "attention_probs", "attention_dense", "attention_varlen",
           "attention_tiled", "attention_backward", "attention_backward_dense",
           "attention_backward_varlen", "attention_backward_padded", "attention_padded",
           "attention_local", "attention_local_dense", "attention_local_backward",
           "attention_local_backward_dense", "local_pairs", "local_visible",
           "ORACLE_DTYPE"]
