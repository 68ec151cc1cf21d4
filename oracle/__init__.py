"""CPU oracle for the attention forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check in the repository's
entry module and the CPU-baseline leg of the benchmark may import or call
anything here. The product path (the HIP library and its Python binding)
never imports this package, and this package imports nothing from the
product path.

Contents:
  attention.py  the plain definition of exact scaled-dot-product attention,
                with the score matrix materialised, in float64.
  tiled.py      the blockwise online-softmax forward exactly as the pages lay
                it out, in float64, used only to cross-check the definition.
"""
from .attention import (attention, attention_probs, attention_dense,
                        attention_varlen, ORACLE_DTYPE)
from .tiled import attention_tiled

__all__ = ["attention", "attention_probs", "attention_dense", "attention_varlen",
           "attention_tiled", "ORACLE_DTYPE"]
