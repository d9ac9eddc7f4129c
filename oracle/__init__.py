"""fp64 CPU oracle for the fused attention forward.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports this
package, and this package imports nothing from the product.

``attn_fwd_oracle`` runs the plain C implementation in ``attn_oracle.c`` (the
textbook definition in fp64: scores, two-pass safe softmax over a materialised
row, then P V; see that file's header for the citations).  ``build_oracle``
compiles it with gcc.  ``attn_fwd_oracle(..., key_range=(k0, k1))`` gives the
partial state of each row over a key subset, and ``merge_partials_oracle``
(numpy fp64) combines such partial states with the online-softmax update.
``attn_bwd_oracle`` gives the gradients of sum(dO * O) through the same
definition (chain rule, softmax Jacobian).  ``attn_decode_paged_oracle``
gathers each sequence's keys from a paged K/V cache through its block table
(``gather_paged_oracle``) and applies the dense forward to them.
"""
from .oracle import (attn_bwd_oracle, attn_decode_paged_oracle,  # noqa: F401
                     attn_fwd_oracle, build_oracle, gather_paged_oracle,
                     merge_partials_oracle, oracle_lib_path)
