"""CPU oracle for streaming exact attention: test infrastructure, not product.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import anything from this package; the HIP library never calls it and it never
calls the HIP library.  It is written to be read against the pages, not to be
fast:

* ``attention`` — the plain definition of scaled dot-product attention with an
  additive bias and a visibility rule, materialising the whole score matrix
  per (batch, head) in float64 (the quantity the online-softmax kernels of
  "StreamAttention: Fused Online Softmax Attention", section "Kernel Design
  (Fused Online Softmax)", and of the "Attention API" page, function
  ``online_softmax_attention``, compute without materialising it).
* ``online_attention`` — the pages' streaming recurrence (running max, rescaled
  numerator and denominator, one key block at a time) in float64, kept to show
  that the recurrence reaches the definition.
* ``attention_bwd`` — the gradients dq, dk, dv of the attention output by
  their definition (the single-sweep backward of the "StreamAttention" page,
  "Recent Updates"; "flash-attn-volta" page, "Backward correctness").
* ``block_sparse_attention`` — attention restricted to selected (query block,
  key block) pairs, the execution step of the "Stem" page (section 2.3),
  written as its pseudo-sparse fallback: the block selection expanded into an
  element mask, then the definition above.
* ``attention_ext`` — ``attention`` with an additive float mask and dropout
  by a Philox4x32-10 rule ("StreamAttention" page, "Recent Updates" and
  "API Reference"); the generator is ``philox``, written from its published
  definition.
* ``merge_states`` — the log-sum-exp weighted combination of partial states
  ("StreamAttention" page, "Engine Direction" and "Distributed and
  Long-Context Variants").
* ``brute`` — a scalar pure-Python version for tiny inputs.

Every function here is pinned by tests that do not go through the oracle's own
code path (closed forms, invariants, a library routine, brute force); none of
them is "parity unpinned".
"""
from .attention import (SPARSE_BLOCK, attention, attention_bwd, attention_ext,
                        block_sparse_attention, online_attention, merge_states,
                        alibi_bias, visible)
from . import brute, philox

__all__ = ["SPARSE_BLOCK", "attention", "attention_bwd", "attention_ext",
           "block_sparse_attention", "philox",
           "online_attention", "merge_states",
           "alibi_bias", "visible", "brute"]
