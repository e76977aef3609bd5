"""CPU fp64 oracle for block-diagonal causal attention over packed users.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg use it.  It shares no code with the HIP
library in ``varlen_causal_attention_amd`` and imports nothing from it.

Contents:
  attention.varlen_causal_attention   per-user dense softmax(scale*QK^T + causal mask) V
  attention.varlen_causal_attention_rows  the same, one selected query row at a time
  attention.varlen_causal_attention_backward  dL/dqkv given dL/dout (derivative of the definition)
  attention.varlen_causal_attention_backward_magnitude  each gradient element with every term
                                      of its expansion taken in absolute value (for error bounds)
  attention.varlen_causal_attention_lse   each row's log-sum-exp of its scaled causal scores
  attention.hstu_mask, varlen_attention_masked  the HSTU-style mask variants (context, candidate
                                      groups, sliding / bidirectional window)
  attention.dense_masked_attention    whole packed stream as one T x T problem with the
                                      block-diagonal causal mask built from the offsets
  attention.block_diagonal_causal_mask
  worklist.reference_worklist         the segment scheduler's (user, q-tile) order
  layer.layer_norm, layer.linear, layer.attention_block  the layer's attention sub-block around
                                      the op (LayerNorm -> Linear_qkv -> attention -> Linear_out + residual)

Every function is pinned by ``tests/test_oracle.py`` to something other than
itself (brute force, closed forms, invariants, a library routine on the
single-segment special case, hand-derived fixtures under ``tests/golden/``).
"""
from .attention import (  # noqa: F401
    block_diagonal_causal_mask,
    dense_masked_attention,
    hstu_mask,
    split_qkv_head,
    varlen_attention_masked,
    varlen_causal_attention,
    varlen_causal_attention_backward,
    varlen_causal_attention_backward_magnitude,
    varlen_causal_attention_lse,
    varlen_causal_attention_rows,
)
from .layer import attention_block, layer_norm, linear  # noqa: F401
from .worklist import reference_worklist, tiles_per_user  # noqa: F401
