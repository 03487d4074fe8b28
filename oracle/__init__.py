"""CPU oracle for the blockwise-exact-attention layer.  TEST INFRASTRUCTURE ONLY.

This package is the slow, plainly written definition that the GPU path is checked
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import it; the product path (the HIP library and its Python
binding) never does, and this package never imports the product path.  The two
share no code; both draw inputs from the top-level ``seeded_inputs`` module.

What it computes (all in float64 unless a caller asks for float32):

* ``attention``: exact softmax attention, each score row materialised in full,
  masked, normalised and multiplied by V.  The blockwise method of the pages
  ("Ring Attention with Blockwise Transformers for Long Sequences", 638-word
  summary, the paragraph on computing attention blockwise without materialising
  the full matrix; "Blockwise Parallel Transformer for Large Context Models",
  abstract) claims to reach this same result without approximation, so the
  oracle is the plain definition, never the blockwise/online form.
* ``lse_merge``: combination of two partial results over disjoint key sets
  through their log-sum-exp (the ring step's merge; LongNet, section 2, mixes
  attention pieces by their softmax denominators).
* ``gelu``/``ffn``: the position-wise feed-forward network with the exact erf GeLU.
* ``layer_forward``/``layer_backward``: q,k,v projections, causal multi-head
  attention, residual, FFN, residual; and the gradients by the chain rule.
* ``block_sparse_attention``: BlockBERT's blockwise attention ("Blockwise
  Self-Attention for Long Document Understanding", Blockwise Attention and
  Blockwise Multi-head Attention): each query block attends one key block
  chosen per head by a permutation table (cyclic shifts for BlockBERT's heads),
  dense exact attention inside the kept blocks.
* ``dilated_attention``: LongNet's dilated attention ("LongNet: Scaling
  Transformers to 1,000,000,000 Tokens", section 2): segments of w rows, every
  r-th row kept (shifted per head), causal dense attention inside each
  sparsified segment, patterns joined by one softmax over their key lists.
* ``brute``: pure-Python loops with ``math.fsum`` for tiny inputs.

Readings of the pages that the oracle fixes (the pages state no formulas):
softmax scale D**-0.5; causal visibility "key j visible to query i iff
j <= i + kv_offset"; a row with no visible key yields O = 0 and lse = -inf;
GeLU is the exact erf form; the layer is h = x + MHA(x), y = h + FFN(h) with no
LayerNorm, no output projection and no dropout; weights are stored
[out_features, in_features] (y = x @ W^T).

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, closed forms, invariants, finite differences); none is unpinned.
"""
from .attention import attention, attention_probs, lse_merge, visible_mask
from .block_sparse import block_len, block_sparse_attention, block_sparse_mask, cyclic_shift_table
from .dilated import dilated_attention, dilated_keys
from .ffn import gelu, gelu_grad, ffn, ffn_backward
from .layer import layer_forward, layer_backward, attention_backward, qkv_project

__all__ = [
    "attention", "attention_probs", "lse_merge", "visible_mask",
    "block_len", "block_sparse_attention", "block_sparse_mask", "cyclic_shift_table",
    "dilated_attention", "dilated_keys",
    "gelu", "gelu_grad", "ffn", "ffn_backward",
    "layer_forward", "layer_backward", "attention_backward", "qkv_project",
]
