"""CPU oracle for the speculative-tree verify step -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import, call or execute anything in this package.  The GPU
library never routes through it, and it shares no code with the GPU path:
it imports nothing from ``tree_attention_verify_parent_amd``.

What is computed, and where the pages say so:

  * The target model checks the draft's proposed tokens in parallel
    (Aurora, chernovdev.ru and everytik.com mirrors, section 2 "serve-to-train
    flywheel", description of the inference server; Runtime Draft Model
    Training, moreh.io, "Overview").
  * A custom attention mask that follows the causal structure of the
    speculative tree lets all branches go through one batched pass (Aurora,
    section 2, closing paragraph on tree attention).
  * Acceptance length is the number of draft tokens the target accepts in one
    verification step (Runtime Draft Model Training, "Evaluation").
  * The accepted and rejected outcomes of each verification are what the
    serving engine streams on (Aurora, section 2): the commit step keeps the
    accepted path's K/V rows and labels every node.
  * The draft model is trained on all accepted and rejected branches in one
    batched forward and backward pass under the same tree mask (Aurora,
    section 2, closing paragraph): the attention's backward pass.
  * Numeric precision (FP8 / FP4) is part of what decides serving speed
    (Aurora, section 1): the fp8-arithmetic attention quantizes each query
    row to e4m3 (``fp8.py``).

Everything is plain: explicit parent-pointer walks, a dense boolean mask,
naive softmax in float64, a linear argmax, a recursive accept walk.

Pins: every function here is checked in ``tests/test_oracle_*.py`` against
closed forms, brute force and independent library routines.  Parity
beyond the stated tolerance for attention is unpinned where the GPU's
internal rounding (bf16 probabilities before the PV product, hardware exp2)
legitimately differs; see each test's docstring.
"""
from .tree import ancestors, build_masks, accept_walk, children_of
from .attention import (bf16_bits_to_f64, e4m3_decode_table, decode_e4m3, e2m1_decode_table,
                        decode_e2m1_packed, dense_tree_mask, tree_attention_bh, tree_attention)
from .argmax import vocab_argmax
from .step import verify_step
from .commit import commit_accepted, LABEL_ACCEPTED, LABEL_REJECTED, LABEL_ROOT
from .paged import gather_pages
from .attention_bwd import tree_attention_backward
from .fp8 import encode_e4m3, quantize_rows_e4m3, dequantize_rows_e4m3

__all__ = [
    "ancestors", "build_masks", "accept_walk", "children_of",
    "bf16_bits_to_f64", "e4m3_decode_table", "decode_e4m3", "e2m1_decode_table", "decode_e2m1_packed",
    "dense_tree_mask",
    "tree_attention_bh", "tree_attention", "vocab_argmax", "verify_step",
    "commit_accepted", "LABEL_ACCEPTED", "LABEL_REJECTED", "LABEL_ROOT", "gather_pages",
    "tree_attention_backward", "encode_e4m3", "quantize_rows_e4m3", "dequantize_rows_e4m3",
]
