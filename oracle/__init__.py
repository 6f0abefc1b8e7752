"""Float64 CPU oracle for tiled online-softmax attention.

TEST INFRASTRUCTURE ONLY. This package is the slow, plain, obviously
correct reference that the HIP path is checked against. Only the test
suite (``tests/``), ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it. The product path (the C-ABI library
and its Python binding) never imports, calls or links anything here, and
nothing here imports the product path: the two share no code.

Sources (the four web pages this method is described on):

* "Naive attention and the online softmax" (mlinterviewnotes.com, inference
  course 03-01): the textbook materialised attention, safe softmax, the
  online recurrence and its proof, the log-sum-exp summary, the merge of two
  states, the empty-state guard, scale-before-multiply.
* "The Online Softmax Recurrence" (inferenceinterviews.com): the (m, l, a)
  state, the state/merge pair with empty branches, the worked example.
* "Decode attention: FlashDecoding, split-K, paged kernels"
  (mlinterviewnotes.com, inference course 03-03): split-KV partials,
  the reduction of segments, paged-KV block-table addressing, GQA head
  mapping.
* "Merge normalized attention without averaging tile outputs"
  (study.greatitself.com): the merge identity, the empty summary, the
  zero-output policy for fully masked rows.

Modules:

* :mod:`oracle.attention` -- materialised three-pass attention (the plain
  definition), decode attention over ragged KV, the paged-KV gather.
* :mod:`oracle.state` -- the per-block partial state, the two-state merge,
  finalisation, the left-to-right online fold, split-KV partials, and the
  two-operand merge in (O, LSE) form.
* :mod:`oracle.brute` -- pure-Python loops (``math.exp``/``math.fsum``) for
  tiny inputs, used only to pin the materialised oracle.
* :mod:`oracle.fp8` -- the values of 8-bit E4M3 K/V codes (OCP format) with
  their per-tensor scales, so that fp8-KV decode is checked as the float64
  decode of those values.

Every function here is pinned by ``-m "not gpu"`` tests against values the
pages print, closed forms, invariants, or brute force (``tests/test_oracle*``).
"""

from .attention import attention_ref, decode_ref, paged_gather_ref, visible_mask
from .state import (
    EMPTY_M,
    state_ref,
    merge_ref,
    finalize_ref,
    online_ref,
    split_states_ref,
    merge_partials_ref,
    merge_lse_ref,
)
from .brute import brute_attention
from .fp8 import e4m3_decode, e4m3_value, E4M3_VALUES

__all__ = [
    "e4m3_decode",
    "e4m3_value",
    "E4M3_VALUES",
    "attention_ref",
    "decode_ref",
    "paged_gather_ref",
    "visible_mask",
    "EMPTY_M",
    "state_ref",
    "merge_ref",
    "finalize_ref",
    "online_ref",
    "split_states_ref",
    "merge_partials_ref",
    "merge_lse_ref",
    "brute_attention",
]
