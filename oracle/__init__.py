"""CPU oracle for the blockwise ring-attention step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. It shares no code with the HIP path
(``ring_attention_blockwise_amd``) and imports nothing from it; the only
module both sides use is ``ring_inputs``, which draws the seeded inputs.

What it computes is the plain definition of the result that the ring of
blockwise steps reaches exactly (up to rounding order): full softmax
attention over the whole global key/value sequence, evaluated in float64 at
the query rows one device holds, with an explicit position mask for causal
attention. It has no blocks, no ring and no running (O, m, l) state.

Sources (the pages and their sections):
* "Ring Attention and Sequence Parallelism" (airsota M4-051), section 3: after
  one full turn of the ring every device has met every K/V block, so its
  output is, mathematically, full attention; section 4 item 2: zigzag
  balancing gives device i segments i and n-1-i (read here as chunks i and
  2n-1-i of 2n chunks, the reading the 8-device/16-chunk workload fixes).
* "distributed training hands-on code" (LLM-101-CN), section 6.2: the block
  step computes S = Q K^T / sqrt(head_dim) and folds exp(S - M) into L and O;
  the forward ends with O / L. Layout [batch, heads, q_len, head_dim].
* Lecture 30 "TP/PP/SP/CP", section 3.2: causal masking is lower-triangular by
  global token position; section 3.4: the ring carries the small GQA KV heads.

``backward.py`` adds the gradient of that attention with respect to Q, K
and V (the pages give the forward only; see its docstring).

Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, a library routine and invariants (see each function's docstring).
"""
from .positions import device_positions, partition_table
from .attention import attention_rows, device_share, visible_pair_count, kv_head_of
from .backward import attention_backward_rows, device_backward, key_gradients, upstream_rows

__all__ = [
    "device_positions", "partition_table", "attention_rows", "device_share",
    "visible_pair_count", "kv_head_of", "attention_backward_rows", "device_backward",
    "key_gradients", "upstream_rows",
]
