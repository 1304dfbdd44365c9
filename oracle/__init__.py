"""CPU oracle for paged attention -- TEST INFRASTRUCTURE, not product code.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import, call or run anything in this package.  The HIP library never
imports it and it imports nothing from the HIP library.

Pinned functions (each pin lives in ``tests/test_oracle.py``):

* ``blocks_needed`` / ``slots_allocated`` / ``waste_fraction`` / ``prealloc_waste``
  -- the worked example of the page "Nano-vLLM-Ascend", section 2.1
  (``tests/golden/block_count_example.txt``).
* ``paged_decode`` / ``paged_decode_one`` -- fp64 brute force on tiny inputs,
  torch's float64 ``scaled_dot_product_attention`` (with ``enable_gqa``) on
  dense contiguous layouts, closed forms (L = 1, q = 0, constant V, needle),
  permutation invariance, softmax rows summing to one.
* ``paged_prefill`` -- float64 causal ``scaled_dot_product_attention`` when
  nothing is cached, equality with successive decodes, brute force.
* ``reshape_and_cache`` -- round trip through independently computed slots,
  padding slots skipped, other slots untouched.

* ``int8_kv`` (INT8 KV cache) -- quantiser closed forms (the row maximum maps to
  +-127, zero rows, half-way ties to even, error at most half a step), a
  float64 re-derivation of each code from its exact rational, and decode on the
  dequantised cache equal to the 16-bit oracle on those values.
* ``context_parallel`` (shard partials and their merge) -- merged shards equal
  full-context attention for contiguous and round-robin splits, one shard is the
  identity, empty shards drop out, the (m, l) scaling freedom, planted mistakes
  (``tests/test_cp_oracle.py``).
* ``rope`` (rotary embedding fused with the cache write) -- exact quarter turns,
  equality with complex multiplication by cos + j sin, pair norms, the inverse
  with -sin (the pages' backward), scores depending on relative position only,
  the float32 rounding of each product (a case built so a fused multiply-add
  differs), the 16-bit rounding against brute force, planted mistakes
  (``tests/test_rope_oracle.py``).
* ``block_manager`` (the block manager model, imported as
  ``oracle.block_manager``) -- the 63-block example and a content simulation
  with planted mistakes (``tests/test_block_manager.py``).

Reading, not pinned by the pages: the rotary primitive's pairing of dimensions
(halves, as the Llama/Qwen models the pages serve use; the pages fix only that
the backward is the same primitive with -sin, which every pairing satisfies).

Parity unpinned: the grouping convention of query heads onto KV heads beyond
what torch's ``enable_gqa`` fixes (the pages never mention grouped-query
attention; contiguous groups are the reading taken).
"""
from .paged_attention import (  # noqa: F401
    attend,
    blocks_needed,
    decode_u16,
    gather_sequence,
    kv_head_of,
    logical_to_physical,
    paged_decode,
    paged_decode_one,
    paged_prefill,
    pool_utilisation,
    prealloc_waste,
    reshape_and_cache,
    slot_position,
    slots_allocated,
    softmax_rows,
    visible_keys,
    waste_fraction,
)
from . import brute_force  # noqa: F401
from . import context_parallel  # noqa: F401
from . import int8_kv  # noqa: F401
from . import rope  # noqa: F401
