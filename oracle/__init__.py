"""CPU oracle for the paged KV-cache decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports, calls or
links anything here; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path: it imports numpy and nothing else, widens bf16 by its own bit
arithmetic and computes every floating-point result in float64.

Sources (three web pages on the subject):

* "PagedAttention" (ai-and-cloud.com glossary): sections "What is
  PagedAttention?" and "Why it mattered enough to launch vLLM".
* "PagedAttention Explained: Virtual Memory for the KV Cache"
  (lycoristechnologies.com): section "How PagedAttention works" (steps 1-5),
  "Sharing blocks between sequences", the table "Contiguous allocation vs
  PagedAttention", "Trade-offs and related techniques".
* "What does PagedAttention change in LLM KV allocation?" (slavadubrov.com
  fast answers): sections "Calculate unused block space" and "Sharing
  requires more than allocation".

The pages fix the block/table mechanics but print no attention formula; the
oracle takes standard per-head scaled-dot-product softmax attention with one
query token per sequence, which is the plain reading of "the attention
computation follows the block table" (second page, step 5).  Every reading the
oracle takes where the pages are silent is listed in the module that takes it.

Modules
-------
``bf16``           exact widening of bfloat16 bit patterns to float64.
``attention``      decode attention over a paged cache (materialise, then
                   attend), the split-K partition states and their merge.
``extend``         multi-token (prefill / chunked extend) causal attention
                   over a paged cache.
``cache_ops``      slot write, block copy and the two-pool block move
                   (bitwise).
``block_manager``  on-demand allocation, reference counts, copy-on-write,
                   release, and waste accounting.

Pins: each function here is checked in ``tests/test_oracle_*.py`` against
facts the pages print (the 35-token worked example, the token-to-block
mapping), closed forms, a library routine on a special case, and brute force
on tiny inputs.  No function here is "parity unpinned".
"""

from .bf16 import widen
from .attention import (
    gather_sequence,
    decode_attention,
    partition_states,
    merge_states,
    split_decode_attention,
)
from .extend import extend_attention, extend_flops
from .cache_ops import kv_write, block_copy, block_move
from .block_manager import BlockManager, OutOfBlocks, blocks_for, tail_waste

__all__ = [
    "widen",
    "gather_sequence",
    "decode_attention",
    "partition_states",
    "merge_states",
    "split_decode_attention",
    "extend_attention",
    "extend_flops",
    "kv_write",
    "block_copy",
    "block_move",
    "BlockManager",
    "OutOfBlocks",
    "blocks_for",
    "tail_waste",
]
