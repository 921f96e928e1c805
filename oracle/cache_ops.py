"""Slot write and block copy, bitwise (oracle; test infrastructure).

* Slot write: each new token's key and value rows (``[kv_heads, head_dim]``)
  go to the slot the caller assigned, i.e. physical block ``slot //
  block_size`` at offset ``slot % block_size`` ("PagedAttention Explained",
  "The problem: the KV cache is big and unpredictable": the cache grows by one
  entry per new token; "How PagedAttention works", steps 2-4 for where it
  lands).  Reading: ``slot = physical_block * block_size + offset``; a
  negative slot means "no write" (padding).  Duplicate slots within one call
  are outside the contract.
* Block copy: before a sequence writes into a block that other sequences
  still reference, the block is copied and the writer's table is pointed at
  the copy (same page, "Sharing blocks between sequences").  Here the copy
  itself: for every ``(src, dst)`` pair, the whole ``dst`` block of both caches
  becomes the pre-call ``src`` block.  Reading: within one call the ``dst`` ids
  are distinct and none equals any ``src``, so the order of pairs does not
  matter.

* Block move: the same copy between two pools of one block shape, the mover
  behind swapping a preempted sequence's blocks out to host memory and back
  ("PagedAttention Explained", "Preemption and scheduling" names swapping as
  one answer to running out of blocks).  For every ``(src, dst)`` pair, block
  ``dst`` of the destination pool becomes block ``src`` of the source pool as
  it was before the call.  Reading: ids outside their pool are an error here
  (the device library skips them as a guard).

All three operate on raw stored values (float32 or uint16 bit patterns) and
never round or convert anything.
"""

import numpy as np


def kv_write(k_cache, v_cache, k, v, slot_mapping, inplace=False):
    """Write token rows into their slots.  Returns the (new) caches.

    ``k``/``v`` are ``[T, kv_heads, head_dim]``; ``slot_mapping`` is ``[T]``.
    """
    if not inplace:
        k_cache = k_cache.copy()
        v_cache = v_cache.copy()
    num_blocks, block_size = k_cache.shape[:2]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        if block >= num_blocks:
            raise IndexError(f"slot {slot} is outside the pool")
        k_cache[block, offset] = k[i]
        v_cache[block, offset] = v[i]
    return k_cache, v_cache


def block_copy(k_cache, v_cache, pairs, inplace=False):
    """Copy whole physical blocks ``src -> dst`` in both caches.

    ``pairs`` is ``[n, 2]`` of ``(src, dst)``.  Sources are read from the
    state before the call.
    """
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    if len(set(dst.tolist())) != len(dst) or set(dst.tolist()) & set(src.tolist()):
        raise ValueError("block copy pairs need distinct dst ids, none equal to a src id")
    k_src = k_cache[src].copy()
    v_src = v_cache[src].copy()
    if not inplace:
        k_cache = k_cache.copy()
        v_cache = v_cache.copy()
    k_cache[dst] = k_src
    v_cache[dst] = v_src
    return k_cache, v_cache


def block_move(src_k, src_v, dst_k, dst_v, pairs):
    """Copy blocks ``src`` of (src_k, src_v) to blocks ``dst`` of (dst_k,
    dst_v); returns new destination pools.  ``pairs`` is ``[n, 2]`` of
    ``(src, dst)``; destination ids must be distinct.  When the two pools are
    the same arrays, the sources are read before any write."""
    pairs = np.asarray(pairs, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0], pairs[:, 1]
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("pools must have the same block shape and dtype")
    if len(set(dst.tolist())) != len(dst):
        raise ValueError("destination ids must be distinct")
    if src.size and (src.min() < 0 or src.max() >= src_k.shape[0]
                     or dst.min() < 0 or dst.max() >= dst_k.shape[0]):
        raise IndexError("a block id is outside its pool")
    k_rows = src_k[src].copy()
    v_rows = src_v[src].copy()
    out_k = dst_k.copy()
    out_v = dst_v.copy()
    out_k[dst] = k_rows
    out_v[dst] = v_rows
    return out_k, out_v
