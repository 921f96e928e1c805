"""Host block manager: allocation, sharing and copy-on-write (oracle; test infrastructure).

What it follows:

* Blocks hold a fixed number of tokens ("PagedAttention Explained", "How
  PagedAttention works", step 1).  A sequence of ``L`` tokens owns
  ``ceil(L / block_size)`` blocks, every one full except possibly the last
  (step 2; and "What does PagedAttention change in LLM KV allocation?",
  "Calculate unused block space", whose 35-token example needs three
  16-token blocks and leaves thirteen slots of the last one empty).
* A new physical block is taken only when the sequence's last block is full;
  nothing is reserved ahead (step 4).  Blocks go back to the pool when the
  request finishes (third page, same section).
* The per-sequence block table maps logical to physical blocks, in any order
  (step 3).  ``free_order`` sets the order in which the pool hands out ids,
  which is how a caller produces scattered placements.
* Several tables may point at one physical block; each block carries a
  reference count.  A sequence about to write into a block whose count is
  above one first gets its own copy, and its table is pointed at the copy
  ("Sharing blocks between sequences").  Reading: the writer copies while the
  count is above one and decrements it, so the last holder writes in place;
  ``append`` reports each copy as a ``(src, dst)`` pair for a block-copy call.
* The only waste of a sequence is the unused tail of its last block, less than
  one block ("How PagedAttention works", closing paragraph, and the table
  "Contiguous allocation vs PagedAttention").
* Prefix caching: requests with identical prefixes can reuse the same
  physical blocks, but the paged layout does not provide the lookup by itself
  ("What does PagedAttention change in LLM KV allocation?", "Sharing requires
  more than allocation").  Reading: a full block is findable under the whole
  token prefix it completes (positions 0 .. end of the block), while some
  sequence holds it; a new request reuses the longest run of such blocks from
  its start.  Blocks filled later through ``append_tokens`` become findable;
  the first block registered under a prefix keeps the entry.
* Preemption by swapping: a sequence's blocks move to host memory and come
  back later ("PagedAttention Explained", "Preemption and scheduling").
  Reading: swap-out copies every block of the sequence, in table order, to
  its own free host block and drops the sequence's device references (blocks
  other sequences share stay on the device for them); swap-in takes fresh
  device blocks in the same order and frees the host blocks.  Sharing is not
  carried through a swap, and a swapped sequence cannot grow or be forked.
"""

from collections import deque

import numpy as np


class OutOfBlocks(RuntimeError):
    """The pool has no free block left."""


def blocks_for(length, block_size):
    """Number of blocks a sequence of ``length`` tokens occupies."""
    if length < 0 or block_size <= 0:
        raise ValueError("length must be >= 0 and block_size > 0")
    return -(-length // block_size)


def tail_waste(length, block_size):
    """Unused slots in a sequence's blocks (all in its last block)."""
    return blocks_for(length, block_size) * block_size - length


class BlockManager:
    """Pool of ``num_blocks`` physical blocks of ``block_size`` token slots."""

    def __init__(self, num_blocks, block_size, free_order=None):
        if num_blocks <= 0 or block_size <= 0:
            raise ValueError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = list(range(num_blocks)) if free_order is None else [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool ids")
        self.free = deque(order)
        self.refcount = [0] * num_blocks
        self.fill = [0] * num_blocks
        self.tables = {}
        self.lengths = {}
        self.tokens = {}          # seq -> token ids, or None when not tracked
        self.cache = {}           # full token prefix (tuple) -> physical block
        self.block_key = {}       # physical block -> its prefix key
        self.reused_blocks = 0
        self.host_free = deque()  # host pool for swapped blocks
        self.host_blocks = 0
        self.swapped = {}         # seq -> (host block table, length, tokens)
        self.swap_outs = 0

    # -- pool -------------------------------------------------------------
    def _take(self):
        if not self.free:
            raise OutOfBlocks("no free block in the pool")
        b = self.free.popleft()
        self.refcount[b] = 1
        self.fill[b] = 0
        return b

    def _drop(self, b):
        self.refcount[b] -= 1
        if self.refcount[b] == 0:
            self.fill[b] = 0
            self.free.append(b)
            key = self.block_key.pop(b, None)
            if key is not None:
                del self.cache[key]

    # -- sequences ----------------------------------------------------------
    def add(self, seq):
        if seq in self.tables or seq in self.swapped:
            raise KeyError(f"sequence {seq!r} exists")
        self.tables[seq] = []
        self.lengths[seq] = 0
        self.tokens[seq] = None

    def add_cached(self, seq, tokens):
        """Start ``seq`` for a request with these token ids, reusing the
        longest run of findable full blocks from its start.  Returns the number
        of reused tokens (a multiple of the block size); the rest of the
        request is for the caller to append."""
        self.add(seq)
        BS = self.block_size
        tokens = [int(t) for t in tokens]
        n = 0
        while n + BS <= len(tokens):
            b = self.cache.get(tuple(tokens[: n + BS]))
            if b is None:
                break
            self.refcount[b] += 1
            self.tables[seq].append(b)
            n += BS
        self.reused_blocks += n // BS
        self.lengths[seq] = n
        self.tokens[seq] = tokens[:n]
        return n

    def append_tokens(self, seq, tokens):
        """``append`` for a request that carries token ids: blocks that
        become full are registered under their prefix."""
        if self.tokens[seq] is None:
            raise ValueError("sequence does not carry token ids")
        tokens = [int(t) for t in tokens]
        start = self.lengths[seq]
        slots, copies = self.append(seq, len(tokens), keep_tokens=True)
        self.tokens[seq] += tokens
        BS = self.block_size
        for j in range(start // BS, self.lengths[seq] // BS):
            key = tuple(self.tokens[seq][: (j + 1) * BS])
            b = self.tables[seq][j]
            if key not in self.cache and b not in self.block_key:
                self.cache[key] = b
                self.block_key[b] = key
        return slots, copies

    def append(self, seq, n=1, keep_tokens=False):
        """Store ``n`` new tokens of ``seq``.

        Returns ``(slots, copies)``: the slot of each new token
        (``physical * block_size + offset``) and the ``(src, dst)`` block
        copies the writes require, in order.
        """
        BS = self.block_size
        table = self.tables[seq]
        if not keep_tokens:
            self.tokens[seq] = None         # token ids no longer known
        slots, copies = [], []
        for _ in range(n):
            t = self.lengths[seq]
            offset = t % BS
            if offset == 0:
                b = self._take()
                table.append(b)
            else:
                b = table[-1]
                if self.refcount[b] > 1:
                    nb = self._take()
                    copies.append((b, nb))
                    self.fill[nb] = self.fill[b]
                    self.refcount[b] -= 1
                    table[-1] = nb
                    b = nb
            slots.append(b * BS + offset)
            self.fill[b] = max(self.fill[b], offset + 1)
            self.lengths[seq] = t + 1
        return slots, copies

    # -- swapping ---------------------------------------------------------------
    def set_swap_space(self, host_blocks):
        if self.host_blocks:
            raise ValueError("swap space is already set")
        self.host_blocks = host_blocks
        self.host_free = deque(range(host_blocks))

    def swap_out(self, seq):
        """Move ``seq`` to host blocks; returns (device, host) block pairs."""
        table = self.tables[seq]
        if len(table) > len(self.host_free):
            raise OutOfBlocks("not enough free host blocks")
        host = [self.host_free.popleft() for _ in table]
        pairs = list(zip(table, host))
        self.swapped[seq] = (host, self.lengths[seq], self.tokens[seq])
        for b in self.tables.pop(seq):
            self._drop(b)
        del self.lengths[seq]
        del self.tokens[seq]
        self.swap_outs += 1
        return pairs

    def swap_in(self, seq):
        """Bring ``seq`` back to fresh device blocks; returns (host, device) pairs."""
        host, length, tokens = self.swapped[seq]
        if len(host) > len(self.free):
            raise OutOfBlocks("not enough free device blocks")
        del self.swapped[seq]
        dev = [self._take() for _ in host]
        BS = self.block_size
        for j, b in enumerate(dev):
            self.fill[b] = min(BS, length - j * BS)
        self.tables[seq] = dev
        self.lengths[seq] = length
        self.tokens[seq] = None            # fresh blocks are not registered
        self.host_free.extend(host)
        return list(zip(host, dev))

    def fork(self, parent, child):
        """``child`` starts as a copy of ``parent`` that shares all its blocks."""
        self.add(child)
        self.tables[child] = list(self.tables[parent])
        self.lengths[child] = self.lengths[parent]
        toks = self.tokens[parent]
        self.tokens[child] = None if toks is None else list(toks)
        for b in self.tables[child]:
            self.refcount[b] += 1

    def free_sequence(self, seq):
        """Release ``seq``; blocks nobody else references return to the pool
        (host blocks to the swap space when it is swapped out)."""
        if seq in self.swapped:
            self.host_free.extend(self.swapped.pop(seq)[0])
            return
        for b in self.tables.pop(seq):
            self._drop(b)
        del self.lengths[seq]
        del self.tokens[seq]

    # -- views --------------------------------------------------------------
    def table_array(self, seqs, width):
        """int32 ``[len(seqs), width]`` block table, unused entries ``-1``."""
        out = np.full((len(seqs), width), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            row = self.tables[s]
            if len(row) > width:
                raise ValueError(f"sequence {s!r} needs {len(row)} table entries > {width}")
            out[i, : len(row)] = row
        return out

    def stats(self):
        """Allocation figures of the pool (the measurements the third page lists)."""
        allocated = [b for b in range(self.num_blocks) if self.refcount[b] > 0]
        used = sum(self.fill[b] for b in allocated)
        slots = len(allocated) * self.block_size
        return {
            "allocated_blocks": len(allocated),
            "allocated_slots": slots,
            "used_slots": used,
            "unused_slots": slots - used,
            "waste_fraction": (slots - used) / slots if slots else 0.0,
            "free_blocks": len(self.free),
            "sequences": len(self.tables),
            "cached_blocks": len(self.cache),
            "reused_blocks": self.reused_blocks,
            "host_blocks_used": self.host_blocks - len(self.host_free),
            "swapped_sequences": len(self.swapped),
            "swap_outs": self.swap_outs,
        }
