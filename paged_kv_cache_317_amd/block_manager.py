"""Python face of the native host block manager in libpkv (pkv_bm_* C calls).

Marshalling only: every rule (on-demand allocation, reference counts,
copy-on-write, release) runs in the C++ library.
"""

import ctypes

import numpy as np

from ._lib import BmStats, PkvError, check, lib


class BlockManager:
    """A pool of ``num_blocks`` blocks of ``block_size`` token slots.

    ``free_order`` (a permutation of the pool ids) sets the order in which
    free blocks are handed out; the default is ascending ids.
    """

    def __init__(self, num_blocks, block_size, free_order=None):
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        handle = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (self.num_blocks,):
                raise ValueError("free_order must list every block once")
        check(lib().pkv_bm_create(self.num_blocks, self.block_size,
                                  None if order is None else order.ctypes.data,
                                  ctypes.byref(handle)))
        self._h = handle

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            lib().pkv_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, seq):
        check(lib().pkv_bm_add(self._h, int(seq)))

    def fork(self, parent, child):
        check(lib().pkv_bm_fork(self._h, int(parent), int(child)))

    def append(self, seq, n=1):
        """Store ``n`` tokens; returns (slots, copies) as Python lists."""
        slots = np.empty(max(n, 1), dtype=np.int64)
        copies = np.empty((1, 2), dtype=np.int64)
        ncop = ctypes.c_int32()
        check(lib().pkv_bm_append(self._h, int(seq), int(n), slots.ctypes.data,
                                  copies.ctypes.data, 1, ctypes.byref(ncop)))
        return slots[:n].tolist(), [tuple(r) for r in copies[:ncop.value].tolist()]

    def add_cached(self, seq, tokens):
        """Start ``seq`` for a request with these token ids, reusing cached
        full blocks from its start; returns the number of reused tokens."""
        arr = np.ascontiguousarray(tokens, dtype=np.int32)
        out = ctypes.c_int32()
        check(lib().pkv_bm_add_cached(self._h, int(seq), arr.ctypes.data if arr.size else None,
                                      len(arr), ctypes.byref(out)))
        return out.value

    def append_tokens(self, seq, tokens):
        """``append`` with token ids; full blocks become findable."""
        arr = np.ascontiguousarray(tokens, dtype=np.int32)
        n = len(arr)
        slots = np.empty(max(n, 1), dtype=np.int64)
        copies = np.empty((1, 2), dtype=np.int64)
        ncop = ctypes.c_int32()
        check(lib().pkv_bm_append_tokens(self._h, int(seq), arr.ctypes.data if n else None, n,
                                         slots.ctypes.data, copies.ctypes.data, 1,
                                         ctypes.byref(ncop)))
        return slots[:n].tolist(), [tuple(r) for r in copies[:ncop.value].tolist()]

    def blocks_needed(self, seq, n):
        out = ctypes.c_int32()
        check(lib().pkv_bm_blocks_needed(self._h, int(seq), int(n), ctypes.byref(out)))
        return out.value

    def free_sequence(self, seq):
        check(lib().pkv_bm_free(self._h, int(seq)))

    def preempt(self, seq):
        check(lib().pkv_bm_preempt(self._h, int(seq)))

    def set_swap_space(self, host_blocks):
        check(lib().pkv_bm_set_swap_space(self._h, int(host_blocks)))

    def _swap(self, fn, seq):
        n = ctypes.c_int32()
        cap = max(self.num_blocks, 1)
        pairs = np.empty((cap, 2), dtype=np.int64)
        check(fn(self._h, int(seq), pairs.ctypes.data, cap, ctypes.byref(n)))
        return [tuple(r) for r in pairs[:n.value].tolist()]

    def swap_out(self, seq):
        """Move ``seq`` to host swap space; returns (device, host) block pairs."""
        return self._swap(lib().pkv_bm_swap_out, seq)

    def swap_in(self, seq):
        """Bring ``seq`` back to fresh device blocks; returns (host, device) pairs."""
        return self._swap(lib().pkv_bm_swap_in, seq)

    def length(self, seq):
        out = ctypes.c_int32()
        check(lib().pkv_bm_length(self._h, int(seq), ctypes.byref(out)))
        return out.value

    def table_array(self, seqs, width):
        ids = np.ascontiguousarray(seqs, dtype=np.int64)
        out = np.empty((len(ids), width), dtype=np.int32)
        check(lib().pkv_bm_table(self._h, ids.ctypes.data, len(ids), int(width),
                                 out.ctypes.data))
        return out

    def stats(self):
        s = BmStats()
        check(lib().pkv_bm_get_stats(self._h, ctypes.byref(s)))
        return {name: getattr(s, name) for name, _ in BmStats._fields_}


def capacity(num_blocks, block_size, lens, reserve_len):
    """(paged, contiguous): leading requests of ``lens`` that fit the pool."""
    arr = np.ascontiguousarray(lens, dtype=np.int32)
    paged, contig = ctypes.c_int32(), ctypes.c_int32()
    check(lib().pkv_capacity(int(num_blocks), int(block_size), arr.ctypes.data, len(arr),
                             int(reserve_len), ctypes.byref(paged), ctypes.byref(contig)))
    return paged.value, contig.value


__all__ = ["BlockManager", "capacity", "PkvError"]
