"""Decode attention over a paged KV cache, in float64 (oracle; test infrastructure).

What is computed, and where it comes from:

* Cache layout: each physical block holds the keys (or values) of
  ``block_size`` consecutive tokens of one sequence, ``[num_blocks,
  block_size, kv_heads, head_dim]``, one array for K and one for V
  ("PagedAttention Explained", "How PagedAttention works", step 1; the
  per-token key/value store is described under "The problem: the KV cache is
  big and unpredictable").
* Token ``t`` of a sequence sits in logical block ``t // block_size`` at
  offset ``t % block_size`` (same section, step 2: the first sixteen tokens
  in block 0, the next sixteen in block 1).
* The sequence's block table maps the logical block to a physical one, which
  may be anywhere in the pool and in any order (step 3).
* The attention follows the table and gathers K and V from the scattered
  blocks (step 5).  The oracle does the plainest thing that satisfies this:
  it materialises each sequence's contiguous K and V through the table, then
  attends over them.

Readings taken where the pages are silent (no page prints a formula):

* The attention is per-head scaled-dot-product softmax attention of one query
  token per sequence: ``out[h] = sum_t softmax_t(scale * q[h].K[t]) V[t]``.
* The query sees positions ``0 .. L-1`` of its sequence, ``L = seq_lens[s]``
  (its own token included: its K/V is written before attention runs).
* ``scale`` is the caller's float32 value, widened exactly to float64.
* Grouped-query attention: query head ``h`` reads KV head ``h // G`` with
  ``G = q_heads // kv_heads`` (contiguous groups; "Trade-offs and related
  techniques" names head sharing but not the mapping).
* ``L == 0`` gives an all-zero output row.
* Slots past ``L`` in the last block, and blocks the table does not reach, are
  never read.

Split-K (not on the pages; the long-context reduction of this build): the
positions ``0..L-1`` are cut into partitions of ``part_tokens``; partition
``p`` yields ``m_p = max x``, ``l_p = sum exp(x - m_p)`` and the unnormalised
``o_p = sum exp(x - m_p) V``; the merge is ``M = max m_p``,
``w_p = exp(m_p - M)``, ``out = sum w_p o_p / sum w_p l_p``.  This equals the
unsplit result exactly in real arithmetic.
"""

import numpy as np

from .bf16 import widen


def gather_sequence(cache, table_row, length, block_size):
    """Contiguous ``[length, kv_heads, head_dim]`` copy of one sequence's cache.

    Row ``t`` comes from physical block ``table_row[t // block_size]`` at offset
    ``t % block_size``.  The raw stored values are returned (no widening).
    """
    t = np.arange(int(length))
    logical = t // block_size
    offset = t % block_size
    physical = np.asarray(table_row)[logical].astype(np.int64)
    if length and (physical.min() < 0 or physical.max() >= cache.shape[0]):
        raise IndexError("block table entry outside the pool for a used position")
    return cache[physical, offset]


def _shapes(q, k_cache, v_cache):
    if q.ndim != 3 or k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [S, Hq, D]; caches [NB, BS, Hkv, D], K and V alike")
    S, Hq, D = q.shape
    NB, BS, Hkv, Dk = k_cache.shape
    if Dk != D:
        raise ValueError("head_dim differs between q and the cache")
    if Hq % Hkv:
        raise ValueError("q_heads must be a multiple of kv_heads")
    return S, Hq, D, BS, Hkv, Hq // Hkv


def decode_attention(q, k_cache, v_cache, block_table, seq_lens, scale, dtype,
                     seqs=None):
    """float64 ``[S, Hq, D]`` decode-attention output.

    ``q`` is ``[S, Hq, D]``, the caches ``[NB, BS, Hkv, D]``, ``block_table``
    ``[S, MB]`` int, ``seq_lens`` ``[S]`` int; ``dtype`` is ``"f32"`` or
    ``"bf16"`` (uint16 bit patterns) and applies to q and both caches.  With
    ``seqs`` given, only those rows are computed (the others stay zero).
    """
    S, Hq, D, BS, Hkv, G = _shapes(q, k_cache, v_cache)
    scale64 = float(np.float32(scale))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(seq_lens[s])
        if L == 0:
            continue
        K = widen(gather_sequence(k_cache, block_table[s], L, BS), dtype)
        V = widen(gather_sequence(v_cache, block_table[s], L, BS), dtype)
        qs = widen(q[s], dtype)
        for h in range(Hq):
            g = h // G
            x = scale64 * (K[:, g, :] @ qs[h])
            p = np.exp(x - x.max())
            out[s, h] = (p @ V[:, g, :]) / p.sum()
    return out


def partition_states(x, values, part_tokens):
    """Softmax states of each partition of one (sequence, head) row.

    ``x`` holds the ``L`` scaled logits, ``values`` the ``[L, D]`` value rows.
    Returns ``(m, l, o)`` with shapes ``[P]``, ``[P]``, ``[P, D]`` where
    ``P = ceil(L / part_tokens)``.
    """
    L = x.shape[0]
    P = -(-L // part_tokens)
    m = np.empty(P)
    l = np.empty(P)
    o = np.empty((P, values.shape[1]))
    for p in range(P):
        lo, hi = p * part_tokens, min(L, (p + 1) * part_tokens)
        m[p] = x[lo:hi].max()
        e = np.exp(x[lo:hi] - m[p])
        l[p] = e.sum()
        o[p] = e @ values[lo:hi]
    return m, l, o


def merge_states(m, l, o):
    """Log-sum-exp merge of partition states into the normalised output row."""
    M = m.max()
    w = np.exp(m - M)
    return (w @ o) / (w @ l)


def split_decode_attention(q, k_cache, v_cache, block_table, seq_lens, scale,
                           dtype, part_tokens, seqs=None):
    """Same result as :func:`decode_attention`, computed partition by partition."""
    if part_tokens <= 0:
        raise ValueError("part_tokens must be positive")
    S, Hq, D, BS, Hkv, G = _shapes(q, k_cache, v_cache)
    scale64 = float(np.float32(scale))
    out = np.zeros((S, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(seq_lens[s])
        if L == 0:
            continue
        K = widen(gather_sequence(k_cache, block_table[s], L, BS), dtype)
        V = widen(gather_sequence(v_cache, block_table[s], L, BS), dtype)
        qs = widen(q[s], dtype)
        for h in range(Hq):
            g = h // G
            x = scale64 * (K[:, g, :] @ qs[h])
            out[s, h] = merge_states(*partition_states(x, V[:, g, :], part_tokens))
    return out
