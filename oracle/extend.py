"""Multi-token query attention over a paged KV cache, in float64 (oracle;
test infrastructure).

A prefill, or the extension of a sequence by a chunk of new tokens, runs the
same block-aware attention as decode ("PagedAttention Explained", "How
PagedAttention works", step 5: the kernel gathers K and V through the block
table) for several query tokens of one sequence at once.  The pages name the
case under "Preemption and scheduling": a preempted sequence may be
recomputed by a prefill pass over its prompt and generated tokens.

Readings taken where the pages are silent:

* The new tokens of sequence ``s`` are its last ``n`` positions: with
  ``L = seq_lens[s]`` (which counts them; their K/V rows are written to the
  cache before attention runs), query ``j`` (``0 <= j < n``) sits at
  position ``p = L - n + j``.
* Causal attention: the query at position ``p`` attends to positions
  ``0 .. p`` of its sequence, itself included, with per-head
  scaled-dot-product softmax; query head ``h`` reads kv head ``h // G``.  For
  ``n = 1`` this is the decode definition.
* Queries are packed: ``q`` and ``out`` are ``[T, Hq, D]``; sequence ``s``
  owns rows ``query_start[s] .. query_start[s + 1] - 1``.
* A query with ``p < 0`` (more new tokens than ``L``) sees nothing and gets
  an all-zero row, as ``L = 0`` does in decode.
"""

import numpy as np

from .attention import gather_sequence
from .bf16 import widen


def extend_attention(q, k_cache, v_cache, block_table, seq_lens, query_start, scale, dtype,
                     seqs=None):
    """float64 ``[T, Hq, D]`` output of the new tokens' causal attention.

    ``q`` ``[T, Hq, D]``; caches ``[NB, BS, Hkv, D]``; ``block_table``
    ``[S, MB]``; ``seq_lens`` ``[S]``; ``query_start`` ``[S + 1]``
    non-decreasing with ``query_start[S] == T``; ``dtype`` ``"f32"`` or
    ``"bf16"`` (uint16 bit patterns) for q and both caches.  With ``seqs``
    given only those sequences' rows are computed (the others stay zero).
    """
    if q.ndim != 3 or k_cache.ndim != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("q must be [T, Hq, D]; caches [NB, BS, Hkv, D], K and V alike")
    T, Hq, D = q.shape
    BS, Hkv = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape[3] != D or Hq % Hkv:
        raise ValueError("head_dim must match and q_heads must be a multiple of kv_heads")
    G = Hq // Hkv
    qs = np.asarray(query_start, dtype=np.int64)
    S = qs.size - 1
    if qs[0] != 0 or qs[-1] != T or np.any(np.diff(qs) < 0):
        raise ValueError("query_start must rise from 0 to the number of query rows")
    scale64 = float(np.float32(scale))
    out = np.zeros((T, Hq, D), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        n, L = int(qs[s + 1] - qs[s]), int(seq_lens[s])
        if n == 0 or L == 0:
            continue
        K = widen(gather_sequence(k_cache, block_table[s], L, BS), dtype)   # [L, Hkv, D]
        V = widen(gather_sequence(v_cache, block_table[s], L, BS), dtype)
        Q = widen(q[qs[s]:qs[s + 1]], dtype)                                # [n, Hq, D]
        pos = L - n + np.arange(n)                                          # query positions
        visible = np.arange(L)[None, :] <= pos[:, None]                     # [n, L]
        for h in range(Hq):
            g = h // G
            x = scale64 * (Q[:, h, :] @ K[:, g, :].T)                       # [n, L]
            x = np.where(visible, x, -np.inf)
            for j in range(n):
                if pos[j] < 0:
                    continue
                p = np.exp(x[j] - x[j].max())
                out[qs[s] + j, h] = (p @ V[:, g, :]) / p.sum()
    return out


def extend_flops(seq_lens, query_start, q_heads, head_dim):
    """Multiply-add work of the causal attention, counted as 2 flops each:
    every query at position ``p`` takes ``p + 1`` dot products of length
    ``head_dim`` for its logits and as many scaled value rows, per head."""
    qs = np.asarray(query_start, dtype=np.int64)
    total = 0
    for s in range(qs.size - 1):
        n, L = int(qs[s + 1] - qs[s]), int(seq_lens[s])
        pos = L - n + np.arange(n)
        total += int(np.clip(pos + 1, 0, None).sum())
    return total * q_heads * 4 * head_dim
