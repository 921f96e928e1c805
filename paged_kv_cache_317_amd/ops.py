"""torch-facing wrappers of the C ABI: shape checks and pointer marshalling.

Every computation happens in the HIP kernels behind ``libpkv.so``; torch only
supplies device memory and the current stream.  Names follow the C entry
points without their ``pkv_`` prefix.
"""

import ctypes

import torch

from ._lib import CacheDesc, PKV_BF16, PKV_F32, check, lib

_DTYPE_CODES = {torch.float32: PKV_F32, torch.bfloat16: PKV_BF16}


def cache_desc(k_cache):
    """``CacheDesc`` of a ``[num_blocks, block_size, kv_heads, head_dim]`` cache tensor."""
    if k_cache.dim() != 4:
        raise ValueError("cache must be [num_blocks, block_size, kv_heads, head_dim]")
    if k_cache.dtype not in _DTYPE_CODES:
        raise TypeError(f"cache dtype {k_cache.dtype} is not float32 or bfloat16")
    nb, bs, hkv, d = k_cache.shape
    return CacheDesc(nb, bs, hkv, d, _DTYPE_CODES[k_cache.dtype])


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, name, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_caches(k_cache, v_cache):
    if k_cache.device.type != "cuda":
        raise ValueError("caches must be on a GPU")
    _require(k_cache, "k_cache", k_cache.device)
    _require(v_cache, "v_cache", k_cache.device, k_cache.dtype, k_cache.shape)
    return cache_desc(k_cache)


def paged_kv_write(k, v, slot_mapping, k_cache, v_cache):
    """Write rows ``k[i]``, ``v[i]`` ([kv_heads, head_dim]) into slot ``slot_mapping[i]``."""
    desc = _check_caches(k_cache, v_cache)
    dev = k_cache.device
    T = k.shape[0] if k.dim() == 3 else -1
    _require(k, "k", dev, k_cache.dtype, (T, desc.kv_heads, desc.head_dim))
    _require(v, "v", dev, k_cache.dtype, k.shape)
    _require(slot_mapping, "slot_mapping", dev, torch.int64, (T,))
    with torch.cuda.device(dev):
        check(lib().pkv_paged_kv_write(_ptr(k), _ptr(v), _ptr(slot_mapping), T, _ptr(k_cache),
                                       _ptr(v_cache), ctypes.byref(desc), _stream(dev)))


def decode_partition_tokens(k_cache, num_seqs, q_heads, max_seq_len, part_tokens=0):
    desc = cache_desc(k_cache)
    n = lib().pkv_decode_partition_tokens(ctypes.byref(desc), num_seqs, q_heads, max_seq_len,
                                          part_tokens)
    if n == 0:
        raise ValueError(lib().pkv_last_error().decode())
    return n


def decode_runs(k_cache, num_seqs, q_heads, max_seq_len, part_tokens=0):
    """Runs (equal shares of the work, one workgroup each per kv-head group)
    the decode call splits into; 1 means one kernel and no workspace."""
    desc = cache_desc(k_cache)
    n = lib().pkv_decode_runs(ctypes.byref(desc), num_seqs, q_heads, max_seq_len, part_tokens)
    if n == 0:
        raise ValueError(lib().pkv_last_error().decode())
    return n


def decode_workspace_size(k_cache, num_seqs, q_heads, max_seq_len, part_tokens=0):
    desc = cache_desc(k_cache)
    n = lib().pkv_decode_workspace_size(ctypes.byref(desc), num_seqs, q_heads, max_seq_len,
                                        part_tokens)
    if n == 0 and lib().pkv_last_error():
        raise ValueError(lib().pkv_last_error().decode())
    return n


def paged_attn_decode(q, k_cache, v_cache, block_table, seq_lens, scale, max_seq_len,
                      out=None, part_tokens=0, workspace=None):
    """Decode attention of one query token per sequence over the paged cache.

    ``max_seq_len`` is a host-side bound on ``seq_lens`` (no device read).
    ``workspace`` (uint8, device) is allocated here when the call splits and
    none is given.  Returns ``out`` ([num_seqs, q_heads, head_dim]).
    """
    desc = _check_caches(k_cache, v_cache)
    dev = k_cache.device
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs, q_heads, head_dim]")
    S, Hq, D = q.shape
    _require(q, "q", dev, k_cache.dtype, (S, Hq, desc.head_dim))
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, table_width]")
    _require(block_table, "block_table", dev, torch.int32, (S, block_table.shape[1]))
    _require(seq_lens, "seq_lens", dev, torch.int32, (S,))
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", dev, q.dtype, q.shape)
    # 0 on invalid arguments too: the call itself then reports them
    need = lib().pkv_decode_workspace_size(ctypes.byref(desc), S, Hq, int(max_seq_len),
                                           int(part_tokens))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if workspace is not None:
        _require(workspace, "workspace", dev)
    with torch.cuda.device(dev):
        check(lib().pkv_paged_attn_decode(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), S, Hq, int(max_seq_len), float(scale),
            _ptr(out), int(part_tokens), _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, scale, max_seq_len,
                              out, part_tokens=0):
    """``paged_attn_decode`` for callers that cannot allocate: ``out`` must be
    given, and the split workspace is the library's own device array (calls
    needing more than ``pkv_decode_noalloc_max_workspace()`` bytes raise).
    Calls overlapping on one GPU race."""
    desc = _check_caches(k_cache, v_cache)
    dev = k_cache.device
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs, q_heads, head_dim]")
    S, Hq, D = q.shape
    _require(q, "q", dev, k_cache.dtype, (S, Hq, desc.head_dim))
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, table_width]")
    _require(block_table, "block_table", dev, torch.int32, (S, block_table.shape[1]))
    _require(seq_lens, "seq_lens", dev, torch.int32, (S,))
    _require(out, "out", dev, q.dtype, q.shape)
    with torch.cuda.device(dev):
        check(lib().pkv_paged_attn_decode_noalloc(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), S, Hq, int(max_seq_len), float(scale),
            _ptr(out), int(part_tokens), _stream(dev)))
    return out


def extend_partition_tokens(k_cache, num_seqs, num_tokens, q_heads, max_query_len,
                            max_seq_len, part_tokens=0):
    desc = cache_desc(k_cache)
    n = lib().pkv_extend_partition_tokens(ctypes.byref(desc), num_seqs, num_tokens, q_heads,
                                          max_query_len, max_seq_len, part_tokens)
    if n == 0:
        raise ValueError(lib().pkv_last_error().decode())
    return n


def extend_workspace_size(k_cache, num_seqs, num_tokens, q_heads, max_query_len, max_seq_len,
                          part_tokens=0):
    desc = cache_desc(k_cache)
    n = lib().pkv_extend_workspace_size(ctypes.byref(desc), num_seqs, num_tokens, q_heads,
                                        max_query_len, max_seq_len, part_tokens)
    if n == 0 and lib().pkv_last_error():
        raise ValueError(lib().pkv_last_error().decode())
    return n


def paged_attn_extend(q, k_cache, v_cache, block_table, seq_lens, query_start, scale,
                      max_query_len, max_seq_len, out=None, part_tokens=0, workspace=None):
    """Causal attention of each sequence's new tokens (prefill or chunked
    extend) over the paged cache.  ``q`` and ``out`` are packed
    ``[T, q_heads, head_dim]``; sequence ``s`` owns rows
    ``query_start[s] .. query_start[s + 1] - 1``.  ``max_query_len`` and
    ``max_seq_len`` are host-side bounds on those counts and on ``seq_lens``.
    ``workspace`` (uint8, device) is allocated here when the call splits and
    none is given.  Returns ``out``."""
    desc = _check_caches(k_cache, v_cache)
    dev = k_cache.device
    if q.dim() != 3:
        raise ValueError("q must be [num_tokens, q_heads, head_dim]")
    T, Hq, D = q.shape
    _require(q, "q", dev, k_cache.dtype, (T, Hq, desc.head_dim))
    if block_table.dim() != 2:
        raise ValueError("block_table must be [num_seqs, table_width]")
    S = block_table.shape[0]
    _require(block_table, "block_table", dev, torch.int32)
    _require(seq_lens, "seq_lens", dev, torch.int32, (S,))
    _require(query_start, "query_start", dev, torch.int32, (S + 1,))
    if out is None:
        out = torch.empty_like(q)
    _require(out, "out", dev, q.dtype, q.shape)
    # 0 on invalid arguments too: the call itself then reports them
    need = lib().pkv_extend_workspace_size(ctypes.byref(desc), S, T, Hq, int(max_query_len),
                                           int(max_seq_len), int(part_tokens))
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if workspace is not None:
        _require(workspace, "workspace", dev)
    with torch.cuda.device(dev):
        check(lib().pkv_paged_attn_extend(
            _ptr(q), _ptr(k_cache), _ptr(v_cache), ctypes.byref(desc), _ptr(block_table),
            block_table.shape[1], _ptr(seq_lens), _ptr(query_start), S, T, Hq,
            int(max_query_len), int(max_seq_len), float(scale), _ptr(out), int(part_tokens),
            _ptr(workspace), ws_bytes, _stream(dev)))
    return out


def paged_block_copy(pairs, k_cache, v_cache):
    """Copy whole blocks ``pairs[i, 0] -> pairs[i, 1]`` in both caches."""
    desc = _check_caches(k_cache, v_cache)
    dev = k_cache.device
    n = pairs.shape[0] if pairs.dim() == 2 else -1
    _require(pairs, "pairs", dev, torch.int64, (n, 2))
    with torch.cuda.device(dev):
        check(lib().pkv_paged_block_copy(_ptr(pairs), n, _ptr(k_cache), _ptr(v_cache),
                                         ctypes.byref(desc), _stream(dev)))


def paged_block_move(pairs, src_k, src_v, dst_k, dst_v):
    """Copy blocks ``pairs[i, 0]`` of (src_k, src_v) to ``pairs[i, 1]`` of
    (dst_k, dst_v); either pool may be a pinned host tensor.  Runs on the
    current stream of the GPU side."""
    for t, name in ((src_k, "src_k"), (src_v, "src_v"), (dst_k, "dst_k"), (dst_v, "dst_v")):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.device.type == "cpu" and not t.is_pinned():
            raise ValueError(f"{name} is host memory that is not pinned")
    if src_k.shape != src_v.shape or dst_k.shape != dst_v.shape:
        raise ValueError("K and V pools of one side must have the same shape")
    if src_k.dtype != dst_k.dtype or src_v.dtype != dst_v.dtype or src_k.dtype != src_v.dtype:
        raise TypeError("all pools must share one dtype")
    gpu = [t.device for t in (src_k, dst_k, pairs) if t.device.type == "cuda"]
    if not gpu:
        raise ValueError("at least one side must be on a GPU")
    dev = gpu[0]
    n = pairs.shape[0] if pairs.dim() == 2 else -1
    if tuple(pairs.shape) != (n, 2) or pairs.dtype != torch.int64 or not pairs.is_contiguous():
        raise ValueError("pairs must be a contiguous int64 [n, 2] tensor")
    if pairs.device.type == "cpu" and not pairs.is_pinned():
        raise ValueError("host pairs must be pinned")
    sdesc, ddesc = cache_desc(src_k), cache_desc(dst_k)
    with torch.cuda.device(dev):
        check(lib().pkv_paged_block_move(_ptr(pairs), n, _ptr(src_k), _ptr(src_v),
                                         ctypes.byref(sdesc), _ptr(dst_k), _ptr(dst_v),
                                         ctypes.byref(ddesc), _stream(dev)))
