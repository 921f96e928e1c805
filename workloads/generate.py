"""Seeded generation of decode inputs (layouts and values).

Recipe (every draw comes from one stream seeded with ``cfg.seed``):

1. Layout, numpy ``default_rng(seed)`` (PCG64):
   * lengths: fixed, or ``integers(lo, hi + 1, size=S)``; with a shared
     prefix the draw is the suffix length and the prefix is added;
   * blocks per sequence ``ceil(L / block_size)``; the prefix's blocks are
     shared by every sequence (prefix lengths must be whole blocks here);
   * pool ``num_blocks``: fixed, or ``ceil(pool_factor * blocks needed)``;
   * placement: ``permutation(num_blocks)`` handed out in (shared prefix,
     then sequence, then logical block) order; the rest of the permutation is
     the free list (``spare_blocks``), in that order.
2. Values, host variant (same numpy stream, continuing): q ``[S, Hq, D]``,
   the whole K pool, the whole V pool, then the new token's K and V rows
   ``[S, Hkv, D]``; each is ``standard_normal(float32) * std`` drawn in
   chunks of 2**22 elements, and for bf16 rounded to nearest-even bf16 bit
   patterns (``uint16``).  Unused slots and unreferenced blocks hold draws
   too.
3. Values, device variant: the same tensors in the same order from a torch
   generator on the device seeded with ``seed``, ``randn(float32) * std``,
   then ``.to(bfloat16)`` (round to nearest even).  Used where the pool is
   gigabytes; its values differ from the host variant's.

The new token of sequence ``s`` is its position ``L - 1``: decode writes its
K/V row into that slot, then attends over positions ``0 .. L-1``.
"""

from dataclasses import dataclass, field

import numpy as np

_CHUNK = 1 << 22


def f32_to_bf16_bits(x):
    """float32 array -> uint16 bf16 bit patterns, round to nearest even.

    Inputs here are finite normal draws, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


@dataclass
class Layout:
    """Lengths, pool size and block tables of one decode batch."""

    block_size: int
    seq_lens: np.ndarray            # int32 [S]
    block_table: np.ndarray         # int32 [S, table_width], -1 where unused
    num_blocks: int
    shared_blocks: np.ndarray       # int64, physical ids of the shared prefix
    spare_blocks: np.ndarray        # int64, ids no table references (free list)

    @property
    def max_seq_len(self):
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def used_blocks(self):
        return int(self.num_blocks - self.spare_blocks.size)


@dataclass
class Workload:
    """One batch: layout plus values, on the host (numpy) or a device (torch)."""

    cfg: object
    layout: Layout
    q: object
    k_cache: object
    v_cache: object
    new_k: object
    new_v: object
    slot_mapping: object
    block_table: object = None
    seq_lens: object = None
    extra: dict = field(default_factory=dict)


def build_layout(cfg, rng=None):
    """Lengths, pool and block tables of ``cfg`` (consumes ``rng`` draws)."""
    rng = np.random.default_rng(cfg.seed) if rng is None else rng
    S, BS = cfg.num_seqs, cfg.block_size
    if cfg.seq_lens:
        lens = np.asarray(cfg.seq_lens, dtype=np.int64)
        if lens.size != S:
            raise ValueError("seq_lens must have num_seqs entries")
    else:
        lo, hi = cfg.len_range
        lens = rng.integers(lo, hi + 1, size=S).astype(np.int64)
    if cfg.prefix_tokens % BS:
        raise ValueError("a shared prefix must be whole blocks in a decode layout")
    shared = cfg.prefix_tokens // BS
    lens = lens + cfg.prefix_tokens
    nblk = -(-lens // BS)
    private = nblk - shared
    need = shared + int(private.sum())
    NB = cfg.pool_blocks if cfg.pool_blocks else int(np.ceil(cfg.pool_factor * need))
    if NB < need:
        raise ValueError(f"pool of {NB} blocks is smaller than the {need} needed")
    MB = cfg.table_width
    if nblk.max(initial=0) > MB:
        raise ValueError("a sequence needs more table entries than the table width")
    perm = rng.permutation(NB).astype(np.int64)
    table = np.full((S, MB), -1, dtype=np.int32)
    shared_ids = perm[:shared]
    cursor = shared
    for s in range(S):
        table[s, :shared] = shared_ids
        n = int(private[s])
        table[s, shared:shared + n] = perm[cursor:cursor + n]
        cursor += n
    return Layout(block_size=BS, seq_lens=lens.astype(np.int32), block_table=table,
                  num_blocks=NB, shared_blocks=shared_ids.copy(),
                  spare_blocks=perm[cursor:].copy())


def decode_slots(block_table, seq_lens, block_size):
    """int64 slot of each sequence's newest token (position ``L - 1``); -1 if ``L == 0``."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    slots = np.full(lens.shape, -1, dtype=np.int64)
    for s, L in enumerate(lens.tolist()):
        if L > 0:
            t = L - 1
            slots[s] = int(block_table[s, t // block_size]) * block_size + t % block_size
    return slots


def _draw_host(rng, shape, cfg):
    n = int(np.prod(shape))
    if cfg.dtype == "f32":
        out = np.empty(n, dtype=np.float32)
    else:
        out = np.empty(n, dtype=np.uint16)
    std = np.float32(cfg.std)
    for off in range(0, n, _CHUNK):
        c = min(_CHUNK, n - off)
        x = rng.standard_normal(c, dtype=np.float32) * std
        out[off:off + c] = x if cfg.dtype == "f32" else f32_to_bf16_bits(x)
    return out.reshape(shape)


def generate_host(cfg):
    """Host (numpy) workload; bf16 values are uint16 bit patterns."""
    rng = np.random.default_rng(cfg.seed)
    layout = build_layout(cfg, rng)
    S, Hq, Hkv, D, BS = cfg.num_seqs, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.block_size
    q = _draw_host(rng, (S, Hq, D), cfg)
    k_cache = _draw_host(rng, (layout.num_blocks, BS, Hkv, D), cfg)
    v_cache = _draw_host(rng, (layout.num_blocks, BS, Hkv, D), cfg)
    new_k = _draw_host(rng, (S, Hkv, D), cfg)
    new_v = _draw_host(rng, (S, Hkv, D), cfg)
    slots = decode_slots(layout.block_table, layout.seq_lens, BS)
    return Workload(cfg=cfg, layout=layout, q=q, k_cache=k_cache, v_cache=v_cache,
                    new_k=new_k, new_v=new_v, slot_mapping=slots,
                    block_table=layout.block_table, seq_lens=layout.seq_lens)


def generate_device(cfg, device="cuda"):
    """Device (torch) workload with the host layout and device-drawn values."""
    import torch

    layout = build_layout(cfg)
    S, Hq, Hkv, D, BS = cfg.num_seqs, cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.block_size
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    dt = torch.float32 if cfg.dtype == "f32" else torch.bfloat16

    def draw(shape):
        out = torch.empty(shape, dtype=dt, device=device)
        flat = out.view(-1)
        for off in range(0, flat.numel(), 1 << 26):
            c = min(1 << 26, flat.numel() - off)
            x = torch.randn(c, generator=gen, device=device, dtype=torch.float32) * cfg.std
            flat[off:off + c] = x.to(dt)
        return out

    q = draw((S, Hq, D))
    k_cache = draw((layout.num_blocks, BS, Hkv, D))
    v_cache = draw((layout.num_blocks, BS, Hkv, D))
    new_k = draw((S, Hkv, D))
    new_v = draw((S, Hkv, D))
    slots = decode_slots(layout.block_table, layout.seq_lens, BS)
    return Workload(
        cfg=cfg, layout=layout, q=q, k_cache=k_cache, v_cache=v_cache,
        new_k=new_k, new_v=new_v,
        slot_mapping=torch.from_numpy(slots).to(device),
        block_table=torch.from_numpy(layout.block_table).to(device),
        seq_lens=torch.from_numpy(layout.seq_lens).to(device))


def cow_layout(layout, prefix_tokens):
    """Copy-on-write scenario on a shared-prefix layout.

    Every sequence starts as ``prefix_tokens`` tokens held in the shared
    blocks.  Each sequence then writes one divergent token at position
    ``w``: ``w = prefix_tokens`` when the prefix ends inside a block (the
    write lands in the shared partial block), else ``w = prefix_tokens - 1``
    (the last shared block is full, and the write replaces its last slot).
    Writers copy the shared block while other holders remain; the last
    sequence holds it alone and writes in place.

    Returns a dict with ``lens_before`` (``prefix_tokens`` each),
    ``table_before`` (shared blocks only), ``pairs`` (int64 ``[S-1, 2]``
    ``(src, dst)``), ``table_after``, ``write_slots`` (int64 ``[S]``) and
    ``lens_after`` (``w + 1`` each).
    """
    BS = layout.block_size
    S, MB = layout.block_table.shape
    nshared = -(-prefix_tokens // BS)
    if nshared == 0 or nshared > layout.shared_blocks.size:
        raise ValueError("prefix must lie within the layout's shared blocks")
    w = prefix_tokens if prefix_tokens % BS else prefix_tokens - 1
    j = w // BS
    if j >= nshared:
        raise ValueError("write position outside the shared prefix blocks")
    if layout.spare_blocks.size < S - 1:
        raise ValueError("not enough free blocks for the copies")
    src = int(layout.shared_blocks[j])
    table_before = np.full((S, MB), -1, dtype=np.int32)
    table_before[:, :nshared] = layout.shared_blocks[:nshared]
    dst = layout.spare_blocks[: S - 1].astype(np.int64)
    pairs = np.stack([np.full(S - 1, src, dtype=np.int64), dst], axis=1)
    table_after = table_before.copy()
    table_after[: S - 1, j] = dst
    write_slots = table_after[:, j].astype(np.int64) * BS + w % BS
    return {
        "lens_before": np.full(S, prefix_tokens, dtype=np.int32),
        "table_before": table_before,
        "pairs": pairs,
        "table_after": table_after,
        "write_slots": write_slots,
        "lens_after": np.full(S, w + 1, dtype=np.int32),
        "write_position": w,
    }
