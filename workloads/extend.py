"""Seeded multi-token query workloads: prefill and chunked extend batches.

Each sequence has ``ctx`` tokens already in the cache and ``new`` tokens
being added; its length is ``L = ctx + new``.  Recipe (one numpy PCG64 stream
seeded with ``cfg.seed``):

1. ``ctx``: fixed or ``integers(lo, hi + 1, size=S)``; then ``new`` the same
   way.
2. Layout: the decode layout recipe for lengths ``L`` (same stream; pool
   ``ceil(pool_factor x blocks needed)``, placement by ``permutation``).
3. Values: q ``[T, Hq, D]`` (``T = sum new``), the K pool, the V pool, then
   the new tokens' K and V rows ``[T, Hkv, D]``; standard normal float32
   times ``std``, rounded to nearest-even bf16 for bf16.  The pools hold
   draws everywhere, the new tokens' slots included: a slot write of the new
   rows comes first in a step.
The device variant draws the same tensors in the same order from a torch
generator on the device (values differ from the host variant's).
"""

from dataclasses import dataclass

import numpy as np

from .configs import DecodeConfig
from .generate import _draw_host, build_layout


@dataclass(frozen=True)
class ExtendConfig:
    name: str
    num_seqs: int
    q_heads: int
    kv_heads: int
    head_dim: int
    block_size: int
    dtype: str
    std: float
    seed: int
    ctx_lens: tuple = ()           # fixed cached lengths (overrides ctx_range)
    ctx_range: tuple = (0, 0)
    new_lens: tuple = ()           # fixed new-token counts (overrides new_range)
    new_range: tuple = (1, 1)
    max_len: int = 0               # table width = ceil(max_len / block_size)
    pool_factor: float = 1.25

    @property
    def group(self):
        return self.q_heads // self.kv_heads

    @property
    def table_width(self):
        return -(-self.max_len // self.block_size)

    @property
    def scale(self):
        return self.head_dim ** -0.5

    @property
    def elem_bytes(self):
        return 4 if self.dtype == "f32" else 2


EXTEND_CONFIGS = {
    # Small parity case: empty context, a one-token extend, ragged tiles.
    "x1_extend_tiny_bf16": ExtendConfig(
        name="x1_extend_tiny_bf16", num_seqs=4, q_heads=8, kv_heads=2, head_dim=128,
        block_size=16, dtype="bf16", std=1.0, seed=317_101,
        ctx_lens=(0, 13, 40, 100), new_lens=(37, 1, 64, 29), max_len=160),
    # Recomputation of preempted sequences: whole prompts, nothing cached.
    "x2_prefill_bf16": ExtendConfig(
        name="x2_prefill_bf16", num_seqs=8, q_heads=32, kv_heads=8, head_dim=128,
        block_size=16, dtype="bf16", std=1.0, seed=317_102,
        ctx_range=(0, 0), new_range=(1024, 4096), max_len=4096),
    # Chunked extend: 512 new tokens on top of a long cached context.
    "x3_extend_bf16": ExtendConfig(
        name="x3_extend_bf16", num_seqs=16, q_heads=32, kv_heads=8, head_dim=128,
        block_size=16, dtype="bf16", std=1.0, seed=317_103,
        ctx_range=(2048, 6144), new_range=(512, 512), max_len=6656),
    # Parity: eight query heads per kv head, 32-token blocks.
    "x4_extend_g8_bs32_bf16": ExtendConfig(
        name="x4_extend_g8_bs32_bf16", num_seqs=4, q_heads=64, kv_heads=8, head_dim=128,
        block_size=32, dtype="bf16", std=1.0, seed=317_104,
        ctx_range=(100, 3000), new_range=(1, 300), max_len=3300),
    # Parity: multi-head (one query head per kv head), two heads per group of blocks.
    "x5_extend_mha_bf16": ExtendConfig(
        name="x5_extend_mha_bf16", num_seqs=4, q_heads=16, kv_heads=16, head_dim=128,
        block_size=16, dtype="bf16", std=1.0, seed=317_105,
        ctx_range=(0, 500), new_range=(1, 200), max_len=700),
    # Chunked extend of one long prompt: 1024 new tokens on 40-56 k cached
    # tokens, too few (sequence, kv head, query tile) units to fill the device
    # without splitting the keys.
    "x6_long_extend_bf16": ExtendConfig(
        name="x6_long_extend_bf16", num_seqs=1, q_heads=32, kv_heads=8, head_dim=128,
        block_size=16, dtype="bf16", std=1.0, seed=317_106,
        ctx_range=(40960, 57344), new_range=(1024, 1024), max_len=58368),
}


def get_extend_config(name):
    return EXTEND_CONFIGS[name]


@dataclass
class ExtendWorkload:
    cfg: ExtendConfig
    layout: object
    ctx_lens: np.ndarray            # int32 [S]
    query_start: np.ndarray         # int32 [S + 1]
    q: object
    k_cache: object
    v_cache: object
    new_k: object
    new_v: object
    slot_mapping: object            # int64 [T]
    block_table: object
    seq_lens: object
    query_start_dev: object = None

    @property
    def num_tokens(self):
        return int(self.query_start[-1])

    @property
    def max_query_len(self):
        return int(np.diff(self.query_start).max(initial=0))

    @property
    def max_seq_len(self):
        return int(np.asarray(self.layout.seq_lens).max(initial=0))


def _lengths(rng, fixed, rng_range, S):
    if fixed:
        out = np.asarray(fixed, dtype=np.int64)
        if out.size != S:
            raise ValueError("fixed lengths must have num_seqs entries")
        return out
    lo, hi = rng_range
    return rng.integers(lo, hi + 1, size=S).astype(np.int64)


def extend_layout(cfg, rng):
    """(ctx, new, layout) of ``cfg``, drawing from ``rng``."""
    S = cfg.num_seqs
    ctx = _lengths(rng, cfg.ctx_lens, cfg.ctx_range, S)
    new = _lengths(rng, cfg.new_lens, cfg.new_range, S)
    dec = DecodeConfig(name=cfg.name, num_seqs=S, q_heads=cfg.q_heads, kv_heads=cfg.kv_heads,
                       head_dim=cfg.head_dim, block_size=cfg.block_size, dtype=cfg.dtype,
                       std=cfg.std, seed=cfg.seed, seq_lens=tuple(int(x) for x in ctx + new),
                       max_len=cfg.max_len, pool_factor=cfg.pool_factor)
    return ctx, new, build_layout(dec, rng)


def extend_slots(block_table, seq_lens, query_start, block_size):
    """int64 slot of every new token, in query order: sequence ``s``'s
    query ``j`` is position ``L - n + j``."""
    qs = np.asarray(query_start, dtype=np.int64)
    slots = np.empty(int(qs[-1]), dtype=np.int64)
    for s in range(qs.size - 1):
        n, L = int(qs[s + 1] - qs[s]), int(seq_lens[s])
        t = np.arange(L - n, L)
        slots[qs[s]:qs[s + 1]] = block_table[s, t // block_size].astype(np.int64) * block_size \
            + t % block_size
    return slots


def generate_extend_host(cfg):
    rng = np.random.default_rng(cfg.seed)
    ctx, new, lay = extend_layout(cfg, rng)
    qs = np.zeros(cfg.num_seqs + 1, dtype=np.int32)
    qs[1:] = np.cumsum(new)
    T, Hq, Hkv, D, BS = int(qs[-1]), cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.block_size
    q = _draw_host(rng, (T, Hq, D), cfg)
    k_cache = _draw_host(rng, (lay.num_blocks, BS, Hkv, D), cfg)
    v_cache = _draw_host(rng, (lay.num_blocks, BS, Hkv, D), cfg)
    new_k = _draw_host(rng, (T, Hkv, D), cfg)
    new_v = _draw_host(rng, (T, Hkv, D), cfg)
    slots = extend_slots(lay.block_table, lay.seq_lens, qs, BS)
    return ExtendWorkload(cfg=cfg, layout=lay, ctx_lens=ctx.astype(np.int32), query_start=qs,
                          q=q, k_cache=k_cache, v_cache=v_cache, new_k=new_k, new_v=new_v,
                          slot_mapping=slots, block_table=lay.block_table,
                          seq_lens=lay.seq_lens)


def generate_extend_device(cfg, device="cuda"):
    import torch

    rng = np.random.default_rng(cfg.seed)
    ctx, new, lay = extend_layout(cfg, rng)
    qs = np.zeros(cfg.num_seqs + 1, dtype=np.int32)
    qs[1:] = np.cumsum(new)
    T, Hq, Hkv, D, BS = int(qs[-1]), cfg.q_heads, cfg.kv_heads, cfg.head_dim, cfg.block_size
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

    q = draw((T, Hq, D))
    k_cache = draw((lay.num_blocks, BS, Hkv, D))
    v_cache = draw((lay.num_blocks, BS, Hkv, D))
    new_k = draw((T, Hkv, D))
    new_v = draw((T, Hkv, D))
    slots = extend_slots(lay.block_table, lay.seq_lens, qs, BS)
    return ExtendWorkload(
        cfg=cfg, layout=lay, ctx_lens=ctx.astype(np.int32), query_start=qs,
        q=q, k_cache=k_cache, v_cache=v_cache, new_k=new_k, new_v=new_v,
        slot_mapping=torch.from_numpy(slots).to(device),
        block_table=torch.from_numpy(lay.block_table).to(device),
        seq_lens=torch.from_numpy(lay.seq_lens).to(device),
        query_start_dev=torch.from_numpy(qs).to(device))
