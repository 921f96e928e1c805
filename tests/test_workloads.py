"""The seeded input generator: determinism and structure of the layouts."""

import numpy as np
import pytest

from workloads import CONFIGS, build_layout, cow_layout, generate_host, get_config, \
    f32_to_bf16_bits, decode_slots, scaled


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    bits = f32_to_bf16_bits(x)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa (1.0) wins;
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even (1+2^-6) wins
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]


def test_host_generation_is_deterministic():
    cfg = get_config("c1_tiny_f32")
    a, b = generate_host(cfg), generate_host(cfg)
    for name in ("q", "k_cache", "v_cache", "new_k", "new_v", "slot_mapping", "block_table"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name


def test_c1_layout():
    cfg = get_config("c1_tiny_f32")
    lay = build_layout(cfg)
    assert list(lay.seq_lens) == [35, 16, 1, 100]
    assert lay.num_blocks == 32 and lay.used_blocks == 12
    used = lay.block_table[lay.block_table >= 0]
    assert len(set(used.tolist())) == 12
    assert [int((row >= 0).sum()) for row in lay.block_table] == [3, 1, 1, 7]


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_layout_structure(name):
    cfg = CONFIGS[name]
    lay = build_layout(cfg)
    BS = cfg.block_size
    S = cfg.num_seqs
    assert lay.seq_lens.shape == (S,)
    lo, hi = cfg.len_range
    if not cfg.seq_lens:
        assert lay.seq_lens.min() >= lo + cfg.prefix_tokens
        assert lay.seq_lens.max() <= hi + cfg.prefix_tokens
    nblk = -(-lay.seq_lens.astype(np.int64) // BS)
    assert np.array_equal((lay.block_table >= 0).sum(1), nblk)
    for s in range(S):
        row = lay.block_table[s]
        assert np.all(row[: nblk[s]] >= 0) and np.all(row[nblk[s]:] == -1)
    # every referenced id is in the pool; private ids appear once
    used = lay.block_table[lay.block_table >= 0].astype(np.int64)
    assert used.min() >= 0 and used.max() < lay.num_blocks
    shared = set(lay.shared_blocks.tolist())
    private = [b for b in used.tolist() if b not in shared]
    assert len(private) == len(set(private))
    assert set(lay.spare_blocks.tolist()).isdisjoint(used.tolist())
    assert lay.used_blocks + lay.spare_blocks.size == lay.num_blocks
    if cfg.pool_blocks == 0:
        assert lay.num_blocks == int(np.ceil(cfg.pool_factor * lay.used_blocks))


def test_c4_shared_prefix_structure():
    cfg = get_config("c4_prefix_bf16")
    lay = build_layout(cfg)
    assert lay.shared_blocks.size == 64
    assert np.all(lay.block_table[:, :64] == lay.shared_blocks[None, :])
    counts = np.bincount(lay.block_table[lay.block_table >= 0], minlength=lay.num_blocks)
    assert np.all(counts[lay.shared_blocks] == 128)


def test_decode_slots_are_last_positions():
    cfg = get_config("c1_tiny_f32")
    lay = build_layout(cfg)
    slots = decode_slots(lay.block_table, lay.seq_lens, cfg.block_size)
    for s, L in enumerate(lay.seq_lens):
        t = L - 1
        assert slots[s] == lay.block_table[s, t // 16] * 16 + t % 16
    assert decode_slots(lay.block_table, np.array([0, 1, 1, 1]), 16)[0] == -1


def test_cow_layout_pairs_and_tables():
    lay = build_layout(get_config("c4_prefix_bf16"))
    sc = cow_layout(lay, 1016)
    assert sc["pairs"].shape == (127, 2)
    assert np.all(sc["pairs"][:, 0] == lay.shared_blocks[63])
    assert len(set(sc["pairs"][:, 1].tolist())) == 127
    assert np.all(sc["table_after"][127] == sc["table_before"][127])
    assert np.all(sc["table_after"][:127, 63] == sc["pairs"][:, 1])
    assert np.all(sc["write_slots"] % 16 == 8)


# --- prefill / extend batches ------------------------------------------------------

from workloads import (EXTEND_CONFIGS, extend_layout, extend_slots,  # noqa: E402
                       generate_extend_host)


@pytest.mark.parametrize("name", sorted(EXTEND_CONFIGS))
def test_extend_layouts_fit_their_tables(name):
    """Every prefill / extend batch's lengths respect its ranges, fit its
    table width and get distinct in-pool blocks (layout only, no values)."""
    cfg = EXTEND_CONFIGS[name]
    ctx, new, lay = extend_layout(cfg, np.random.default_rng(cfg.seed))
    if not cfg.ctx_lens:
        assert ctx.min() >= cfg.ctx_range[0] and ctx.max() <= cfg.ctx_range[1]
    if not cfg.new_lens:
        assert new.min() >= cfg.new_range[0] and new.max() <= cfg.new_range[1]
    assert np.array_equal(lay.seq_lens, ctx + new)
    assert lay.seq_lens.max() <= cfg.max_len
    assert lay.block_table.shape == (cfg.num_seqs, cfg.table_width)
    used = lay.block_table[lay.block_table >= 0]
    assert used.size == int((-(-lay.seq_lens // cfg.block_size)).sum())
    assert np.unique(used).size == used.size and used.max() < lay.num_blocks


@pytest.mark.parametrize("name", ["x1_extend_tiny_bf16", "x4_extend_g8_bs32_bf16",
                                  "x5_extend_mha_bf16"])
def test_extend_batches_are_consistent(name):
    cfg = EXTEND_CONFIGS[name]
    w = generate_extend_host(cfg)
    lay, BS = w.layout, cfg.block_size
    new = np.diff(w.query_start)
    assert np.array_equal(lay.seq_lens, w.ctx_lens + new)
    assert w.q.shape == (w.num_tokens, cfg.q_heads, cfg.head_dim)
    assert w.new_k.shape == (w.num_tokens, cfg.kv_heads, cfg.head_dim)
    used = lay.block_table[lay.block_table >= 0]
    assert np.unique(used).size == used.size and used.max() < lay.num_blocks
    slots = w.slot_mapping
    assert np.unique(slots).size == slots.size
    for s in range(cfg.num_seqs):
        for j in range(int(new[s])):
            t = int(w.ctx_lens[s]) + j
            row = int(w.query_start[s]) + j
            assert slots[row] == lay.block_table[s, t // BS] * BS + t % BS
    again = generate_extend_host(cfg)
    assert np.array_equal(again.q, w.q) and np.array_equal(again.k_cache, w.k_cache)


def test_extend_slots_of_a_hand_made_table():
    table = np.array([[5, 2, -1], [0, 7, 3]], dtype=np.int32)
    slots = extend_slots(table, np.array([6, 9]), np.array([0, 3, 5]), 4)
    # sequence 0: positions 3, 4, 5; sequence 1: positions 7, 8
    assert slots.tolist() == [5 * 4 + 3, 2 * 4 + 0, 2 * 4 + 1, 7 * 4 + 3, 3 * 4 + 0]


def test_decode_slot_of_the_35_token_example():
    """The worked example of "What does PagedAttention change in LLM KV
    allocation?" ("Calculate unused block space"): 35 tokens at block size
    16 fill blocks 16, 16 and 3, so the newest token (position 34) is the
    third slot of logical block 2, whatever physical block that is."""
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                     "worked_example_35_tokens.json")))
    bs, n = fx["block_size"], fx["tokens"]
    last_block = len(fx["block_fill"]) - 1
    offset = fx["block_fill"][-1] - 1
    table = np.array([[40, 7, 23, -1]], dtype=np.int32)
    slot = decode_slots(table, np.array([n]), bs)[0]
    assert slot == table[0, last_block] * bs + offset == 23 * 16 + 2


@pytest.mark.parametrize("name,kw", [
    ("c1_tiny_f32", {}),
    ("c2_mha_bf16", dict(num_seqs=9, len_range=(1, 700), max_len=704)),
    ("c5_long_bf16", dict(num_seqs=3, len_range=(1, 3000), max_len=3072)),
])
def test_decode_slots_match_the_oracle_block_manager(name, kw):
    """The generator's slot for each sequence's newest token is the slot the
    oracle's block manager hands out for that token when it appends every
    token of the same sequences (blocks taken in the layout's placement
    order), and the manager's tables are the layout's."""
    import oracle
    cfg = scaled(get_config(name), **kw)
    lay = build_layout(cfg)
    BS, S = cfg.block_size, cfg.num_seqs
    order = [int(b) for b in lay.block_table.ravel() if b >= 0] + [int(b) for b in lay.spare_blocks]
    bm = oracle.BlockManager(lay.num_blocks, BS, free_order=order)
    last = []
    for s in range(S):
        bm.add(s)
        slots, copies = bm.append(s, int(lay.seq_lens[s]))
        assert copies == []
        last.append(slots[-1])
    assert np.array_equal(bm.table_array(range(S), cfg.table_width), lay.block_table)
    assert np.array_equal(decode_slots(lay.block_table, lay.seq_lens, BS), np.array(last))
