"""Pins of the host block manager: the pages' worked example, the waste bound,
on-demand allocation, sharing, copy-on-write and release."""

import json
import os

import numpy as np
import pytest

from oracle.block_manager import BlockManager, OutOfBlocks, blocks_for, tail_waste
from workloads import build_layout, cow_layout, get_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_35_tokens():
    fx = json.load(open(os.path.join(GOLDEN, "worked_example_35_tokens.json")))
    BS, L = fx["block_size"], fx["tokens"]
    assert blocks_for(L, BS) == fx["blocks"]
    assert tail_waste(L, BS) == fx["unused_slots"]
    bm = BlockManager(8, BS)
    bm.add("r")
    bm.append("r", L)
    st = bm.stats()
    assert st["allocated_blocks"] == fx["blocks"]
    assert st["allocated_slots"] == fx["slots"]
    assert st["unused_slots"] == fx["unused_slots"]
    assert round(st["waste_fraction"], 2) == fx["unused_fraction_approx"]
    assert [bm.fill[b] for b in bm.tables["r"]] == fx["block_fill"]


@pytest.mark.parametrize("BS", [1, 8, 16, 32])
def test_waste_bound_brute_force(BS):
    """The only waste is the last block's tail: 0 <= waste <= BS - 1."""
    for L in range(0, 10_001):
        n = blocks_for(L, BS)
        w = tail_waste(L, BS)
        assert 0 <= w <= BS - 1
        assert n * BS >= L and (n - 1) * BS < L or (L == 0 and n == 0)


def test_every_block_but_the_last_is_full():
    for BS in (4, 16):
        for L in range(0, 200, 7):
            bm = BlockManager(64, BS)
            bm.add(0)
            bm.append(0, L)
            fills = [bm.fill[b] for b in bm.tables[0]]
            assert all(f == BS for f in fills[:-1])
            assert sum(fills) == L


def test_allocation_only_when_last_block_is_full():
    bm = BlockManager(10, 4)
    bm.add(0)
    before = []
    for t in range(13):
        before.append(bm.stats()["allocated_blocks"])
        bm.append(0)
        grew = bm.stats()["allocated_blocks"] - before[-1]
        assert grew == (1 if t % 4 == 0 else 0)


def test_slots_follow_the_table():
    bm = BlockManager(6, 16, free_order=[5, 2, 0, 1, 3, 4])
    bm.add(0)
    slots, copies = bm.append(0, 35)
    assert copies == []
    assert bm.tables[0] == [5, 2, 0]
    assert slots == [5 * 16 + i for i in range(16)] + [2 * 16 + i for i in range(16)] + [0, 1, 2]


def test_fork_shares_and_copy_on_write_diverges():
    bm = BlockManager(16, 4)
    bm.add("p")
    bm.append("p", 10)                      # blocks 0, 1 full; block 2 holds 2 tokens
    bm.fork("p", "c1")
    bm.fork("p", "c2")
    assert [bm.refcount[b] for b in bm.tables["p"]] == [3, 3, 3]
    slots, copies = bm.append("c1")         # writes into the shared partial block
    assert copies == [(2, 3)]
    assert bm.tables["c1"] == [0, 1, 3] and bm.tables["p"] == [0, 1, 2]
    assert bm.refcount[2] == 2 and bm.refcount[3] == 1
    assert slots == [3 * 4 + 2]
    _, copies = bm.append("c2")
    assert copies == [(2, 4)]
    _, copies = bm.append("p")              # last holder writes in place
    assert copies == [] and bm.tables["p"] == [0, 1, 2] and bm.refcount[2] == 1


def test_free_returns_blocks_when_unreferenced():
    bm = BlockManager(8, 4)
    bm.add("a")
    bm.append("a", 8)
    bm.fork("a", "b")
    bm.append("b", 1)                       # new block for b only
    bm.free_sequence("a")
    assert bm.stats()["allocated_blocks"] == 3     # shared two stay for b
    bm.free_sequence("b")
    st = bm.stats()
    assert st["allocated_blocks"] == 0 and st["free_blocks"] == 8


def test_out_of_blocks():
    bm = BlockManager(2, 4)
    bm.add(0)
    bm.append(0, 8)
    with pytest.raises(OutOfBlocks):
        bm.append(0, 1)


def test_short_requests_pay_a_whole_block_each():
    """[GL] "What people get wrong": capacity is counted in whole pages, so
    thousands of short requests still hold one block each."""
    BS, n = 16, 4096
    bm = BlockManager(n, BS)
    for s in range(n):
        bm.add(s)
        bm.append(s, 1 + s % 4)           # 1..4 tokens, 2.5 on average
    st = bm.stats()
    assert st["allocated_blocks"] == n and st["free_blocks"] == 0
    assert st["used_slots"] == 10_240     # 1024 requests of each length 1..4
    assert st["unused_slots"] == n * BS - 10_240
    assert st["waste_fraction"] == 1 - 10_240 / (n * BS)   # 84.4%
    bm.add(n)
    with pytest.raises(OutOfBlocks):
        bm.append(n, 1)


def test_c4_layout_replays_through_the_block_manager():
    """Fork 128 sequences from a 1024-token prefix, then append each suffix."""
    cfg = get_config("c4_prefix_bf16")
    lay = build_layout(cfg)
    S, BS = cfg.num_seqs, cfg.block_size
    order = list(lay.shared_blocks) + [int(b) for b in lay.block_table[:, 64:].ravel() if b >= 0]
    order += list(lay.spare_blocks)
    bm = BlockManager(lay.num_blocks, BS, free_order=order)
    bm.add(0)
    bm.append(0, cfg.prefix_tokens)
    for s in range(1, S):
        bm.fork(0, s)
    assert all(bm.refcount[b] == S for b in lay.shared_blocks)
    for s in range(S):
        _, copies = bm.append(s, int(lay.seq_lens[s]) - cfg.prefix_tokens)
        assert copies == []                 # whole-block prefix: no copy needed
    assert np.array_equal(bm.table_array(list(range(S)), cfg.table_width), lay.block_table)


@pytest.mark.parametrize("prefix", [1016, 1024])
def test_cow_scenario_matches_block_manager(prefix):
    cfg = get_config("c4_prefix_bf16")
    lay = build_layout(cfg)
    sc = cow_layout(lay, prefix)
    S, BS = cfg.num_seqs, cfg.block_size
    nshared = -(-prefix // BS)
    order = list(lay.shared_blocks[:nshared]) + list(lay.spare_blocks)
    order += [b for b in range(lay.num_blocks) if b not in set(order)]
    bm = BlockManager(lay.num_blocks, BS, free_order=order)
    holder = S - 1                           # the sequence that ends up writing in place
    bm.add(holder)
    w = sc["write_position"]
    bm.append(holder, w)                     # positions 0 .. w-1
    for s in range(S - 1):
        bm.fork(holder, s)
    assert np.array_equal(bm.table_array(list(range(S)), cfg.table_width),
                          np.where(np.arange(cfg.table_width) < -(-w // BS),
                                   sc["table_before"], -1))
    pairs, slots = [], []
    for s in range(S):
        sl, cp = bm.append(s)
        pairs += cp
        slots += sl
    assert w % BS != 0                       # the write lands in a partly filled block
    assert np.array_equal(np.array(pairs), sc["pairs"])
    assert np.array_equal(np.array(slots), sc["write_slots"])
    assert np.array_equal(bm.table_array(list(range(S)), cfg.table_width), sc["table_after"])


# --- prefix cache --------------------------------------------------------------------

def test_identical_prompt_reuses_its_full_blocks():
    bm = BlockManager(32, 4)
    prompt = list(range(100, 111))                 # 11 tokens: 2 full blocks + 3
    assert bm.add_cached("a", prompt) == 0         # nothing cached yet
    bm.append_tokens("a", prompt)
    assert bm.add_cached("b", prompt) == 8         # the two full blocks
    assert bm.tables["b"] == bm.tables["a"][:2]
    assert all(bm.refcount[b] == 2 for b in bm.tables["a"][:2])
    assert bm.refcount[bm.tables["a"][2]] == 1     # partial block not shared


def test_reuse_stops_at_the_first_differing_block():
    bm = BlockManager(32, 4)
    base = list(range(20))
    bm.add_cached(0, [])
    bm.append_tokens(0, base)
    other = base[:9] + [999] + base[10:]           # differs inside block 2
    assert bm.add_cached(1, other) == 8
    assert bm.add_cached(2, [7] + base[1:]) == 0   # differs in block 0


def test_nothing_is_found_after_the_holder_leaves():
    bm = BlockManager(16, 4)
    bm.add_cached(0, [])
    bm.append_tokens(0, range(8))
    bm.free_sequence(0)
    assert bm.add_cached(1, range(8)) == 0
    assert bm.stats()["cached_blocks"] == 0


def test_plain_append_stops_registration():
    bm = BlockManager(16, 4)
    bm.add_cached(0, [])
    bm.append(0, 8)                                # token ids unknown
    with pytest.raises(ValueError):
        bm.append_tokens(0, [1])
    assert bm.stats()["cached_blocks"] == 0


def test_shared_prefix_batch_from_token_ids():
    """128 requests with one 1024-token prefix share its 64 blocks, as in the
    shared-prefix workload."""
    rng = np.random.default_rng(4)
    prefix = rng.integers(0, 32000, 1024).tolist()
    bm = BlockManager(4000, 16)
    for s in range(128):
        suffix = rng.integers(0, 32000, int(rng.integers(1, 513))).tolist()
        reused = bm.add_cached(s, prefix + suffix)
        assert reused == (0 if s == 0 else 1024)
        bm.append_tokens(s, (prefix + suffix)[reused:])
    tables = [bm.tables[s][:64] for s in range(128)]
    assert all(t == tables[0] for t in tables)
    assert all(bm.refcount[b] == 128 for b in tables[0])
    assert bm.stats()["reused_blocks"] == 127 * 64


# --- swapping ------------------------------------------------------------------------

def test_swap_out_and_in_round_trip():
    bm = BlockManager(8, 4)
    bm.set_swap_space(6)
    bm.add(0)
    bm.append(0, 10)                             # 3 blocks, last holds 2
    table = list(bm.tables[0])
    out = bm.swap_out(0)
    assert [d for d, _ in out] == table and len({h for _, h in out}) == 3
    st = bm.stats()
    assert st["allocated_blocks"] == 0 and st["host_blocks_used"] == 3
    assert st["swapped_sequences"] == 1 and st["swap_outs"] == 1
    back = bm.swap_in(0)
    assert [h for h, _ in back] == [h for _, h in out]
    assert bm.lengths[0] == 10 and len(bm.tables[0]) == 3
    assert bm.stats()["used_slots"] == 10 and bm.stats()["host_blocks_used"] == 0
    slots, _ = bm.append(0, 1)                   # grows again in its last block
    assert slots == [bm.tables[0][2] * 4 + 2]


def test_swap_keeps_shared_blocks_for_the_others():
    bm = BlockManager(8, 4)
    bm.set_swap_space(8)
    bm.add(0)
    bm.append(0, 8)
    bm.fork(0, 1)
    bm.swap_out(1)
    assert all(bm.refcount[b] == 1 for b in bm.tables[0])
    bm.swap_in(1)
    assert set(bm.tables[1]).isdisjoint(bm.tables[0])   # no sharing after a swap


def test_swap_refusals_and_free_while_swapped():
    bm = BlockManager(5, 4)
    bm.set_swap_space(2)
    bm.add(0)
    bm.append(0, 12)                             # 3 blocks > 2 host blocks
    with pytest.raises(OutOfBlocks):
        bm.swap_out(0)
    assert bm.lengths[0] == 12 and bm.stats()["host_blocks_used"] == 0
    bm.add(1)
    bm.append(1, 5)
    bm.swap_out(1)
    bm.append(0, 4)                              # takes one of the two freed blocks
    with pytest.raises(OutOfBlocks):
        bm.swap_in(1)                            # needs 2, device has 1
    bm.free_sequence(1)                          # finished while swapped out
    st = bm.stats()
    assert st["host_blocks_used"] == 0 and st["swapped_sequences"] == 0
