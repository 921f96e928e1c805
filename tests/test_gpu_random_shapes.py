"""Seeded random shapes across the supported space, decode and extend, each
compared with the fp64 oracle on every output row: lengths on and off block
and tile boundaries, every built G and block size, explicit partition
lengths, sequences of length 0 or 1, random table placement and pool slack;
for decode also groups of sequences sharing leading blocks and table entries
outside the pool."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_317_amd as pkv
from workloads.generate import f32_to_bf16_bits

from helpers import compare, drop_bad_blocks, log, to_device

pytestmark = pytest.mark.gpu


def _pool(rng, lens, BS, Hkv, D, dtype, slack):
    """A pool with each sequence's blocks at random places (the test's own
    layout, built without the workload generator)."""
    nblk = [-(-int(L) // BS) for L in lens]
    NB = sum(nblk) + slack
    perm = rng.permutation(NB)
    MB = max(max(nblk), 1) + int(rng.integers(0, 3))
    table = np.full((len(lens), MB), -1, dtype=np.int32)
    cur = 0
    for s, n in enumerate(nblk):
        table[s, :n] = perm[cur:cur + n]
        cur += n
    shape = (NB, BS, Hkv, D)
    x = rng.standard_normal(shape, dtype=np.float32)
    y = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x), f32_to_bf16_bits(y), table
    return x, y, table


def _values(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("seed", range(32))
def test_decode_random_shapes(seed):
    rng = np.random.default_rng(5000 + seed)
    dtype = "f32" if seed % 4 == 0 else "bf16"
    D = 64 if dtype == "f32" else 128
    BS = int(rng.choice([16, 32]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.integers(1, 40))
    lens = rng.integers(0, 1200, size=S)
    lens[rng.integers(0, S)] = int(rng.choice([0, 1, BS, BS + 1, 16 * 7, 16 * 7 + 3]))
    part = int(rng.choice([0, 0, 16, 64, 256, 512]))
    kc, vc, table = _pool(rng, lens, BS, Hkv, D, dtype, int(rng.integers(0, 20)))
    q = _values(rng, (S, Hkv * G, D), dtype)
    scale = float(rng.uniform(0.02, 0.2))
    # Consecutive sequences (16 / G per group for bf16) share leading blocks
    # in half of the cases, and one table entry lies outside the pool in a
    # quarter of them.
    shared = rng.random() < 0.5
    if shared:
        gs = 16 // G if dtype == "bf16" else int(rng.choice([2, 4]))
        for s0 in range(0, S, gs):
            members = range(s0, min(s0 + gs, S))
            nb = min(-(-int(lens[s]) // BS) for s in members)
            J = int(rng.integers(0, nb + 1))
            for s in members:
                table[s, :J] = table[s0, :J]
    if rng.random() < 0.25:
        s = int(rng.integers(0, S))
        nb = -(-int(lens[s]) // BS)
        if nb:
            table[s, int(rng.integers(0, nb))] = int(rng.choice([-1, kc.shape[0], 1 << 30]))
    log(f"decode seed {seed}: {dtype} S={S} BS={BS} Hkv={Hkv} G={G} part={part} "
        f"shared={shared}")
    max_len = int(lens.max())
    out = pkv.paged_attn_decode(to_device(q, dtype), to_device(kc, dtype), to_device(vc, dtype),
                                to_device(table, None), to_device(lens.astype(np.int32), None),
                                scale, max_len, part_tokens=part)
    torch.cuda.synchronize()
    t2, l2 = drop_bad_blocks(table, lens, BS, kc.shape[0])
    ref = oracle.decode_attention(q, kc, vc, t2, l2, scale, dtype)
    compare(out, ref, dtype)


@pytest.mark.parametrize("dtype,Hkv,G,part", [
    ("bf16", 3, 4, 0),      # one kv head per workgroup, three workgroups per run
    ("bf16", 6, 4, 64),     # two kv heads per workgroup, three per run
    ("bf16", 12, 2, 0),     # four kv heads per workgroup, three per run
    ("bf16", 5, 8, 16),
    ("f32", 6, 2, 0),
])
def test_decode_kv_head_counts_not_a_power_of_two(dtype, Hkv, G, part):
    """Kv head counts that split into 3 or 5 workgroups per run (the run
    mapping without the one-group-per-XCD layout of sharing batches), with
    groups of sequences that share leading blocks; every row against the
    oracle."""
    rng = np.random.default_rng(5600 + Hkv * 10 + G)
    D = 64 if dtype == "f32" else 128
    BS = 16
    S = int(rng.integers(30, 70))
    lens = rng.integers(0, 900, size=S)
    lens[0] = 0
    kc, vc, table = _pool(rng, lens, BS, Hkv, D, dtype, 9)
    gs = 16 // G if dtype == "bf16" else 2
    for s0 in range(0, S, gs):
        members = range(s0, min(s0 + gs, S))
        nb = min(-(-int(lens[s]) // BS) for s in members)
        J = int(rng.integers(0, nb + 1))
        for s in members:
            table[s, :J] = table[s0, :J]
    q = _values(rng, (S, Hkv * G, D), dtype)
    log(f"decode kv heads {Hkv}: {dtype} S={S} G={G} part={part}")
    out = pkv.paged_attn_decode(to_device(q, dtype), to_device(kc, dtype), to_device(vc, dtype),
                                to_device(table, None), to_device(lens.astype(np.int32), None),
                                0.1, int(lens.max()), part_tokens=part)
    torch.cuda.synchronize()
    ref = oracle.decode_attention(q, kc, vc, table, lens, 0.1, dtype)
    compare(out, ref, dtype)


@pytest.mark.parametrize("seed", range(32))
def test_extend_random_shapes(seed):
    rng = np.random.default_rng(6000 + seed)
    BS = int(rng.choice([16, 32]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.integers(1, 8))
    ctx = rng.integers(0, 700, size=S)
    new = rng.integers(0, 300, size=S)
    new[rng.integers(0, S)] = int(rng.choice([0, 1, 63, 64, 65, 256 // G]))
    lens = ctx + new
    kc, vc, table = _pool(rng, lens, BS, Hkv, 128, "bf16", int(rng.integers(0, 20)))
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    T = int(qs[-1])
    q = _values(rng, (max(T, 1), Hkv * G, 128), "bf16")[:T]
    scale = float(rng.uniform(0.02, 0.2))
    part = int(rng.choice([0, 0, 64, 128, 320, 1024]))
    log(f"extend seed {seed}: S={S} T={T} BS={BS} Hkv={Hkv} G={G} part={part}")
    if T == 0:
        pytest.skip("no new tokens drawn")
    out = pkv.paged_attn_extend(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
                                to_device(table, None), to_device(lens.astype(np.int32), None),
                                to_device(qs, None), scale, int(new.max()), int(lens.max()),
                                part_tokens=part)
    torch.cuda.synchronize()
    ref = oracle.extend_attention(q, kc, vc, table, lens, qs, scale, "bf16")
    compare(out, ref, "bf16")


@pytest.mark.parametrize("S,Hkv,G,new_hi,part", [
    (12, 8, 8, 200, 0),      # up to 7 query tiles per sequence, some sequences without any
    (12, 8, 8, 200, 128),    # the same split into 128-key partitions
    (64, 8, 2, 300, 0),      # 64 (sequence, kv head) pairs per XCD: the most that are packed
    (40, 16, 1, 300, 0),     # 80 pairs per XCD: the grid keeps its empty slots
    (43, 12, 1, 100, 0),     # 516 pairs: XCDs 0-3 keep their empty slots, 4-7 pack
])
def test_extend_units_of_uneven_query_tiles(S, Hkv, G, new_hi, part):
    """Sequences with different numbers of new tokens have different numbers
    of query tiles, while the grid has max_query_len's worth for each.  In
    batches of up to 64 sequences whose XCDs hold at most 64 (sequence, kv
    head) pairs each, every workgroup maps its slot onto the live query tiles
    of its XCD's pairs, the empty slots last; otherwise the slots keep their
    fixed places.  Both, on the same XCD mix and split, every output row
    against the oracle."""
    rng = np.random.default_rng(7500 + S + Hkv + part)
    BS = 16
    ctx = rng.integers(0, 120, size=S)
    new = rng.integers(0, new_hi + 1, size=S)
    new[rng.integers(0, S, size=max(1, S // 8))] = 0
    new[rng.integers(0, S)] = new_hi
    lens = ctx + new
    kc, vc, table = _pool(rng, lens, BS, Hkv, 128, "bf16", 9)
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    T = int(qs[-1])
    q = _values(rng, (T, Hkv * G, 128), "bf16")
    scale = 0.09
    log(f"extend uneven query tiles: S={S} Hkv={Hkv} G={G} T={T} part={part}")
    out = pkv.paged_attn_extend(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
                                to_device(table, None), to_device(lens.astype(np.int32), None),
                                to_device(qs, None), scale, int(new.max()), int(lens.max()),
                                part_tokens=part)
    torch.cuda.synchronize()
    ref = oracle.extend_attention(q, kc, vc, table, lens, qs, scale, "bf16")
    compare(out, ref, "bf16")


@pytest.mark.parametrize("S", [40, 80])
def test_extend_split_with_tiles_inside_the_first_partition(S):
    """A split call in which many query tiles' keys fit the first 64-key
    partition (those workgroups store their rows and the merge skips them)
    and the others span two or three partitions, in a batch the workgroups
    rank (40 sequences) and one they keep in batch order (80); every output
    row against the oracle."""
    rng = np.random.default_rng(7700 + S)
    BS, Hkv, G = 16, 2, 4
    ctx = rng.integers(0, 120, size=S)
    new = rng.integers(0, 11, size=S)
    ctx[rng.integers(0, S, size=S // 4)] = 0            # some tiles end below 64 keys
    lens = ctx + new
    kc, vc, table = _pool(rng, lens, BS, Hkv, 128, "bf16", 5)
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    T = int(qs[-1])
    q = _values(rng, (T, Hkv * G, 128), "bf16")
    log(f"extend split, tiles in the first partition: S={S} T={T}")
    assert pkv.extend_partition_tokens(to_device(kc, "bf16"), S, T, Hkv * G, int(new.max()),
                                       int(lens.max()), 64) == 64
    out = pkv.paged_attn_extend(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
                                to_device(table, None), to_device(lens.astype(np.int32), None),
                                to_device(qs, None), 0.09, int(new.max()), int(lens.max()),
                                part_tokens=64)
    torch.cuda.synchronize()
    ref = oracle.extend_attention(q, kc, vc, table, lens, qs, 0.09, "bf16")
    compare(out, ref, "bf16")


@pytest.mark.parametrize("S,ties", [(63, False), (64, False), (65, False), (513, False),
                                    (60, True)])
def test_extend_many_sequences_in_any_unit_order(S, ties):
    """The extend kernel orders its units by each sequence's work when the
    batch has at most 64 sequences (every workgroup ranks them) and keeps the
    batch order beyond: batches just below, at and above that size, a large
    one, and one whose sequences all have the same work (the ranking falls
    back on the sequence index), every output row against the oracle.  Short
    sequences (0-40 cached, 0-5 new tokens), so that the oracle stays
    quick."""
    rng = np.random.default_rng(7000 + S)
    BS, Hkv, G = 16, 2, 4
    if ties:
        ctx = np.full(S, 23)
        new = np.full(S, 3)
    else:
        ctx = rng.integers(0, 41, size=S)
        new = rng.integers(0, 6, size=S)
        new[0] = 0
    lens = ctx + new
    kc, vc, table = _pool(rng, lens, BS, Hkv, 128, "bf16", 7)
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    T = int(qs[-1])
    q = _values(rng, (T, Hkv * G, 128), "bf16")
    scale = 0.09
    log(f"extend order: S={S} T={T} ties={ties}")
    out = pkv.paged_attn_extend(to_device(q, "bf16"), to_device(kc, "bf16"), to_device(vc, "bf16"),
                                to_device(table, None), to_device(lens.astype(np.int32), None),
                                to_device(qs, None), scale, int(new.max()), int(lens.max()))
    torch.cuda.synchronize()
    ref = oracle.extend_attention(q, kc, vc, table, lens, qs, scale, "bf16")
    compare(out, ref, "bf16")
