"""GPU slot write and block copy against the oracle: bit for bit."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_317_amd as pkv
from paged_kv_cache_317_amd.block_manager import BlockManager
from workloads import build_layout, cow_layout, generate_host, get_config, scaled

from helpers import compare, log, to_device, to_host, upload

pytestmark = pytest.mark.gpu


def _small(name, **kw):
    return generate_host(scaled(get_config(name), **kw))


@pytest.mark.parametrize("name,kw", [
    ("c1_tiny_f32", {}),
    ("c3_gqa4k_bf16", dict(num_seqs=7, len_range=(20, 90), max_len=128)),
    ("c5_long_bf16", dict(num_seqs=3, len_range=(40, 200), max_len=256, part_tokens=0)),
    ("c2_mha_bf16", dict(num_seqs=5, len_range=(1, 64), max_len=64)),
])
def test_kv_write_bit_exact(name, kw):
    w = _small(name, **kw)
    log(f"kv_write {name} T={len(w.slot_mapping)}")
    d = upload(w)
    slots = w.slot_mapping.copy()
    slots[1] = -1                                  # padding token
    d["slot_mapping"] = to_device(slots, None)
    pkv.paged_kv_write(d["new_k"], d["new_v"], d["slot_mapping"], d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    rk, rv = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, slots)
    assert np.array_equal(to_host(d["k_cache"], w.cfg.dtype), rk)
    assert np.array_equal(to_host(d["v_cache"], w.cfg.dtype), rv)


def test_kv_write_many_tokens_and_guards():
    """A prefill-sized write; slots outside the pool are skipped, not written."""
    cfg = scaled(get_config("c3_gqa4k_bf16"), num_seqs=4, len_range=(100, 200), max_len=256)
    w = generate_host(cfg)
    rng = np.random.default_rng(5)
    nslots = w.layout.num_blocks * cfg.block_size
    T = 700
    slots = rng.choice(nslots, size=T, replace=False).astype(np.int64)
    slots[[3, 50]] = nslots + 7                    # outside the pool: skipped
    slots[[4, 60]] = -5
    k = rng.integers(0, 1 << 16, (T, cfg.kv_heads, cfg.head_dim)).astype(np.uint16)
    v = rng.integers(0, 1 << 16, (T, cfg.kv_heads, cfg.head_dim)).astype(np.uint16)
    d = upload(w)
    pkv.paged_kv_write(to_device(k, "bf16"), to_device(v, "bf16"), to_device(slots, None),
                       d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    ok = slots.copy()
    ok[ok >= nslots] = -1
    rk, rv = oracle.kv_write(w.k_cache, w.v_cache, k, v, ok)
    assert np.array_equal(to_host(d["k_cache"], "bf16"), rk)
    assert np.array_equal(to_host(d["v_cache"], "bf16"), rv)


def test_kv_write_zero_tokens_is_a_noop():
    w = _small("c1_tiny_f32")
    d = upload(w)
    empty = torch.empty((0, 8, 64), dtype=torch.float32, device="cuda")
    pkv.paged_kv_write(empty, empty, torch.empty(0, dtype=torch.int64, device="cuda"),
                       d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(d["k_cache"], "f32"), w.k_cache)


@pytest.mark.parametrize("prefix", [1016, 1024])
def test_block_copy_cow_pairs_bit_exact(prefix):
    cfg = get_config("c4_prefix_bf16")
    w = generate_host(cfg)
    sc = cow_layout(w.layout, prefix)
    log(f"block_copy c4 prefix={prefix} pairs={len(sc['pairs'])}")
    d = upload(w)
    pkv.paged_block_copy(to_device(sc["pairs"], None), d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    rk, rv = oracle.block_copy(w.k_cache, w.v_cache, sc["pairs"])
    assert np.array_equal(to_host(d["k_cache"], "bf16"), rk)
    assert np.array_equal(to_host(d["v_cache"], "bf16"), rv)


def test_block_copy_f32_block32_and_guards():
    cfg = scaled(get_config("c1_tiny_f32"), block_size=32, max_len=128)
    w = generate_host(cfg)
    NB = w.layout.num_blocks
    pairs = np.array([[0, 5], [3, 7], [NB + 2, 1], [2, -1], [6, 4]], dtype=np.int64)
    d = upload(w)
    pkv.paged_block_copy(to_device(pairs, None), d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    valid = pairs[[0, 1, 4]]
    rk, rv = oracle.block_copy(w.k_cache, w.v_cache, valid)
    assert np.array_equal(to_host(d["k_cache"], "f32"), rk)
    assert np.array_equal(to_host(d["v_cache"], "f32"), rv)


def test_block_copy_zero_pairs_is_a_noop():
    w = _small("c1_tiny_f32")
    d = upload(w)
    pkv.paged_block_copy(torch.empty((0, 2), dtype=torch.int64, device="cuda"),
                         d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(d["k_cache"], "f32"), w.k_cache)


def test_ops_replay_correctly_inside_a_captured_graph():
    """Slot write, decode and block copy captured in one HIP graph, replayed
    several times with eager work in between; every replay matches eager."""
    cfg = scaled(get_config("c5_long_bf16"), num_seqs=3, len_range=(600, 1500), max_len=1536,
                 part_tokens=256)
    w = generate_host(cfg)
    d = upload(w)
    lay = w.layout
    pairs = torch.from_numpy(np.stack([lay.spare_blocks[:2], lay.spare_blocks[2:4]], 1)
                             .astype(np.int64)).cuda()
    out = torch.empty_like(d["q"])
    ws = torch.empty(pkv.decode_workspace_size(d["k_cache"], cfg.num_seqs, cfg.q_heads,
                                               lay.max_seq_len, cfg.part_tokens),
                     dtype=torch.uint8, device="cuda")

    def step():
        pkv.paged_kv_write(d["new_k"], d["new_v"], d["slot_mapping"], d["k_cache"], d["v_cache"])
        pkv.paged_block_copy(pairs, d["k_cache"], d["v_cache"])
        pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"], d["seq_lens"],
                              cfg.scale, lay.max_seq_len, out=out, part_tokens=cfg.part_tokens,
                              workspace=ws)

    step()
    torch.cuda.synchronize()
    eager_out = out.clone()
    eager_k, eager_v = d["k_cache"].clone(), d["v_cache"].clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.zero_()
        d["k_cache"].copy_(to_device(w.k_cache, "bf16"))
        d["v_cache"].copy_(to_device(w.v_cache, "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), f"replay {r}"
        assert torch.equal(d["k_cache"].view(torch.int16), eager_k.view(torch.int16))
        assert torch.equal(d["v_cache"].view(torch.int16), eager_v.view(torch.int16))


# --- block move between the device pool and a pinned host pool (swapping) ---------

def _pinned_pool(shape, dtype):
    return torch.zeros(shape, dtype=dtype).pin_memory()


# Block shapes around the copy kernel's 32 KiB chunk: 8 KiB (f32, 2 kv
# heads, head_dim 64: one partial chunk) and 48 KiB (bf16, 12 kv heads: one
# whole chunk and a half).
PARTIAL_CHUNK_SHAPES = [
    ("c1_tiny_f32", dict(q_heads=2, kv_heads=2)),
    ("c3_gqa4k_bf16", dict(num_seqs=6, q_heads=12, kv_heads=12, len_range=(30, 200),
                           max_len=256)),
]


@pytest.mark.parametrize("name,kw", PARTIAL_CHUNK_SHAPES)
def test_block_copy_partial_chunks_bit_exact(name, kw):
    """Blocks that are not a whole number of the kernel's 32 KiB chunks."""
    cfg = scaled(get_config(name), **kw)
    w = generate_host(cfg)
    NB = w.layout.num_blocks
    rng = np.random.default_rng(5)
    ids = rng.choice(NB, size=12, replace=False)
    pairs = np.stack([ids[:6], ids[6:]], 1).astype(np.int64)
    log(f"block_copy {name} {kw} block_bytes={w.k_cache[0].nbytes} pairs={len(pairs)}")
    d = upload(w)
    pkv.paged_block_copy(to_device(pairs, None), d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    rk, rv = oracle.block_copy(w.k_cache, w.v_cache, pairs)
    assert np.array_equal(to_host(d["k_cache"], cfg.dtype), rk)
    assert np.array_equal(to_host(d["v_cache"], cfg.dtype), rv)


@pytest.mark.parametrize("name,kw", [
    ("c1_tiny_f32", {}),
    ("c3_gqa4k_bf16", dict(num_seqs=6, len_range=(30, 200), max_len=256)),
] + PARTIAL_CHUNK_SHAPES)
def test_block_move_device_host_device_bit_exact(name, kw):
    cfg = scaled(get_config(name), **kw)
    w = generate_host(cfg)
    d = upload(w)
    NB = w.layout.num_blocks
    rng = np.random.default_rng(11)
    HB = 40
    src = rng.choice(NB, size=24, replace=False)
    host = rng.choice(HB, size=24, replace=False)
    out_pairs = np.stack([src, host], 1).astype(np.int64)
    log(f"block_move d2h {name} pairs={len(out_pairs)}")
    hk = _pinned_pool((HB,) + tuple(d["k_cache"].shape[1:]), d["k_cache"].dtype)
    hv = _pinned_pool((HB,) + tuple(d["v_cache"].shape[1:]), d["v_cache"].dtype)
    pkv.paged_block_move(to_device(out_pairs, None), d["k_cache"], d["v_cache"], hk, hv)
    torch.cuda.synchronize()
    zeros = np.zeros((HB,) + w.k_cache.shape[1:], w.k_cache.dtype)
    ek, ev = oracle.block_move(w.k_cache, w.v_cache, zeros, zeros, out_pairs)
    assert np.array_equal(to_host(hk, cfg.dtype), ek)
    assert np.array_equal(to_host(hv, cfg.dtype), ev)
    # back into other device blocks; pairs in pinned host memory this time
    dst = rng.choice(NB, size=24, replace=False)
    in_pairs = torch.from_numpy(np.stack([host, dst], 1).astype(np.int64)).pin_memory()
    log(f"block_move h2d {name} pairs={len(in_pairs)}")
    pkv.paged_block_move(in_pairs, hk, hv, d["k_cache"], d["v_cache"])
    torch.cuda.synchronize()
    rk, rv = oracle.block_move(ek, ev, w.k_cache, w.v_cache, in_pairs.numpy())
    assert np.array_equal(to_host(d["k_cache"], cfg.dtype), rk)
    assert np.array_equal(to_host(d["v_cache"], cfg.dtype), rv)


def test_decode_is_unchanged_by_a_swap_round_trip():
    """Every sequence swapped out, the device pool cleared, then swapped back
    into other blocks (through the native block manager's pairs): decode over
    the new tables gives the rows the oracle gives for the old ones."""
    cfg = scaled(get_config("c4_prefix_bf16"), num_seqs=5, prefix_tokens=256,
                 len_range=(1, 200), max_len=512)
    w = generate_host(cfg)
    lay = w.layout
    S, BS = cfg.num_seqs, cfg.block_size
    NB = S * cfg.table_width + 8       # room for the unshared copies after swap-in
    d = upload(w)
    for name in ("k_cache", "v_cache"):
        big = torch.zeros((NB,) + tuple(d[name].shape[1:]), dtype=d[name].dtype, device="cuda")
        big[:lay.num_blocks] = d[name]
        d[name] = big
    before = pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                   d["seq_lens"], cfg.scale, lay.max_seq_len)
    torch.cuda.synchronize()
    # A manager that holds the same tables: forks of the shared prefix, then suffixes.
    nshared = len(lay.shared_blocks)
    order = list(lay.shared_blocks) + [int(b) for b in lay.block_table[:, nshared:].ravel()
                                       if b >= 0] + list(lay.spare_blocks)
    order += list(range(lay.num_blocks, NB))
    bm = BlockManager(NB, BS, free_order=order)
    bm.set_swap_space(NB)
    bm.add(0)
    bm.append(0, cfg.prefix_tokens)
    for s in range(1, S):
        bm.fork(0, s)
    for s in range(S):
        bm.append(s, int(lay.seq_lens[s]) - cfg.prefix_tokens)
    assert np.array_equal(bm.table_array(range(S), cfg.table_width), lay.block_table)
    hk = _pinned_pool(tuple(d["k_cache"].shape), torch.bfloat16)
    hv = _pinned_pool(tuple(d["v_cache"].shape), torch.bfloat16)
    moves = []
    for s in range(S):
        moves += bm.swap_out(s)
    log(f"swap out {len(moves)} blocks")
    pkv.paged_block_move(torch.tensor(moves, dtype=torch.int64, device="cuda"),
                         d["k_cache"], d["v_cache"], hk, hv)
    d["k_cache"].zero_()
    d["v_cache"].zero_()
    bm.add(S)                                       # shifts where swapped blocks land
    bm.append(S, 3 * BS)
    moves = []
    for s in reversed(range(S)):
        moves += bm.swap_in(s)
    log(f"swap in {len(moves)} blocks")
    pkv.paged_block_move(torch.tensor(moves, dtype=torch.int64, device="cuda"),
                         hk, hv, d["k_cache"], d["v_cache"])
    table = bm.table_array(range(S), cfg.table_width)
    assert not np.array_equal(table, lay.block_table)
    after = pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], to_device(table, None),
                                  d["seq_lens"], cfg.scale, lay.max_seq_len)
    torch.cuda.synchronize()
    # The blocks' contents are back bit for bit, so the oracle gives the same
    # rows before and after.  Sharing does not survive a swap: the prefix is
    # now held privately and the GPU splits the work differently, so its
    # rows agree to the tolerance, not bitwise.
    kc_after = to_host(d["k_cache"], cfg.dtype)
    vc_after = to_host(d["v_cache"], cfg.dtype)
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, lay.block_table, lay.seq_lens,
                                  cfg.scale, cfg.dtype)
    assert np.array_equal(ref, oracle.decode_attention(w.q, kc_after, vc_after, table,
                                                       lay.seq_lens, cfg.scale, cfg.dtype))
    compare(before, ref, cfg.dtype)
    compare(after, ref, cfg.dtype)
    assert bm.stats()["swap_outs"] == S and bm.stats()["host_blocks_used"] == 0


def test_block_move_guards():
    """Pairs outside either pool are skipped; pageable host memory and
    mismatched block shapes are refused before any launch."""
    cfg = scaled(get_config("c1_tiny_f32"), max_len=128)
    w = generate_host(cfg)
    d = upload(w)
    NB = w.layout.num_blocks
    hk = _pinned_pool((4,) + tuple(d["k_cache"].shape[1:]), torch.float32)
    hv = _pinned_pool((4,) + tuple(d["v_cache"].shape[1:]), torch.float32)
    pairs = np.array([[1, 0], [NB, 1], [2, 4], [-1, 2], [3, 3]], dtype=np.int64)
    pkv.paged_block_move(to_device(pairs, None), d["k_cache"], d["v_cache"], hk, hv)
    torch.cuda.synchronize()
    ek = np.zeros((4,) + w.k_cache.shape[1:], np.float32)
    ek[0], ek[3] = w.k_cache[1], w.k_cache[3]
    assert np.array_equal(hk.numpy(), ek)
    assert not hv[1].any() and not hv[2].any()
    # pageable pools: the library refuses them (every pair is also outside
    # the pools, so no launch could touch them either way)
    lib = pkv._lib.lib()
    desc = pkv._lib.CacheDesc(4, cfg.block_size, cfg.kv_heads, cfg.head_dim, pkv._lib.PKV_F32)
    ddesc = pkv._lib.CacheDesc(NB, cfg.block_size, cfg.kv_heads, cfg.head_dim, pkv._lib.PKV_F32)
    pageable = np.zeros((4,) + w.k_cache.shape[1:], np.float32)
    skip = to_device(np.array([[-1, -1]], dtype=np.int64), None)
    st = lib.pkv_paged_block_move(skip.data_ptr(), 1, d["k_cache"].data_ptr(),
                                  d["v_cache"].data_ptr(), ctypes.byref(ddesc),
                                  pageable.ctypes.data, pageable.ctypes.data,
                                  ctypes.byref(desc), None)
    assert pkv._lib.STATUS_NAMES[st] == "PKV_ERR_UNSUPPORTED"
    with pytest.raises(ValueError):
        pkv.paged_block_move(skip, d["k_cache"], d["v_cache"], torch.zeros_like(hk),
                             torch.zeros_like(hv))
    bad = _pinned_pool((4, cfg.block_size * 2, cfg.kv_heads, cfg.head_dim), torch.float32)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_block_move(skip, d["k_cache"], d["v_cache"], bad, bad)
    assert e.value.status_name == "PKV_ERR_SHAPE"
