"""Pins of the oracle's bf16 widening, slot write and block copy."""

import numpy as np
import pytest
import torch

import oracle
from oracle.block_manager import BlockManager


def test_widen_matches_torch_on_every_bf16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_widen_known_values():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x3FC0: 1.5, 0x0001: 2.0 ** -133,
             0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x8000: -0.0}
    got = oracle.widen(np.array(list(cases), dtype=np.uint16), "bf16")
    assert list(got) == list(cases.values())


def test_widen_rejects_wrong_storage():
    with pytest.raises(TypeError):
        oracle.widen(np.zeros(3, np.float32), "bf16")
    with pytest.raises(TypeError):
        oracle.widen(np.zeros(3, np.uint16), "f32")


# --- slot write ------------------------------------------------------------------

def _flat_write(cache, rows, slots):
    """Element loop over the flat row-major pool: slot s's row starts at s*Hkv*D."""
    out = cache.copy()
    flat = out.reshape(-1)
    row = int(np.prod(cache.shape[2:]))
    for i, s in enumerate(slots):
        if s < 0:
            continue
        src = rows[i].reshape(-1)
        for j in range(row):
            flat[s * row + j] = src[j]
    return out


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_kv_write_matches_flat_element_loop(dtype):
    rng = np.random.default_rng(20)
    NB, BS, Hkv, D, T = 6, 4, 2, 3, 9
    kc = rng.integers(0, 60000, (NB, BS, Hkv, D)).astype(dtype)
    vc = rng.integers(0, 60000, (NB, BS, Hkv, D)).astype(dtype)
    k = rng.integers(0, 60000, (T, Hkv, D)).astype(dtype)
    v = rng.integers(0, 60000, (T, Hkv, D)).astype(dtype)
    slots = rng.choice(NB * BS, size=T, replace=False).astype(np.int64)
    slots[[2, 5]] = -1
    gk, gv = oracle.kv_write(kc, vc, k, v, slots)
    assert np.array_equal(gk, _flat_write(kc, k, slots))
    assert np.array_equal(gv, _flat_write(vc, v, slots))
    # the input caches are untouched unless asked
    assert not np.array_equal(gk, kc)


def test_kv_write_then_gather_round_trip():
    """Slots from the block manager, scattered, read back through the table."""
    rng = np.random.default_rng(21)
    BS, Hkv, D = 16, 2, 4
    bm = BlockManager(20, BS, free_order=rng.permutation(20))
    bm.add("a")
    bm.add("b")
    sa, _ = bm.append("a", 35)
    sb, _ = bm.append("b", 50)
    ka = rng.standard_normal((35, Hkv, D)).astype(np.float32)
    kb = rng.standard_normal((50, Hkv, D)).astype(np.float32)
    kc = np.full((20, BS, Hkv, D), np.nan, dtype=np.float32)
    kc, _ = oracle.kv_write(kc, kc.copy(), np.concatenate([ka, kb]),
                            np.concatenate([ka, kb]), np.array(sa + sb), inplace=True)
    table = bm.table_array(["a", "b"], 4)
    assert np.array_equal(oracle.gather_sequence(kc, table[0], 35, BS), ka)
    assert np.array_equal(oracle.gather_sequence(kc, table[1], 50, BS), kb)


def test_kv_write_rejects_slot_outside_pool():
    kc = np.zeros((2, 4, 1, 1), np.float32)
    with pytest.raises(IndexError):
        oracle.kv_write(kc, kc, np.ones((1, 1, 1), np.float32), np.ones((1, 1, 1), np.float32),
                        np.array([8]))


# --- block copy --------------------------------------------------------------------

def test_block_copy_semantics():
    rng = np.random.default_rng(22)
    kc = rng.integers(0, 1 << 16, (10, 4, 2, 3)).astype(np.uint16)
    vc = rng.integers(0, 1 << 16, (10, 4, 2, 3)).astype(np.uint16)
    pairs = np.array([[1, 7], [1, 8], [4, 2]])
    gk, gv = oracle.block_copy(kc, vc, pairs)
    for src, dst in pairs:
        assert np.array_equal(gk[dst], kc[src]) and np.array_equal(gv[dst], vc[src])
    untouched = [b for b in range(10) if b not in (7, 8, 2)]
    assert np.array_equal(gk[untouched], kc[untouched])
    assert np.array_equal(gv[untouched], vc[untouched])
    # order of pairs does not matter
    gk2, gv2 = oracle.block_copy(kc, vc, pairs[::-1])
    assert np.array_equal(gk, gk2) and np.array_equal(gv, gv2)


def test_block_copy_rejects_overlapping_pairs():
    kc = np.zeros((4, 2, 1, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.block_copy(kc, kc, [[0, 1], [2, 1]])      # duplicate dst
    with pytest.raises(ValueError):
        oracle.block_copy(kc, kc, [[0, 1], [1, 2]])      # dst is also a src


def test_block_move_matches_an_element_loop_and_round_trips():
    """Two pools of one block shape: every element of each destination block
    is the source block's, element by element (a plain loop, no numpy
    indexing); blocks not named as a destination keep their bits; moving out
    then back into the same ids restores the first pool."""
    rng = np.random.default_rng(9)
    dev_k = rng.integers(0, 1 << 16, size=(12, 4, 2, 3), dtype=np.uint16)
    dev_v = rng.integers(0, 1 << 16, size=(12, 4, 2, 3), dtype=np.uint16)
    host_k = np.zeros((5, 4, 2, 3), np.uint16)
    host_v = np.zeros((5, 4, 2, 3), np.uint16)
    pairs = [(7, 0), (2, 3), (11, 1)]
    hk, hv = oracle.block_move(dev_k, dev_v, host_k, host_v, pairs)
    for b in range(5):
        src = dict((d, s) for s, d in pairs).get(b)
        for i in range(4):
            for j in range(2):
                for e in range(3):
                    want_k = dev_k[src, i, j, e] if src is not None else 0
                    want_v = dev_v[src, i, j, e] if src is not None else 0
                    assert hk[b, i, j, e] == want_k and hv[b, i, j, e] == want_v
    # back into other device blocks, then into the original ones
    cleared_k, cleared_v = dev_k.copy(), dev_v.copy()
    for s, _ in pairs:
        cleared_k[s] = 0
        cleared_v[s] = 0
    back_k, back_v = oracle.block_move(hk, hv, cleared_k, cleared_v, [(d, s) for s, d in pairs])
    assert np.array_equal(back_k, dev_k) and np.array_equal(back_v, dev_v)


def test_block_move_within_one_pool_is_block_copy():
    rng = np.random.default_rng(10)
    k = rng.standard_normal((9, 4, 2, 3)).astype(np.float32)
    v = rng.standard_normal((9, 4, 2, 3)).astype(np.float32)
    pairs = [(1, 4), (1, 5), (8, 0)]
    mk, mv = oracle.block_move(k, v, k, v, pairs)
    ck, cv = oracle.block_copy(k, v, pairs)
    assert np.array_equal(mk, ck) and np.array_equal(mv, cv)


def test_block_move_rejects_bad_pairs():
    k = np.zeros((4, 2, 1, 2), np.float32)
    h = np.zeros((2, 2, 1, 2), np.float32)
    with pytest.raises(IndexError):
        oracle.block_move(k, k, h, h, [(3, 2)])
    with pytest.raises(ValueError):
        oracle.block_move(k, k, h, h, [(0, 1), (2, 1)])
    with pytest.raises(ValueError):
        oracle.block_move(k, k, np.zeros((2, 4, 1, 2), np.float32), h, [(0, 1)])
