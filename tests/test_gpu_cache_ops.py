"""GPU slot write and block copy against the oracle: bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_317_amd as pkv
from workloads import build_layout, cow_layout, generate_host, get_config, scaled

from helpers import log, to_device, to_host, upload

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
