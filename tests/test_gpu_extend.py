"""Prefill / chunked-extend attention on the GPU against the oracle.

Each case writes the new tokens' K/V rows with the slot-write kernel, then
runs the extend kernel, as one step of a prefill does; the oracle applies
its own slot write to the host pools and computes every (or a sampled set
of) query rows in float64.  Tolerance: the bf16 decode bar (global max-abs
2e-2, per-row max-rel 1e-2).
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_317_amd as pkv
from workloads import EXTEND_CONFIGS, generate_extend_device, generate_extend_host

from helpers import compare, log, to_device, to_host

pytestmark = pytest.mark.gpu


def _upload(w):
    dt = w.cfg.dtype
    return {
        "q": to_device(w.q, dt), "k_cache": to_device(w.k_cache, dt),
        "v_cache": to_device(w.v_cache, dt), "new_k": to_device(w.new_k, dt),
        "new_v": to_device(w.new_v, dt), "slot_mapping": to_device(w.slot_mapping, None),
        "block_table": to_device(w.block_table, None), "seq_lens": to_device(w.seq_lens, None),
        "query_start": to_device(w.query_start, None),
    }


def _step(d, cfg, max_query_len, max_seq_len, out=None, part_tokens=0):
    pkv.paged_kv_write(d["new_k"], d["new_v"], d["slot_mapping"], d["k_cache"], d["v_cache"])
    out = pkv.paged_attn_extend(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                d["seq_lens"], d["query_start"], cfg.scale, max_query_len,
                                max_seq_len, out=out, part_tokens=part_tokens)
    torch.cuda.synchronize()
    return out


def _oracle(w, kc=None, vc=None, seqs=None, table=None, lens=None, qs=None):
    return oracle.extend_attention(w.q, w.k_cache if kc is None else kc,
                                   w.v_cache if vc is None else vc,
                                   w.block_table if table is None else table,
                                   w.seq_lens if lens is None else lens,
                                   w.query_start if qs is None else qs, w.cfg.scale, w.cfg.dtype,
                                   seqs=seqs)


@pytest.mark.parametrize("part_tokens", [0, 64, 192, 1024])
@pytest.mark.parametrize("name", ["x1_extend_tiny_bf16", "x4_extend_g8_bs32_bf16",
                                  "x5_extend_mha_bf16"])
def test_extend_matches_the_oracle(name, part_tokens):
    """Whole batches against the oracle, unsplit (0: these batches are too
    short for the library to split) and with the keys cut into partitions of
    64, 192 and 1024 that a merge kernel combines."""
    cfg = EXTEND_CONFIGS[name]
    w = generate_extend_host(cfg)
    log(f"extend {name} part {part_tokens}: T={w.num_tokens} max_q={w.max_query_len} "
        f"pool={w.layout.num_blocks}")
    d = _upload(w)
    out = _step(d, cfg, w.max_query_len, w.max_seq_len, part_tokens=part_tokens)
    kc, vc = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
    ref = _oracle(w, kc, vc)
    mabs, mrel = compare(out, ref, cfg.dtype)
    log(f"  max-abs {mabs:.3e} row max-rel {mrel:.3e}")


@pytest.mark.parametrize("part_tokens", [0, 64])
def test_extend_ignores_unused_slots_and_unreferenced_blocks(part_tokens):
    """NaN in every slot no sequence uses changes nothing, split or not."""
    cfg = EXTEND_CONFIGS["x1_extend_tiny_bf16"]
    w = generate_extend_host(cfg)
    kc, vc = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
    BS = cfg.block_size
    used = np.zeros(kc.shape[:2], dtype=bool)
    for s in range(cfg.num_seqs):
        for t in range(int(w.seq_lens[s])):
            used[w.block_table[s, t // BS], t % BS] = True
    nan = np.uint16(0x7FC0)
    kp, vp = kc.copy(), vc.copy()
    kp[~used] = nan
    vp[~used] = nan
    d = _upload(w)
    d["k_cache"], d["v_cache"] = to_device(kp, "bf16"), to_device(vp, "bf16")
    out = pkv.paged_attn_extend(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                d["seq_lens"], d["query_start"], cfg.scale, w.max_query_len,
                                w.max_seq_len, part_tokens=part_tokens)
    d2 = _upload(w)
    d2["k_cache"], d2["v_cache"] = to_device(kc, "bf16"), to_device(vc, "bf16")
    clean = pkv.paged_attn_extend(d2["q"], d2["k_cache"], d2["v_cache"], d2["block_table"],
                                  d2["seq_lens"], d2["query_start"], cfg.scale, w.max_query_len,
                                  w.max_seq_len, part_tokens=part_tokens)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    assert torch.equal(out.view(torch.int16), clean.view(torch.int16))


@pytest.mark.parametrize("part_tokens", [0, 64])
def test_extend_degenerate_cases(part_tokens):
    """Queries before position 0 and an empty sequence give zero rows; a
    sequence with no new tokens writes nothing; rows past max_query_len are
    left as they were; a table entry outside the pool ends the sequence.
    Split calls give the same rows (partitions with no visible key merge to
    nothing)."""
    cfg = EXTEND_CONFIGS["x1_extend_tiny_bf16"]
    w = generate_extend_host(cfg)
    d = _upload(w)
    lens = w.seq_lens.copy()
    qs = w.query_start.copy()
    # sequence 0: 37 new tokens but L = 20 -> the first 17 queries sit before 0
    lens[0] = 20
    # sequence 1: L = 0 with one query
    lens[1] = 0
    # sequence 3: table cut at logical block 4 (positions >= 64 excluded)
    table = w.block_table.copy()
    table[3, 4] = -7
    d["seq_lens"] = to_device(lens, None)
    d["block_table"] = to_device(table, None)
    sentinel = torch.full_like(d["q"], 3.0)
    out = pkv.paged_attn_extend(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                d["seq_lens"], d["query_start"], cfg.scale, 40,
                                int(lens.max()), out=sentinel, part_tokens=part_tokens)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    ref = _oracle(w, lens=lens, seqs=[0, 1, 2])
    n = np.diff(qs)
    # sequence 0: rows 0..16 zero, rows 17..36 compared
    assert not got[qs[0]:qs[0] + 17].any()
    compare(torch.from_numpy(got[qs[0] + 17:qs[1]]), ref[qs[0] + 17:qs[1]], "bf16")
    assert not got[qs[1]:qs[2]].any()
    # sequence 2: 64 new tokens, only the first 40 written
    compare(torch.from_numpy(got[qs[2]:qs[2] + 40]), ref[qs[2]:qs[2] + 40], "bf16")
    assert np.all(got[qs[2] + 40:qs[3]] == 3.0)
    # sequence 3: its 29 queries sit at positions 100..128, past the cut at
    # 64, so each sees exactly keys 0..63: one query over a 64-token sequence.
    assert n[3] == 29
    for r in range(qs[3], qs[4]):
        row = oracle.extend_attention(w.q[r:r + 1], w.k_cache, w.v_cache, table[3:4, :4],
                                      np.array([64]), np.array([0, 1]), cfg.scale, "bf16")
        compare(torch.from_numpy(got[r:r + 1]), row, "bf16")


@pytest.mark.parametrize("part_tokens", [0, 64])
def test_extend_max_seq_len_cuts_the_keys(part_tokens):
    """A max_seq_len below some lengths cuts those sequences' keys: the query
    at position p sees keys 0 .. min(p + 1, max_seq_len) - 1 (positions keep
    their uncut values); the oracle computes each row as one query over a
    sequence of that many keys."""
    cfg = EXTEND_CONFIGS["x1_extend_tiny_bf16"]
    w = generate_extend_host(cfg)
    cut = 72
    assert w.max_seq_len > cut
    d = _upload(w)
    out = _step(d, cfg, w.max_query_len, cut, part_tokens=part_tokens)
    kc, vc = oracle.kv_write(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping)
    qs, lens = w.query_start, w.seq_lens
    got = out.float().cpu().numpy()
    for s in range(cfg.num_seqs):
        n = int(qs[s + 1] - qs[s])
        for j in range(n):
            r = int(qs[s]) + j
            keys = min(int(lens[s]) - n + j + 1, cut)
            row = oracle.extend_attention(w.q[r:r + 1], kc, vc, w.block_table[s:s + 1],
                                          np.array([keys]), np.array([0, 1]), cfg.scale, "bf16")
            compare(torch.from_numpy(got[r:r + 1]), row, "bf16")


def test_extend_rejects_what_it_does_not_support():
    cfg = EXTEND_CONFIGS["x1_extend_tiny_bf16"]
    w = generate_extend_host(cfg)
    d = _upload(w)
    kf = d["k_cache"].float()
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attn_extend(d["q"].float(), kf, kf, d["block_table"], d["seq_lens"],
                              d["query_start"], cfg.scale, w.max_query_len, w.max_seq_len)
    assert e.value.status_name == "PKV_ERR_UNSUPPORTED"
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_attn_extend(d["q"][:, :6].contiguous(), d["k_cache"], d["v_cache"],
                              d["block_table"], d["seq_lens"], d["query_start"], cfg.scale,
                              w.max_query_len, w.max_seq_len)
    assert e.value.status_name == "PKV_ERR_UNSUPPORTED"      # G = 3


@pytest.mark.parametrize("name,nsample,part", [("x2_prefill_bf16", 3, 0), ("x3_extend_bf16", 4, 0),
                                               ("x3_extend_bf16", 2, 1024)])
def test_extend_full_size_sampled(name, nsample, part):
    """Full-size batches drawn on the device; the oracle computes a seeded
    sample of sequences (plus the longest) from the pools copied back.  The
    chunked-extend batch also runs split into 1024-key partitions."""
    cfg = EXTEND_CONFIGS[name]
    w = generate_extend_device(cfg)
    log(f"extend full {name} part {part}: T={w.num_tokens} pool={w.layout.num_blocks}")
    d = {"q": w.q, "k_cache": w.k_cache, "v_cache": w.v_cache, "new_k": w.new_k,
         "new_v": w.new_v, "slot_mapping": w.slot_mapping, "block_table": w.block_table,
         "seq_lens": w.seq_lens, "query_start": w.query_start_dev}
    out = _step(d, cfg, w.max_query_len, w.max_seq_len, part_tokens=part)
    kc, vc = to_host(w.k_cache, "bf16"), to_host(w.v_cache, "bf16")
    q = to_host(w.q, "bf16")
    rng = np.random.default_rng(7)
    lens = w.layout.seq_lens
    seqs = sorted(set(rng.choice(cfg.num_seqs, nsample, replace=False).tolist())
                  | {int(np.argmax(lens))})
    qs = w.query_start
    ref = oracle.extend_attention(q, kc, vc, w.layout.block_table, lens, qs, cfg.scale, "bf16",
                                  seqs=seqs)
    rows = np.concatenate([np.arange(qs[s], qs[s + 1]) for s in seqs])
    mabs, mrel = compare(out, ref, "bf16", rows=rows)
    log(f"  sequences {seqs}: max-abs {mabs:.3e} row max-rel {mrel:.3e}")


def test_extend_long_context_split_sampled():
    """One prompt with 40-56 k cached tokens and 1024 new ones: too few units
    to fill the device, so the library splits the keys.  The oracle checks
    windows of 16 consecutive queries (first, middle, last of each sequence)
    for two kv heads: a window [a, b) of sequence s is the same problem as a
    sequence of length ctx + b whose new tokens are those b - a queries."""
    cfg = EXTEND_CONFIGS["x6_long_extend_bf16"]
    w = generate_extend_device(cfg)
    T, Hq, G = w.num_tokens, cfg.q_heads, cfg.group
    part = pkv.extend_partition_tokens(w.k_cache, cfg.num_seqs, T, Hq, w.max_query_len,
                                       w.max_seq_len)
    log(f"extend long: T={T} max_len={w.max_seq_len} partition {part}")
    assert part < w.max_seq_len
    d = {"q": w.q, "k_cache": w.k_cache, "v_cache": w.v_cache, "new_k": w.new_k,
         "new_v": w.new_v, "slot_mapping": w.slot_mapping, "block_table": w.block_table,
         "seq_lens": w.seq_lens, "query_start": w.query_start_dev}
    out = _step(d, cfg, w.max_query_len, w.max_seq_len)
    kc, vc = to_host(w.k_cache, "bf16"), to_host(w.v_cache, "bf16")
    q = to_host(w.q, "bf16")
    qs, lens, table = w.query_start, w.layout.seq_lens, w.layout.block_table
    worst, worst_rel = 0.0, 0.0
    for s in range(cfg.num_seqs):
        n = int(qs[s + 1] - qs[s])
        ctx = int(lens[s]) - n
        for a in (0, n // 2 - 8, n - 16):
            b = a + 16
            for g in (0, cfg.kv_heads - 3):
                heads = slice(g * G, (g + 1) * G)
                ref = oracle.extend_attention(
                    np.ascontiguousarray(q[qs[s] + a:qs[s] + b, heads]),
                    np.ascontiguousarray(kc[:, :, g:g + 1]), np.ascontiguousarray(vc[:, :, g:g + 1]),
                    table[s:s + 1], np.array([ctx + b]), np.array([0, b - a]), cfg.scale, "bf16")
                got = out[qs[s] + a:qs[s] + b, heads]
                mabs, mrel = compare(got, ref, "bf16")
                worst, worst_rel = max(worst, mabs), max(worst_rel, mrel)
    log(f"  max-abs {worst:.3e} row max-rel {worst_rel:.3e}")


@pytest.mark.parametrize("part_tokens", [0, 64])
def test_extend_and_block_move_replay_inside_a_captured_graph(part_tokens):
    """Slot write, extend (unsplit, or split with its merge kernel and a
    caller-provided workspace) and a device-to-pinned-host block move
    captured in one HIP graph, replayed several times with eager work in
    between; every replay matches the eager result bit for bit."""
    cfg = EXTEND_CONFIGS["x5_extend_mha_bf16"]
    w = generate_extend_host(cfg)
    d = _upload(w)
    out = torch.empty_like(d["q"])
    need = pkv.extend_workspace_size(d["k_cache"], cfg.num_seqs, w.num_tokens, cfg.q_heads,
                                     w.max_query_len, w.max_seq_len, part_tokens)
    assert (need > 0) == (part_tokens > 0)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    NB = w.layout.num_blocks
    host_k = torch.zeros((8,) + tuple(d["k_cache"].shape[1:]), dtype=torch.bfloat16).pin_memory()
    host_v = torch.zeros_like(host_k).pin_memory()
    pairs = torch.tensor([[b, i] for i, b in enumerate(range(0, NB, max(NB // 8, 1)))][:8],
                         dtype=torch.int64, device="cuda")

    def step():
        pkv.paged_kv_write(d["new_k"], d["new_v"], d["slot_mapping"], d["k_cache"], d["v_cache"])
        pkv.paged_attn_extend(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                              d["seq_lens"], d["query_start"], cfg.scale, w.max_query_len,
                              w.max_seq_len, out=out, part_tokens=part_tokens, workspace=ws)
        pkv.paged_block_move(pairs, d["k_cache"], d["v_cache"], host_k, host_v)

    step()
    torch.cuda.synchronize()
    eager_out = out.clone()
    eager_hk, eager_hv = host_k.clone(), host_v.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.zero_()
        host_k.zero_()
        host_v.zero_()
        d["k_cache"].copy_(to_device(w.k_cache, "bf16"))
        d["v_cache"].copy_(to_device(w.v_cache, "bf16"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager_out.view(torch.int16)), f"replay {r}"
        assert torch.equal(host_k.view(torch.int16), eager_hk.view(torch.int16)), f"replay {r}"
        assert torch.equal(host_v.view(torch.int16), eager_hv.view(torch.int16)), f"replay {r}"
