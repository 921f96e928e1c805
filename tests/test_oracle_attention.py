"""Pins of the decode-attention oracle against facts outside it.

Each test checks the oracle against something it does not itself compute: a
fact the pages print, a closed form, a library routine on a special case, a
brute-force scalar evaluation, or an invariant the pages state.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import get_config, generate_host, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _paged_from_contiguous(seqs_k, seqs_v, block_size, rng, spare=3):
    """Scatter per-sequence contiguous K/V ([L, Hkv, D] float32) into a random pool."""
    Hkv, D = seqs_k[0].shape[1:]
    need = [-(-k.shape[0] // block_size) for k in seqs_k]
    NB = sum(need) + spare
    perm = rng.permutation(NB)
    kc = rng.standard_normal((NB, block_size, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal((NB, block_size, Hkv, D)).astype(np.float32)
    width = max(need + [1])
    table = np.full((len(seqs_k), width), -1, dtype=np.int32)
    cur = 0
    for s, (k, v) in enumerate(zip(seqs_k, seqs_v)):
        for j in range(need[s]):
            b = perm[cur]
            cur += 1
            table[s, j] = b
            rows = k[j * block_size:(j + 1) * block_size]
            kc[b, : rows.shape[0]] = rows
            vc[b, : rows.shape[0]] = v[j * block_size:(j + 1) * block_size]
    return kc, vc, table


def _random_case(rng, S, Hq, Hkv, D, BS, max_len, min_len=1):
    lens = rng.integers(min_len, max_len + 1, size=S)
    ks = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    vs = [rng.standard_normal((L, Hkv, D)).astype(np.float32) for L in lens]
    q = rng.standard_normal((S, Hq, D)).astype(np.float32)
    kc, vc, table = _paged_from_contiguous(ks, vs, BS, rng)
    return q, kc, vc, table, lens.astype(np.int32), ks, vs


# --- the page's token-to-block fact --------------------------------------------

def test_gather_follows_logical_block_mapping():
    """Positions 0-15 come from the table's entry 0, 16-31 from entry 1 (block 16)."""
    fx = json.load(open(os.path.join(GOLDEN, "logical_blocks_bs16.json")))
    BS = fx["block_size"]
    NB = 5
    # each slot stores (physical block, offset) so the gather's source is visible
    cache = np.zeros((NB, BS, 1, 2), dtype=np.float32)
    for b in range(NB):
        for o in range(BS):
            cache[b, o, 0] = (b, o)
    table = np.array([3, 0, 4], dtype=np.int32)
    rows = oracle.gather_sequence(cache, table, 40, BS)
    for lo, hi, logical in fx["ranges"]:
        for t in range(lo, hi + 1):
            assert tuple(rows[t, 0]) == (table[logical], t - lo)
    # and the third logical block continues the pattern
    assert tuple(rows[32, 0]) == (4, 0) and tuple(rows[39, 0]) == (4, 7)


# --- library routine on a special case -----------------------------------------

@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_matches_torch_sdpa_fp64(G):
    rng = np.random.default_rng(100 + G)
    Hkv, D, BS = 2, 16, 4
    Hq = Hkv * G
    q, kc, vc, table, lens, ks, vs = _random_case(rng, 5, Hq, Hkv, D, BS, 37)
    scale = np.float32(0.3)
    got = oracle.decode_attention(q, kc, vc, table, lens, scale, "f32")
    for s in range(len(lens)):
        K = torch.from_numpy(ks[s].astype(np.float64)).permute(1, 0, 2)   # [Hkv, L, D]
        V = torch.from_numpy(vs[s].astype(np.float64)).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0).contiguous()
        V = V.repeat_interleave(G, dim=0).contiguous()
        Q = torch.from_numpy(q[s].astype(np.float64))[:, None, :]          # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, scale=float(scale))[:, 0, :].numpy()
        np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-12)


# --- brute force ------------------------------------------------------------------

def _brute_force(q, kc, vc, table, lens, scale, to_float):
    """Scalar triple loop with Python floats and math.exp (no numpy arithmetic)."""
    S, Hq, D = q.shape
    _, BS, Hkv, _ = kc.shape
    G = Hq // Hkv
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(S)]
    sc = float(np.float32(scale))
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        for h in range(Hq):
            g = h // G
            logits = []
            for t in range(L):
                b, o = int(table[s][t // BS]), t % BS
                acc = 0.0
                for d in range(D):
                    acc += to_float(q[s, h, d]) * to_float(kc[b, o, g, d])
                logits.append(sc * acc)
            mx = max(logits)
            w = [math.exp(x - mx) for x in logits]
            tot = sum(w)
            for d in range(D):
                acc = 0.0
                for t in range(L):
                    b, o = int(table[s][t // BS]), t % BS
                    acc += w[t] * to_float(vc[b, o, g, d])
                out[s][h][d] = acc / tot
    return np.array(out)


def test_brute_force_tiny_random_cases():
    rng = np.random.default_rng(7)
    for case in range(20):
        G = [1, 2, 4][case % 3]
        Hkv = 1 + case % 2
        D = int(rng.integers(1, 9))
        BS = int(rng.choice([1, 2, 4, 16]))
        S = int(rng.integers(1, 4))
        q, kc, vc, table, lens, _, _ = _random_case(rng, S, Hkv * G, Hkv, D, BS, 40)
        scale = np.float32(rng.uniform(0.05, 1.0))
        got = oracle.decode_attention(q, kc, vc, table, lens, scale, "f32")
        ref = _brute_force(q, kc, vc, table, lens, scale, float)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_brute_force_c1():
    w = generate_host(get_config("c1_tiny_f32"))
    cfg = w.cfg
    got = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                                  cfg.scale, "f32")
    ref = _brute_force(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, cfg.scale, float)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_brute_force_bf16_widening():
    """bf16 path: the brute force widens each element through torch's bf16."""
    rng = np.random.default_rng(11)
    q, kc, vc, table, lens, _, _ = _random_case(rng, 2, 4, 2, 8, 4, 23)
    qb, kb, vb = (f32_to_bf16_bits(a) for a in (q, kc, vc))
    to_float = lambda bits: float(torch.tensor([int(bits)], dtype=torch.int32)
                                  .to(torch.int16).view(torch.bfloat16).double())
    got = oracle.decode_attention(qb, kb, vb, table, lens, 0.25, "bf16")
    ref = _brute_force(qb, kb, vb, table, lens, 0.25, to_float)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# --- closed forms -----------------------------------------------------------------

def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(3)
    q, kc, vc, table, _, _, _ = _random_case(rng, 3, 8, 2, 16, 16, 5)
    lens = np.ones(3, dtype=np.int32)
    out = oracle.decode_attention(q, kc, vc, table, lens, 0.7, "f32")
    for s in range(3):
        for h in range(8):
            assert np.array_equal(out[s, h], vc[table[s, 0], 0, h // 4].astype(np.float64))


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(4)
    q, kc, vc, table, lens, _, vs = _random_case(rng, 3, 4, 4, 8, 4, 30)
    q[:] = 0
    out = oracle.decode_attention(q, kc, vc, table, lens, 1.0, "f32")
    for s in range(3):
        np.testing.assert_allclose(out[s], vs[s].astype(np.float64).mean(axis=0),
                                   rtol=0, atol=1e-13)


def test_constant_values_give_the_constant():
    rng = np.random.default_rng(5)
    q, kc, vc, table, lens, _, _ = _random_case(rng, 3, 4, 2, 8, 4, 30)
    vc[:] = np.float32(-1.25)
    out = oracle.decode_attention(q, kc, vc, table, lens, 0.5, "f32")
    np.testing.assert_allclose(out, -1.25, rtol=0, atol=1e-14)


def test_large_scale_selects_the_best_matching_key():
    """As scale grows the softmax becomes one-hot on the largest logit."""
    rng = np.random.default_rng(6)
    q, kc, vc, table, lens, ks, vs = _random_case(rng, 4, 2, 1, 8, 4, 30, min_len=2)
    out = oracle.decode_attention(q, kc, vc, table, lens, 1e6, "f32")
    for s in range(4):
        for h in range(2):
            x = ks[s][:, 0, :].astype(np.float64) @ q[s, h].astype(np.float64)
            assert np.array_equal(out[s, h], vs[s][int(np.argmax(x)), 0].astype(np.float64))


def test_empty_sequence_gives_zero_row():
    rng = np.random.default_rng(8)
    q, kc, vc, table, lens, _, _ = _random_case(rng, 3, 2, 2, 4, 4, 10)
    lens[1] = 0
    out = oracle.decode_attention(q, kc, vc, table, lens, 1.0, "f32")
    assert np.all(out[1] == 0)
    assert np.all(np.isfinite(out))


# --- invariants the pages state ---------------------------------------------------

def test_unused_slots_and_blocks_never_reach_the_output():
    """Only the last block is partly filled; its tail and unreferenced blocks are never read."""
    rng = np.random.default_rng(9)
    q, kc, vc, table, lens, _, _ = _random_case(rng, 4, 4, 2, 8, 16, 70)
    ref = oracle.decode_attention(q, kc, vc, table, lens, 0.4, "f32")
    used = np.zeros(kc.shape[:2], dtype=bool)
    for s, L in enumerate(lens):
        for t in range(L):
            used[table[s, t // 16], t % 16] = True
    kp, vp = kc.copy(), vc.copy()
    kp[~used] = np.nan
    vp[~used] = np.nan
    got = oracle.decode_attention(q, kp, vp, table, lens, 0.4, "f32")
    assert np.array_equal(got, ref)


def test_placement_permutation_invariance():
    """Physical blocks may sit anywhere and in any order."""
    rng = np.random.default_rng(10)
    q, kc, vc, table, lens, _, _ = _random_case(rng, 4, 8, 2, 16, 4, 50)
    ref = oracle.decode_attention(q, kc, vc, table, lens, 0.2, "f32")
    perm = rng.permutation(kc.shape[0])          # new id of old block b is perm[b]
    kp = np.empty_like(kc)
    vp = np.empty_like(vc)
    kp[perm] = kc
    vp[perm] = vc
    tp = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    got = oracle.decode_attention(q, kp, vp, tp, lens, 0.2, "f32")
    assert np.array_equal(got, ref)


def test_shared_block_equals_private_copies():
    """Sequences pointing at one physical block see what private copies would give."""
    rng = np.random.default_rng(12)
    BS, Hkv, D, S = 4, 2, 8, 3
    prefix = rng.standard_normal((8, Hkv, D)).astype(np.float32)     # two full blocks
    kc = rng.standard_normal((2 + 2 * S + 2 * S, BS, Hkv, D)).astype(np.float32)
    vc = rng.standard_normal(kc.shape).astype(np.float32)
    kc[0:2] = prefix.reshape(2, BS, Hkv, D)
    vc[0:2] = -prefix.reshape(2, BS, Hkv, D)
    q = rng.standard_normal((S, 4, D)).astype(np.float32)
    lens = np.array([9, 11, 8], dtype=np.int32)
    shared = np.full((S, 3), -1, dtype=np.int32)
    private = np.full((S, 3), -1, dtype=np.int32)
    for s in range(S):
        shared[s, :2] = [0, 1]
        a, b = 2 + 2 * s, 3 + 2 * s
        kc[a:b + 1] = kc[0:2]
        vc[a:b + 1] = vc[0:2]
        private[s, :2] = [a, b]
        shared[s, 2] = private[s, 2] = 2 + 2 * S + s
    r_shared = oracle.decode_attention(q, kc, vc, shared, lens, 0.5, "f32")
    r_private = oracle.decode_attention(q, kc, vc, private, lens, 0.5, "f32")
    assert np.array_equal(r_shared, r_private)


def test_gqa_equals_mha_on_duplicated_kv_heads():
    rng = np.random.default_rng(13)
    G, Hkv = 4, 2
    q, kc, vc, table, lens, _, _ = _random_case(rng, 3, G * Hkv, Hkv, 8, 4, 25)
    gqa = oracle.decode_attention(q, kc, vc, table, lens, 0.6, "f32")
    kd = np.repeat(kc, G, axis=2)          # KV head g becomes heads g*G .. g*G+G-1
    vd = np.repeat(vc, G, axis=2)
    mha = oracle.decode_attention(q, kd, vd, table, lens, 0.6, "f32")
    assert np.array_equal(gqa, mha)


# --- split-K ------------------------------------------------------------------------

@pytest.mark.parametrize("part", [1, 3, 16, 17, 64, 1000])
def test_split_merge_equals_unsplit(part):
    rng = np.random.default_rng(14)
    q, kc, vc, table, lens, _, _ = _random_case(rng, 4, 4, 2, 8, 4, 90)
    ref = oracle.decode_attention(q, kc, vc, table, lens, 0.45, "f32")
    got = oracle.split_decode_attention(q, kc, vc, table, lens, 0.45, "f32", part)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_partition_states_closed_forms():
    """One partition: l is the softmax denominator and o/l the unsplit output."""
    x = np.array([0.5, -1.0, 2.0, 0.0])
    V = np.arange(8, dtype=np.float64).reshape(4, 2)
    m, l, o = oracle.partition_states(x, V, 4)
    assert m[0] == 2.0
    np.testing.assert_allclose(l[0], sum(math.exp(v - 2.0) for v in x), rtol=1e-15)
    # two partitions of two: states are those of each half
    m2, l2, o2 = oracle.partition_states(x, V, 2)
    assert list(m2) == [0.5, 2.0]
    np.testing.assert_allclose(o2[0], math.exp(0) * V[0] + math.exp(-1.5) * V[1], rtol=1e-15)
    np.testing.assert_allclose(oracle.merge_states(m2, l2, o2), o[0] / l[0], rtol=1e-15)
