"""Pins of the multi-token (prefill / extend) oracle.

Each check ties ``oracle.extend_attention`` to something other than itself:
the pinned decode oracle run one position at a time, torch's
scaled-dot-product attention on a contiguous copy built independently of the
oracle's gather, closed forms, and the causal invariant.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import widen
from workloads import EXTEND_CONFIGS, generate_extend_host


def _paged_from_contiguous(rng, K, V, BS, extra_blocks=3):
    """Scatter contiguous per-sequence K/V ([L, Hkv, D] each) into a pool of
    blocks at random places; returns (k_cache, v_cache, table)."""
    lens = [k.shape[0] for k in K]
    nblk = [-(-L // BS) for L in lens]
    NB = sum(nblk) + extra_blocks
    Hkv, D = K[0].shape[1], K[0].shape[2]
    perm = rng.permutation(NB)
    kc = rng.standard_normal((NB, BS, Hkv, D))
    vc = rng.standard_normal((NB, BS, Hkv, D))
    table = np.full((len(K), max(nblk)), -1, dtype=np.int32)
    cur = 0
    for s, L in enumerate(lens):
        for b in range(nblk[s]):
            phys = int(perm[cur])
            cur += 1
            table[s, b] = phys
            rows = slice(b * BS, min(L, (b + 1) * BS))
            n = rows.stop - rows.start
            kc[phys, :n] = K[s][rows]
            vc[phys, :n] = V[s][rows]
    return kc, vc, table


def test_one_new_token_is_decode():
    w = generate_extend_host(EXTEND_CONFIGS["x1_extend_tiny_bf16"])
    S = w.cfg.num_seqs
    qs = np.arange(S + 1, dtype=np.int32)
    q = w.q[:S]
    got = oracle.extend_attention(q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, qs,
                                  w.cfg.scale, "bf16")
    ref = oracle.decode_attention(q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                                  w.cfg.scale, "bf16")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("name", ["x1_extend_tiny_bf16", "x5_extend_mha_bf16"])
def test_every_query_is_a_decode_of_its_prefix(name):
    """Query j of sequence s equals decode of the sequence cut to p + 1 tokens."""
    w = generate_extend_host(EXTEND_CONFIGS[name])
    cfg = w.cfg
    got = oracle.extend_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                                  w.query_start, cfg.scale, "bf16")
    rng = np.random.default_rng(0)
    for s in range(cfg.num_seqs):
        n, L = int(w.query_start[s + 1] - w.query_start[s]), int(w.seq_lens[s])
        for j in rng.choice(n, size=min(n, 12), replace=False):
            row = int(w.query_start[s]) + int(j)
            p = L - n + int(j)
            ref = oracle.decode_attention(w.q[row:row + 1], w.k_cache, w.v_cache,
                                          w.block_table[s:s + 1], np.array([p + 1]),
                                          cfg.scale, "bf16")
            np.testing.assert_allclose(got[row], ref[0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("G", [1, 4])
def test_matches_torch_sdpa_on_a_contiguous_copy(G):
    """A prefill (nothing cached) and an extend (context cached) against
    torch's scaled_dot_product_attention over contiguous K/V; the paged
    copy is scattered by this test, not by the oracle."""
    rng = np.random.default_rng(40 + G)
    Hkv, D, BS = 2, 32, 4
    Hq = Hkv * G
    ctx, new = [0, 9, 3], [11, 6, 1]
    lens = [c + n for c, n in zip(ctx, new)]
    K = [rng.standard_normal((L, Hkv, D)) for L in lens]
    V = [rng.standard_normal((L, Hkv, D)) for L in lens]
    kc, vc, table = _paged_from_contiguous(rng, K, V, BS)
    qs = np.concatenate([[0], np.cumsum(new)]).astype(np.int32)
    q = rng.standard_normal((int(qs[-1]), Hq, D))
    scale = 0.3
    got = oracle.extend_attention(q, kc, vc, table, np.array(lens), qs, scale, "f64")
    for s, (L, n) in enumerate(zip(lens, new)):
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]]).permute(1, 0, 2)            # [Hq, n, D]
        Kt = torch.from_numpy(K[s]).permute(1, 0, 2).repeat_interleave(G, 0)  # [Hq, L, D]
        Vt = torch.from_numpy(V[s]).permute(1, 0, 2).repeat_interleave(G, 0)
        mask = torch.ones(n, L, dtype=torch.bool).tril(diagonal=L - n)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, Kt, Vt, attn_mask=mask, scale=float(np.float32(scale)))
        np.testing.assert_allclose(got[qs[s]:qs[s + 1]], ref.permute(1, 0, 2).numpy(),
                                   rtol=0, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(7)
    Hkv, G, D, BS, L = 2, 2, 16, 4, 13
    K = [rng.standard_normal((L, Hkv, D))]
    V = [rng.standard_normal((L, Hkv, D))]
    kc, vc, table = _paged_from_contiguous(rng, K, V, BS)
    n = 5
    qs = np.array([0, n], dtype=np.int32)
    # q = 0: uniform weights, the mean of the visible value rows.
    out = oracle.extend_attention(np.zeros((n, Hkv * G, D)), kc, vc, table, np.array([L]), qs,
                                  1.0, "f64")
    for j in range(n):
        p = L - n + j
        for h in range(Hkv * G):
            np.testing.assert_allclose(out[j, h], V[0][:p + 1, h // G].mean(0), atol=1e-12)
    # constant values give that constant.
    vc_const = np.full_like(vc, 0.625)
    out = oracle.extend_attention(rng.standard_normal((n, Hkv * G, D)), kc, vc_const, table,
                                  np.array([L]), qs, 0.5, "f64")
    np.testing.assert_allclose(out, 0.625, atol=1e-12)
    # a prefill's first token sees only itself.
    out = oracle.extend_attention(rng.standard_normal((L, Hkv * G, D)), kc, vc, table,
                                  np.array([L]), np.array([0, L], dtype=np.int32), 0.5, "f64")
    for h in range(Hkv * G):
        np.testing.assert_array_equal(out[0, h], V[0][0, h // G])


def test_later_positions_do_not_leak():
    """Changing keys and values after a query's position leaves its row as is."""
    rng = np.random.default_rng(8)
    Hkv, D, BS, L, n = 1, 8, 4, 10, 6
    K = [rng.standard_normal((L, Hkv, D))]
    V = [rng.standard_normal((L, Hkv, D))]
    kc, vc, table = _paged_from_contiguous(rng, K, V, BS)
    qs = np.array([0, n], dtype=np.int32)
    q = rng.standard_normal((n, 2, D))
    base = oracle.extend_attention(q, kc, vc, table, np.array([L]), qs, 0.4, "f64")
    for cut in range(L - n, L):
        K2 = [K[0].copy()]
        V2 = [V[0].copy()]
        K2[0][cut + 1:] += 5.0
        V2[0][cut + 1:] -= 3.0
        kc2, vc2, table2 = _paged_from_contiguous(np.random.default_rng(9), K2, V2, BS)
        out = oracle.extend_attention(q, kc2, vc2, table2, np.array([L]), qs, 0.4, "f64")
        j = cut - (L - n)
        np.testing.assert_allclose(out[:j + 1], base[:j + 1], atol=1e-12)
        if cut + 1 < L:
            assert not np.allclose(out[j + 1:], base[j + 1:])


def test_degenerate_rows_are_zero():
    rng = np.random.default_rng(10)
    kc = rng.standard_normal((4, 4, 1, 8))
    table = np.array([[2, 0], [1, -1]], dtype=np.int32)
    q = rng.standard_normal((7, 1, 8))
    qs = np.array([0, 5, 7], dtype=np.int32)
    # sequence 0: 5 queries but L = 3 -> the first two sit before position 0
    out = oracle.extend_attention(q, kc, kc, table, np.array([3, 0]), qs, 1.0, "f64")
    assert not out[:2].any() and not out[5:].any()
    assert np.abs(out[2:5]).sum() > 0


def test_flop_count_by_enumeration():
    lens, new = [7, 3, 0], [4, 3, 0]
    qs = np.concatenate([[0], np.cumsum(new)])
    count = 0
    for L, n in zip(lens, new):
        for p in range(L - n, L):
            count += sum(1 for t in range(L) if t <= p)
    assert oracle.extend_flops(lens, qs, 8, 64) == count * 8 * 4 * 64


def test_bf16_widening_path_matches_f64_of_the_same_values():
    """The bf16 entry point is the float64 computation of the widened bits."""
    w = generate_extend_host(EXTEND_CONFIGS["x1_extend_tiny_bf16"])
    a = oracle.extend_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                                w.query_start, w.cfg.scale, "bf16", seqs=[1, 3])
    b = oracle.extend_attention(widen(w.q, "bf16"), widen(w.k_cache, "bf16"),
                                widen(w.v_cache, "bf16"), w.block_table, w.seq_lens,
                                w.query_start, w.cfg.scale, "f64", seqs=[1, 3])
    np.testing.assert_array_equal(a, b)
