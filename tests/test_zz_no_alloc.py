"""The decode entry point that allocates nothing, through the C ABI.

pkv_paged_attn_decode_noalloc takes its split workspace from the library's
own device array.  Two calls in a row, the second with a smaller batch (the
array then holds the first call's states), each give the bits of
pkv_paged_attn_decode with a caller workspace, and both match the oracle.
A call that would need more than the array holds is refused before any
launch; a call that needs no workspace works too.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_317_amd as pkv
from paged_kv_cache_317_amd._lib import lib
from workloads import generate_host, get_config, scaled

from helpers import compare, log, upload

pytestmark = pytest.mark.gpu


def _noalloc(d, w, out, part=0):
    """One call of the entry point through ctypes."""
    cfg = w.cfg
    desc = pkv.cache_desc(d["k_cache"])
    st = lib().pkv_paged_attn_decode_noalloc(
        d["q"].data_ptr(), d["k_cache"].data_ptr(), d["v_cache"].data_ptr(), ctypes.byref(desc),
        d["block_table"].data_ptr(), d["block_table"].shape[1], d["seq_lens"].data_ptr(),
        cfg.num_seqs, cfg.q_heads, w.layout.max_seq_len, cfg.scale, out.data_ptr(), part,
        torch.cuda.current_stream().cuda_stream)
    return st


def _case(**kw):
    return generate_host(scaled(get_config("c3_gqa4k_bf16"), **kw))


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    big = _case(num_seqs=48, len_range=(500, 3000), max_len=3072)
    small = _case(num_seqs=7, len_range=(1, 900), max_len=1024)
    for w, part in ((big, 0), (small, 0), (big, 64), (small, 512)):
        cfg = w.cfg
        d = upload(w)
        need = pkv.decode_workspace_size(d["k_cache"], cfg.num_seqs, cfg.q_heads,
                                         w.layout.max_seq_len, part)
        runs = pkv.decode_runs(d["k_cache"], cfg.num_seqs, cfg.q_heads, w.layout.max_seq_len,
                               part)
        log(f"noalloc S={cfg.num_seqs} part={part} runs={runs} workspace={need}")
        assert runs > 1 and 0 < need <= lib().pkv_decode_noalloc_max_workspace()
        out = torch.full_like(d["q"], float("nan"))
        assert _noalloc(d, w, out, part) == 0, lib().pkv_last_error()
        torch.cuda.synchronize()
        ref_gpu = pkv.paged_attn_decode(d["q"], d["k_cache"], d["v_cache"], d["block_table"],
                                        d["seq_lens"], cfg.scale, w.layout.max_seq_len,
                                        part_tokens=part)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_gpu.view(torch.int16))
        ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                                      cfg.scale, cfg.dtype)
        compare(out, ref, cfg.dtype)


def test_noalloc_single_run_and_refusal():
    # one run (a single sequence of one tile): no workspace at all
    w = generate_host(scaled(get_config("c1_tiny_f32"), num_seqs=1, seq_lens=(13,), max_len=16))
    d = upload(w)
    assert pkv.decode_runs(d["k_cache"], 1, 8, w.layout.max_seq_len) == 1
    out = torch.empty_like(d["q"])
    assert _noalloc(d, w, out) == 0
    torch.cuda.synchronize()
    ref = oracle.decode_attention(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                                  w.cfg.scale, w.cfg.dtype)
    compare(out, ref, "f32")
    # a batch whose workspace exceeds the array: refused on the host
    desc = pkv.cache_desc(d["k_cache"])
    S, Hq, maxlen = 6000, 64, 16384
    big = lib().pkv_decode_workspace_size(ctypes.byref(desc), S, Hq, maxlen, 0)
    assert big > lib().pkv_decode_noalloc_max_workspace()
    st = lib().pkv_paged_attn_decode_noalloc(1 << 12, 1 << 12, 1 << 12, ctypes.byref(desc),
                                             1 << 12, 1, 1 << 12, S, Hq, maxlen, 0.1, 1 << 12, 0,
                                             None)
    assert st == 5 and "workspace" in lib().pkv_last_error().decode()
