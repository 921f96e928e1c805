"""A continuous-batching run through every layer, step by step.

The native block manager admits requests (reusing the cached full blocks of a
common system prompt), forks running sequences (parallel sampling), appends
one token per running sequence per step (copy-on-write where a block is
shared), swaps sequences out to pinned host blocks and back, and frees them.
Its slots and block pairs drive the kernels: the slot write, the block copy,
the block move, prefill / chunked-extend attention for each admission and
decode attention for every step.  A host mirror of both pools (and of the
host swap pool) is kept with the oracle's own slot write, block copy and
block move from the same pairs, and every attention output is compared with
the oracle on that mirror ("PagedAttention Explained", "How PagedAttention
works", "Sharing blocks between sequences", "Preemption and scheduling").
At the end the device pools equal the mirror bit for bit.

A token's K and V rows are a fixed function of its id and position, as a
model's would be, so that a request that reuses another's cached prompt
blocks attends over exactly the rows it would have written itself.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_317_amd as pkv
from paged_kv_cache_317_amd.block_manager import BlockManager
from workloads.generate import f32_to_bf16_bits

from helpers import compare, log, to_device, to_host

pytestmark = pytest.mark.gpu

BS, HKV, G, D = 16, 2, 4, 128
NUM_BLOCKS = 640
WIDTH = 24                      # table width: 384 positions per sequence at most
SYSTEM_PROMPT = 40              # tokens every request starts with (2 full blocks cached)
SCALE = 0.09


def _kv_rows(tokens, positions):
    """bf16 K and V rows [n, HKV, D] of tokens at positions (seeded by both)."""
    k = np.empty((len(tokens), HKV, D), dtype=np.float32)
    v = np.empty_like(k)
    for i, (t, p) in enumerate(zip(tokens, positions)):
        r = np.random.default_rng([int(t), int(p), 317])
        k[i] = r.standard_normal((HKV, D), dtype=np.float32)
        v[i] = r.standard_normal((HKV, D), dtype=np.float32)
    return f32_to_bf16_bits(k), f32_to_bf16_bits(v)


class _Run:
    """Device pools, their host mirror and the block manager of one run."""

    def __init__(self, rng):
        self.rng = rng
        shape = (NUM_BLOCKS, BS, HKV, D)
        self.kc_h = np.zeros(shape, dtype=np.uint16)
        self.vc_h = np.zeros(shape, dtype=np.uint16)
        self.hk_h = np.zeros(shape, dtype=np.uint16)      # host swap pool mirror
        self.hv_h = np.zeros(shape, dtype=np.uint16)
        self.kc = to_device(self.kc_h, "bf16")
        self.vc = to_device(self.vc_h, "bf16")
        self.hk = torch.zeros(shape, dtype=torch.bfloat16).pin_memory()
        self.hv = torch.zeros(shape, dtype=torch.bfloat16).pin_memory()
        self.bm = BlockManager(NUM_BLOCKS, BS)
        self.bm.set_swap_space(NUM_BLOCKS)
        self.tokens = {}                                  # sequence -> token ids so far
        # Sequences the manager no longer tracks by token id (a swapped-in
        # sequence comes back without them, and so do its forks): their
        # appends carry no ids.
        self.untracked = set()
        self.next_id = 0
        self.system = rng.integers(0, 50_000, size=SYSTEM_PROMPT).tolist()

    def copy_blocks(self, pairs):
        if not pairs:
            return
        pkv.paged_block_copy(torch.tensor(pairs, dtype=torch.int64, device="cuda"),
                             self.kc, self.vc)
        oracle.block_copy(self.kc_h, self.vc_h, pairs, inplace=True)

    def write(self, slots, tokens, positions):
        k, v = _kv_rows(tokens, positions)
        pkv.paged_kv_write(to_device(k, "bf16"), to_device(v, "bf16"),
                           torch.tensor(slots, dtype=torch.int64, device="cuda"),
                           self.kc, self.vc)
        oracle.kv_write(self.kc_h, self.vc_h, k, v, slots, inplace=True)

    def admit(self, count):
        """New requests: system prompt + user tokens, cached blocks reused;
        the uncached part written and attended by one extend call."""
        ids, news, ctxs = [], [], []
        for _ in range(count):
            s = self.next_id
            self.next_id += 1
            prompt = self.system + self.rng.integers(0, 50_000,
                                                     size=int(self.rng.integers(1, 150))).tolist()
            reused = self.bm.add_cached(s, prompt)
            new = prompt[reused:]
            slots, copies = self.bm.append_tokens(s, new)
            assert not copies
            self.write(slots, new, range(reused, len(prompt)))
            self.tokens[s] = prompt
            ids.append(s)
            news.append(len(new))
            ctxs.append(reused)
        lens = np.array([len(self.tokens[s]) for s in ids], dtype=np.int32)
        qs = np.concatenate([[0], np.cumsum(news)]).astype(np.int32)
        q = f32_to_bf16_bits(self.rng.standard_normal((int(qs[-1]), HKV * G, D),
                                                      dtype=np.float32))
        table = self.bm.table_array(ids, WIDTH)
        out = pkv.paged_attn_extend(to_device(q, "bf16"), self.kc, self.vc, to_device(table, None),
                                    to_device(lens, None), to_device(qs, None), SCALE,
                                    int(max(news)), int(lens.max()))
        torch.cuda.synchronize()
        ref = oracle.extend_attention(q, self.kc_h, self.vc_h, table, lens, qs, SCALE, "bf16")
        compare(out, ref, "bf16")
        return ids, ctxs

    def decode_step(self, running):
        """One token per running sequence: appends (copy-on-write pairs
        first, then every slot write), then decode over all of them."""
        slots, copies, toks, poss = [], [], [], []
        for s in running:
            t = int(self.rng.integers(0, 50_000))
            if s in self.untracked:
                sl, cp = self.bm.append(s, 1)
            else:
                sl, cp = self.bm.append_tokens(s, [t])
            slots += sl
            copies += cp
            toks.append(t)
            poss.append(len(self.tokens[s]))
            self.tokens[s].append(t)
        self.copy_blocks(copies)
        self.write(slots, toks, poss)
        lens = np.array([len(self.tokens[s]) for s in running], dtype=np.int32)
        assert all(self.bm.length(s) == len(self.tokens[s]) for s in running)
        q = f32_to_bf16_bits(self.rng.standard_normal((len(running), HKV * G, D),
                                                      dtype=np.float32))
        table = self.bm.table_array(running, WIDTH)
        out = pkv.paged_attn_decode(to_device(q, "bf16"), self.kc, self.vc,
                                    to_device(table, None), to_device(lens, None), SCALE,
                                    int(lens.max()))
        torch.cuda.synchronize()
        ref = oracle.decode_attention(q, self.kc_h, self.vc_h, table, lens, SCALE, "bf16")
        compare(out, ref, "bf16")
        return len(copies)

    def swap_out(self, s):
        pairs = self.bm.swap_out(s)
        pkv.paged_block_move(torch.tensor(pairs, dtype=torch.int64, device="cuda"),
                             self.kc, self.vc, self.hk, self.hv)
        self.hk_h, self.hv_h = oracle.block_move(self.kc_h, self.vc_h, self.hk_h, self.hv_h,
                                                 pairs)
        return len(pairs)

    def swap_in(self, s):
        pairs = self.bm.swap_in(s)
        self.untracked.add(s)
        pkv.paged_block_move(torch.tensor(pairs, dtype=torch.int64, device="cuda"),
                             self.hk, self.hv, self.kc, self.vc)
        self.kc_h, self.vc_h = oracle.block_move(self.hk_h, self.hv_h, self.kc_h, self.vc_h,
                                                 pairs)
        return len(pairs)


@pytest.mark.parametrize("seed", [0, 1])
def test_serving_steps_against_the_oracle(seed):
    rng = np.random.default_rng(9100 + seed)
    run = _Run(rng)
    running, swapped = [], []
    reused_total = cow_total = moved_total = 0
    for step in range(24):
        if step % 4 == 0:
            ids, ctxs = run.admit(2 if step else 3)
            running += ids
            reused_total += sum(ctxs)
        if step % 5 == 2:                           # parallel sampling: a second completion
            parent = running[int(rng.integers(0, len(running)))]
            child = run.next_id
            run.next_id += 1
            run.bm.fork(parent, child)
            run.tokens[child] = list(run.tokens[parent])
            if parent in run.untracked:
                run.untracked.add(child)
            running.append(child)
        if step % 6 == 3 and len(running) > 2:      # preemption by swapping
            s = running.pop(int(rng.integers(0, len(running))))
            moved_total += run.swap_out(s)
            swapped.append(s)
        if step % 6 == 5 and swapped:
            s = swapped.pop(0)
            moved_total += run.swap_in(s)
            running.append(s)
        if step % 7 == 6 and len(running) > 3:      # a finished request
            s = running.pop(0)
            run.bm.free_sequence(s)
            del run.tokens[s]
        cow_total += run.decode_step(running)
        log(f"seed {seed} step {step}: running {len(running)} swapped {len(swapped)} "
            f"reused {reused_total} cow {cow_total} moved {moved_total}")
    # Every path the run was meant to take was taken.
    assert reused_total > 0 and cow_total > 0 and moved_total > 0
    torch.cuda.synchronize()
    assert np.array_equal(to_host(run.kc, "bf16"), run.kc_h)
    assert np.array_equal(to_host(run.vc, "bf16"), run.vc_h)
    assert np.array_equal(to_host(run.hk, "bf16"), run.hk_h)
    assert np.array_equal(to_host(run.hv, "bf16"), run.hv_h)
    run.bm.close()
