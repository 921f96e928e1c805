#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV-cache path on one MI355X.

One step = ``paged_kv_write`` of every sequence's new token, then
``paged_attn_decode`` over the whole batch, both on the current stream, with
every input already resident in HBM.  The default workload is the bf16 GQA
4k-context batch (256 sequences, lengths U{3072..4096}, 32 query / 8 KV heads,
head dim 128, block 16), drawn on the device from its seed.

Prints one JSON line.  ``value`` is the step's effective KV throughput: the
algorithmic bytes of one step (every cached K/V byte the batch attends to
read once, q and out, the tables, the new rows written) divided by the
wall-clock time per step.  ``roofline`` reports the decode launch alone,
timed with events recorded on the launch stream around it in every timed step.
``cpu_baseline`` times the fp64 oracle on the host on a bounded sample of the
same batch.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

With a prefill/extend workload (``--workload x2_prefill_bf16``,
``x3_extend_bf16`` or ``x6_long_extend_bf16``) the step is the slot write of
every new token followed by ``paged_attn_extend``, and ``value`` is the causal attention's TFLOP/s
against the bf16 matrix-core peak.
"""

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attention: effective KV GB/s (% HBM peak) + seqs/sec, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
DEFAULT_WORKLOAD = "c3_gqa4k_bf16"


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--part-tokens", type=int, default=None,
                   help="split-K partition length (default: the workload's, else the library's)")
    p.add_argument("--block-size", type=int, default=None,
                   help="run the batch with this block size instead of its own (same "
                        "lengths and values recipe, new placement)")
    p.add_argument("--cpu-sample", type=int, default=256,
                   help="sequences the oracle computes for the CPU baseline (0 skips it)")
    p.add_argument("--copy-probe", type=float, default=0.0, metavar="GIB",
                   help="instead of the decode step, time a plain device-to-device copy of "
                        "GIB GiB (the reference kernel for HBM byte counters)")
    p.add_argument("--cpu-oracle", default=None, help=argparse.SUPPRESS)
    return p.parse_args(argv)


def copy_probe(gib, steps, warmup):
    """Plain copy of a known size: its time gives a practical HBM ceiling and
    its counter readings the scale of FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = int(gib * (1 << 30))
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    print(json.dumps({"copy_bytes": n, "ms_per_copy": round(ms, 5),
                      "read_plus_write_GBps": round(2 * n / (ms * 1e-3) / 1e9, 1)}), flush=True)
    return 0


DECODE_SOURCES = ["paged_kv_cache_317_amd/csrc/attn_decode.hip",
                  "paged_kv_cache_317_amd/csrc/device_common.hpp",
                  "paged_kv_cache_317_amd/csrc/decode.hpp",
                  "paged_kv_cache_317_amd/csrc/pkv_api.cpp"]   # the run count
EXTEND_SOURCES = ["paged_kv_cache_317_amd/csrc/attn_extend.hip",
                  "paged_kv_cache_317_amd/csrc/device_common.hpp",
                  "paged_kv_cache_317_amd/csrc/extend.hpp"]
# Counter summaries per (kernel, workload): the HBM bytes per launch they
# record count only while the kernel sources hash to the recorded value.
PROFILES = {
    DEFAULT_WORKLOAD: ("paged_attn_decode_c3_gqa4k_bf16.md", DECODE_SOURCES),
    "c5_long_bf16": ("paged_attn_decode_c5_long_bf16.md", DECODE_SOURCES),
    "c1_tiny_f32": ("paged_attn_decode_c1_tiny_f32.md", DECODE_SOURCES),
    "c2_mha_bf16": ("paged_attn_decode_c2_mha_bf16.md", DECODE_SOURCES),
    "c4_prefix_bf16": ("paged_attn_decode_c4_prefix_bf16.md", DECODE_SOURCES),
    "x3_extend_bf16": ("paged_attn_extend_x3_extend_bf16.md", EXTEND_SOURCES),
    "x6_long_extend_bf16": ("paged_attn_extend_x6_long_extend_bf16.md", EXTEND_SOURCES),
    "x2_prefill_bf16": ("paged_attn_extend_x2_prefill_bf16.md", EXTEND_SOURCES),
    "x4_extend_g8_bs32_bf16": ("paged_attn_extend_x4_extend_g8_bs32_bf16.md", EXTEND_SOURCES),
}


def profiled_traffic(workload):
    """HBM bytes per launch of the workload's attention kernel from the
    committed counter summary, or None when there is none for this workload
    or the kernel sources changed since it was taken."""
    import hashlib
    import re
    if workload not in PROFILES:
        return None
    name, sources = PROFILES[workload]
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    traffic = re.search(r"traffic_bytes_per_launch:\s*(\d+)", text)
    if not sha or not traffic:
        return None
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return int(traffic.group(1)) if h.hexdigest() == sha.group(1) else None


def step_bytes(cfg, lens):
    """Algorithmic bytes of one decode launch and of one slot-write launch."""
    import numpy as np
    e = cfg.elem_bytes
    lens = np.asarray(lens, dtype=np.int64)
    blocks = -(-lens // cfg.block_size)
    kv = int(lens.sum()) * cfg.kv_heads * cfg.head_dim * e * 2
    qo = cfg.num_seqs * cfg.q_heads * cfg.head_dim * e * 2
    tables = int(blocks.sum()) * 4 + cfg.num_seqs * 4
    decode = kv + qo + tables
    write = cfg.num_seqs * (cfg.kv_heads * cfg.head_dim * e * 2 * 2 + 8)
    repeat = (cfg.num_seqs - 1) * cfg.prefix_tokens * cfg.kv_heads * cfg.head_dim * e * 2
    return {"decode": decode, "kv_read": kv, "kv_write": write,
            "shared_repeat": repeat if cfg.prefix_tokens else 0}


def host_array(t):
    """Device tensor -> numpy in the oracle's storage (uint16 bit patterns for bf16)."""
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def visible_cores():
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# A GPU machine's host share is 16 cores per GPU, whatever the affinity mask
# shows; the oracle timing uses the visible cores up to that share.
HOST_CORE_SHARE = 16


def host_workers():
    """Worker count for the oracle timing: the visible cores, at most the
    box's per-GPU share."""
    return max(1, min(visible_cores(), HOST_CORE_SHARE))


# The oracle's timing runs in a child Python process (this one has the GPU
# open; a fresh child does not inherit it), which forks one worker process
# per visible core.  The inputs travel as .npy files in memory-backed
# storage and are memory-mapped by the child and its workers.
_ORACLE = {}


def _oracle_task(share):
    """One worker's share: decode sequence indices, or extend query windows
    [lo, hi)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    a, job = _ORACLE["arrays"], _ORACLE["job"]
    with threadpool_limits(limits=1):
        if job["kind"] == "decode":
            oracle.decode_attention(a["q"], a["k_cache"], a["v_cache"], a["table"], a["lens"],
                                    job["scale"], job["dtype"], seqs=share)
        else:
            for lo, hi in share:
                # queries [lo, hi) are the new tokens of a sequence of length ctx0 + hi
                oracle.extend_attention(a["q"][lo:hi], a["k_cache"], a["v_cache"], a["table"],
                                        np.array([job["ctx0"] + hi]), np.array([0, hi - lo]),
                                        job["scale"], job["dtype"])
    return len(share)


def _noop(_):
    return 0


def cpu_oracle_child(job_path):
    """Child-process side: time the oracle on every worker, then on one core;
    prints one JSON line."""
    import multiprocessing as mp
    import numpy as np
    job = json.load(open(job_path))
    d = job["dir"]
    _ORACLE["job"] = job
    _ORACLE["arrays"] = {k: np.load(os.path.join(d, k + ".npy"), mmap_mode="r")
                         for k in job["arrays"]}
    items = job["items"]
    workers = job["workers"]
    shares = [items[i::workers] for i in range(workers)]
    with mp.get_context("fork").Pool(workers) as pool:
        pool.map(_noop, range(workers))            # workers started before the clock
        t0 = time.perf_counter()
        pool.map(_oracle_task, shares, chunksize=1)
        multi = time.perf_counter() - t0
    t0 = time.perf_counter()
    _oracle_task(job.get("whole", items))
    one = time.perf_counter() - t0
    print(json.dumps({"multi_s": multi, "one_s": one, "workers": workers}), flush=True)
    return 0


def run_cpu_oracle(kind, arrays, items, **job):
    """Parent side: hand the arrays to a child process and return its
    timings ({"multi_s", "one_s", "workers"})."""
    import shutil
    import subprocess
    import tempfile
    import numpy as np
    base = "/dev/shm" if os.access("/dev/shm", os.W_OK) else None
    d = tempfile.mkdtemp(prefix="pkv_oracle_", dir=base)
    try:
        for k, v in arrays.items():
            np.save(os.path.join(d, k + ".npy"), np.ascontiguousarray(v))
        job.update(kind=kind, dir=d, arrays=list(arrays), items=items,
                   workers=min(host_workers(), len(items)))
        path = os.path.join(d, "job.json")
        with open(path, "w") as f:
            json.dump(job, f)
        res = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-oracle", path],
                             capture_output=True, text=True, timeout=900)
        if res.returncode != 0:
            raise RuntimeError(f"oracle timing failed ({res.returncode}): {res.stderr[-2000:]}")
        return json.loads(res.stdout.strip().splitlines()[-1])
    finally:
        shutil.rmtree(d, ignore_errors=True)


def cpu_baseline(cfg, q, k_cache, v_cache, table, lens, nseq):
    """The oracle on the first ``nseq`` sequences of the batch: one worker
    process per visible core (one BLAS thread each, the sequences dealt out
    in turn), then one core."""
    import numpy as np
    nseq = min(nseq, cfg.num_seqs)
    t = run_cpu_oracle("decode", {"q": q, "k_cache": k_cache, "v_cache": v_cache,
                                  "table": table, "lens": np.asarray(lens)},
                       list(range(nseq)), scale=float(cfg.scale), dtype=cfg.dtype)
    dt, dt1, workers = t["multi_s"], t["one_s"], t["workers"]
    sub = np.asarray(lens[:nseq], dtype=np.int64)
    kv = int(sub.sum()) * cfg.kv_heads * cfg.head_dim * cfg.elem_bytes * 2
    return {
        "value": round(kv / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "workers": workers,
        "visible_cores": visible_cores(),
        "core_share": HOST_CORE_SHARE,
        "kind": "oracle",
        "seqs_per_s": round(nseq / dt, 3),
        "wall_s": round(dt, 3),
        "one_core": {"value": round(kv / dt1 / 1e9, 4), "seqs_per_s": round(nseq / dt1, 3),
                     "wall_s": round(dt1, 3)},
        "sample": f"first {nseq} of {cfg.num_seqs} sequences of the same batch (same pools), "
                  f"one decode step, fp64 numpy; {workers} worker processes with one BLAS "
                  f"thread each, then one core",
    }


def percentiles(ms):
    """p10 / median / p90 of per-step times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 5),
            "p50": round(float(np.percentile(a, 50)), 5),
            "p90": round(float(np.percentile(a, 90)), 5)}


def time_cache_ops(pkv, w, cfg, dev, per_graph=100, replays=5):
    """Slot write (one token per sequence) and a copy-on-write sized block
    copy (one block per sequence but the last, free source and destination
    blocks), each timed on its own.  The launches are captured in a HIP graph
    so that the figure is device time, not the host's launch rate; bytes are
    read + written."""
    import numpy as np
    import torch
    lay = w.layout
    res = {}

    def timed(fn, per_graph=per_graph):
        fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(replays):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / (replays * per_graph)

    row = cfg.kv_heads * cfg.head_dim * cfg.elem_bytes
    ms = timed(lambda: pkv.paged_kv_write(w.new_k, w.new_v, w.slot_mapping, w.k_cache, w.v_cache))
    nbytes = cfg.num_seqs * (row * 2 * 2 + 8)
    res["paged_kv_write"] = {"tokens": cfg.num_seqs, "us": round(ms * 1e3, 3),
                             "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    npairs = min(cfg.num_seqs - 1, lay.spare_blocks.size // 2)
    if npairs > 0:
        src = lay.spare_blocks[:npairs]
        dst = lay.spare_blocks[npairs:2 * npairs]
        pairs = torch.from_numpy(np.stack([src, dst], axis=1).astype(np.int64)).to(dev)
        ms = timed(lambda: pkv.paged_block_copy(pairs, w.k_cache, w.v_cache))
        nbytes = npairs * row * cfg.block_size * 2 * 2
        res["paged_block_copy"] = {"pairs": int(npairs), "us": round(ms * 1e3, 3),
                                   "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    # Swapping: scattered device blocks to a pinned host pool and back.
    nswap = min(1024, lay.num_blocks)
    shape = (nswap,) + tuple(w.k_cache.shape[1:])
    hk = torch.empty(shape, dtype=w.k_cache.dtype).pin_memory()
    hv = torch.empty(shape, dtype=w.v_cache.dtype).pin_memory()
    rng = np.random.default_rng(3)
    dev_ids = rng.choice(lay.num_blocks, size=nswap, replace=False)
    host_ids = np.arange(nswap)
    out_pairs = torch.from_numpy(np.stack([dev_ids, host_ids], 1).astype(np.int64)).to(dev)
    in_pairs = torch.from_numpy(np.stack([host_ids, dev_ids], 1).astype(np.int64)).to(dev)
    nbytes = nswap * row * cfg.block_size * 2
    for key, fn in (("paged_block_move_d2h",
                     lambda: pkv.paged_block_move(out_pairs, w.k_cache, w.v_cache, hk, hv)),
                    ("paged_block_move_h2d",
                     lambda: pkv.paged_block_move(in_pairs, hk, hv, w.k_cache, w.v_cache))):
        ms = timed(fn, per_graph=5)
        res[key] = {"blocks": int(nswap), "us": round(ms * 1e3, 3),
                    "GBps_host_link": round(nbytes / (ms * 1e-3) / 1e9, 1)}
    return res


def allocator_report(cfg, lay):
    """The batch's tables built through the native block manager (a shared
    prefix by fork), then one decode step of one-token appends; then the
    same pool filled with more sequences of the batch's lengths until the
    manager refuses (the concurrent capacity), against a max-length
    reservation of the same pool."""
    import numpy as np
    from paged_kv_cache_317_amd.block_manager import BlockManager, PkvError
    BS, S = cfg.block_size, cfg.num_seqs
    lens = lay.seq_lens.astype(np.int64)
    pre = cfg.prefix_tokens

    def populate(bm, count):
        """Add `count` sequences (lengths cycle through the batch); returns how
        many fit and the appended token count."""
        tokens = 0
        if pre:
            bm.add(-1)
            bm.append(-1, pre)
        for i in range(count):
            L = int(lens[i % S])
            try:
                if pre:
                    bm.fork(-1, i)
                    bm.append(i, L - pre)
                    tokens += L - pre
                else:
                    bm.add(i)
                    bm.append(i, L)
                    tokens += L
            except PkvError as e:
                if e.status_name != "PKV_ERR_NO_BLOCKS":
                    raise
                bm.free_sequence(i)
                return i, tokens
        return count, tokens

    bm = BlockManager(lay.num_blocks, BS)
    t0 = time.perf_counter()
    _, tokens = populate(bm, S)
    t_bulk = time.perf_counter() - t0
    t0 = time.perf_counter()
    for i in range(S):
        bm.append(i, 1)
    t_step = time.perf_counter() - t0
    st = bm.stats()
    cap, _ = populate(BlockManager(lay.num_blocks, BS), 1 << 30)
    return {
        "allocated_blocks": st["allocated_blocks"],
        "used_slots": st["used_slots"],
        "waste_fraction": round(st["waste_fraction"], 5),
        "contiguous_waste_fraction": round(1 - st["logical_tokens"] / (S * cfg.max_len), 5),
        "max_sequences_paged": cap,
        "max_sequences_contiguous": lay.num_blocks * BS // cfg.max_len,
        "append_ns_per_token": round(t_bulk / max(tokens, 1) * 1e9, 2),
        "decode_append_us": round(t_step / S * 1e6, 3),
        "prefix_cache": prefix_cache_report(cfg, lay),
    }


def prefix_cache_report(cfg, lay):
    """The batch's requests as token ids: a common system prompt (the batch's
    shared prefix, else 1024 tokens) then private tokens up to each length,
    started through the prefix cache of the native block manager (a lookup
    over the full blocks, then the rest stored with their token ids)."""
    import numpy as np
    from paged_kv_cache_317_amd.block_manager import BlockManager
    BS, S = cfg.block_size, cfg.num_seqs
    lens = lay.seq_lens.astype(np.int64)
    rng = np.random.default_rng(cfg.seed)
    common = int(cfg.prefix_tokens or min(1024, int(lens.min())))
    system = rng.integers(0, 32000, size=common).astype(np.int32)
    reqs = [np.concatenate([system, rng.integers(0, 32000, size=max(int(L) - common, 0))
                            .astype(np.int32)])[:int(L)] for L in lens]
    bm = BlockManager(lay.num_blocks, BS)
    t_lookup = t_store = 0.0
    reused = 0
    for i, toks in enumerate(reqs):
        t0 = time.perf_counter()
        n = bm.add_cached(i, toks)
        t1 = time.perf_counter()
        bm.append_tokens(i, toks[n:])
        t_store += time.perf_counter() - t1
        t_lookup += t1 - t0
        reused += n
    st = bm.stats()
    stored = int(lens.sum()) - reused
    return {
        "requests": S,
        "common_prefix_tokens": common,
        "reused_tokens": reused,
        "allocated_blocks": st["allocated_blocks"],
        "blocks_without_reuse": int(sum(-(-int(L) // BS) for L in lens)),
        "add_cached_us_per_request": round(t_lookup / S * 1e6, 2),
        "append_tokens_ns_per_token": round(t_store / max(stored, 1) * 1e9, 2),
    }


EXTEND_METRIC = "paged prefill/extend attention: causal TFLOP/s, 1 GPU"
FLUSH_BYTES = 1 << 30      # written between cold iterations to evict L2 and Infinity Cache
CPU_EXTEND_FLOPS = 2.5e11
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, published


def causal_work(lens, query_start, q_heads, head_dim):
    """(flops, query positions) of a prefill/extend batch: a query at
    position p takes p + 1 logits and as many weighted value rows per head,
    2 * head_dim flops each."""
    import numpy as np
    qs = np.asarray(query_start, dtype=np.int64)
    n = np.diff(qs)
    keys = 0
    for s in range(n.size):
        p = int(lens[s]) - int(n[s]) + np.arange(int(n[s]))
        keys += int(np.clip(p + 1, 0, None).sum())
    return keys * q_heads * 4 * head_dim, keys


def extend_bench(args):
    """Prefill / chunked-extend step: slot write of every new token, then the
    causal attention of all new tokens over the paged cache."""
    import numpy as np
    import torch

    import paged_kv_cache_317_amd as pkv
    from paged_kv_cache_317_amd.build import ensure_built
    from workloads import EXTEND_CONFIGS, generate_extend_device

    ensure_built()
    cfg = EXTEND_CONFIGS[args.workload]
    if args.block_size is not None:
        cfg = dataclasses.replace(cfg, block_size=args.block_size)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"# workload {cfg.name}: generating on {torch.cuda.get_device_name(dev)}",
          file=sys.stderr, flush=True)
    w = generate_extend_device(cfg, device=dev)
    lay = w.layout
    maxq, maxl = w.max_query_len, w.max_seq_len
    out = torch.empty_like(w.q)
    T = w.num_tokens
    part = pkv.extend_partition_tokens(w.k_cache, cfg.num_seqs, T, cfg.q_heads, maxq, maxl,
                                       args.part_tokens or 0)
    ws_bytes = pkv.extend_workspace_size(w.k_cache, cfg.num_seqs, T, cfg.q_heads, maxq, maxl,
                                         args.part_tokens or 0)
    workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    num_parts = -(-maxl // part)

    def write():
        pkv.paged_kv_write(w.new_k, w.new_v, w.slot_mapping, w.k_cache, w.v_cache)

    def attend():
        pkv.paged_attn_extend(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens,
                              w.query_start_dev, cfg.scale, maxq, maxl, out=out,
                              part_tokens=args.part_tokens or 0, workspace=workspace)

    for _ in range(args.warmup):
        write()
        attend()
    torch.cuda.synchronize()
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        write()
        ev[i][0].record()
        attend()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_list = [a.elapsed_time(b) for a, b in ev]
    attn_ms = float(np.mean(attn_list))
    step_ms = wall * 1e3 / K
    print(f"# {K} steps: {step_ms:.4f} ms/step, extend {attn_ms:.4f} ms", file=sys.stderr,
          flush=True)
    flops, _ = causal_work(lay.seq_lens, w.query_start, cfg.q_heads, cfg.head_dim)
    row = cfg.kv_heads * cfg.head_dim * cfg.elem_bytes
    kv_bytes = int(lay.seq_lens.astype(np.int64).sum()) * row * 2
    io_bytes = 2 * T * cfg.q_heads * cfg.head_dim * cfg.elem_bytes
    achieved = flops / (attn_ms * 1e-3) / 1e12

    cpu = None
    if args.cpu_sample > 0:
        # A bounded sample: the first new tokens of the shortest sequence, as
        # many as keep the causal work near CPU_EXTEND_FLOPS (10-30 s of the
        # fp64 oracle on one core).
        s = int(np.argmin(lay.seq_lens))
        qs = w.query_start
        n_new = int(qs[s + 1] - qs[s])
        ctx = int(lay.seq_lens[s]) - n_new
        nq = 1
        while nq < min(n_new, 1024) and causal_work(
                np.array([ctx + 2 * nq]), np.array([0, 2 * nq]), cfg.q_heads,
                cfg.head_dim)[0] <= CPU_EXTEND_FLOPS:
            nq *= 2
        nq = min(nq, n_new)
        q = host_array(w.q)[qs[s]:qs[s] + nq]
        kc, vc = host_array(w.k_cache), host_array(w.v_cache)
        L = int(lay.seq_lens[s])
        n_all = int(qs[s + 1] - qs[s])
        # the sample's own sequence: its first nq queries at their true positions
        lens = np.array([L - n_all + nq])
        sflops, _ = causal_work(lens, np.array([0, nq]), cfg.q_heads, cfg.head_dim)
        # One window of consecutive queries per worker, cut so that each
        # sees about the same number of keys; the one-core run is the whole
        # sample in one call.
        ctx0 = L - n_all
        nwin = min(host_workers(), nq)
        work = np.cumsum(ctx0 + np.arange(nq) + 1, dtype=np.float64)
        cuts = [0] + [int(np.searchsorted(work, work[-1] * k / nwin)) + 1
                      for k in range(1, nwin)] + [nq]
        windows = [[a, b] for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
        t = run_cpu_oracle("extend", {"q": q, "k_cache": kc, "v_cache": vc,
                                      "table": lay.block_table[s:s + 1]},
                           windows, scale=float(cfg.scale),
                           dtype=cfg.dtype, ctx0=ctx0, whole=[[0, nq]])
        dt, dt1, workers = t["multi_s"], t["one_s"], t["workers"]
        cpu = {"value": round(sflops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
               "workers": workers, "visible_cores": visible_cores(),
               "core_share": HOST_CORE_SHARE, "kind": "oracle", "wall_s": round(dt, 3),
               "one_core": {"value": round(sflops / dt1 / 1e12, 6), "wall_s": round(dt1, 3)},
               "sample": f"first {nq} new tokens of sequence {s} (length {L}) of the same "
                         f"batch, fp64 numpy; {workers} worker processes, one window of "
                         f"consecutive queries each, one BLAS thread each; then one core"}

    line = {
        "metric": EXTEND_METRIC,
        "value": round(achieved, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded, drawn on the device)",
        "config": {
            "workload": cfg.name,
            "num_seqs": cfg.num_seqs,
            "q_heads": cfg.q_heads,
            "kv_heads": cfg.kv_heads,
            "head_dim": cfg.head_dim,
            "block_size": cfg.block_size,
            "new_tokens": T,
            "seq_lens": [int(lay.seq_lens.min()), int(lay.seq_lens.max())],
            "pool_blocks": lay.num_blocks,
            "partition_tokens": part,
            "partitions": num_parts,
            "step": "paged_kv_write (every new token) + paged_attn_extend",
        },
        "tokens_per_s": round(T / (step_ms * 1e-3), 1),
        "extend_ms": round(attn_ms, 5),
        "extend_timing_ms": percentiles(attn_list),
        "roofline": {
            "bound": "mfma",
            "kernel": "paged_attn_extend" + (" (partition + merge)" if num_parts > 1 else ""),
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "flops_per_launch": flops,
            "kv_bytes_per_launch": kv_bytes + io_bytes,
            # the summaries were taken at the library's own partition choice
            "traffic": (profiled_traffic(cfg.name)
                        if not args.part_tokens and args.block_size is None else None),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    if args.cpu_oracle:
        return cpu_oracle_child(args.cpu_oracle)
    if args.copy_probe > 0:
        return copy_probe(args.copy_probe, args.steps, args.warmup)

    from workloads import EXTEND_CONFIGS
    if args.workload in EXTEND_CONFIGS:
        return extend_bench(args)

    import numpy as np
    import torch

    import paged_kv_cache_317_amd as pkv
    from paged_kv_cache_317_amd.build import ensure_built
    from workloads import generate_device, get_config, scaled

    ensure_built()
    cfg = get_config(args.workload)
    if args.part_tokens is not None:
        cfg = scaled(cfg, part_tokens=args.part_tokens)
    if args.block_size is not None:
        cfg = scaled(cfg, block_size=args.block_size)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"# workload {cfg.name}: generating on {torch.cuda.get_device_name(dev)}",
          file=sys.stderr, flush=True)
    w = generate_device(cfg, device=dev)
    lay = w.layout
    max_len = lay.max_seq_len
    out = torch.empty_like(w.q)
    ws_bytes = pkv.decode_workspace_size(w.k_cache, cfg.num_seqs, cfg.q_heads, max_len,
                                         cfg.part_tokens)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    part = pkv.decode_partition_tokens(w.k_cache, cfg.num_seqs, cfg.q_heads, max_len,
                                       cfg.part_tokens)
    runs = pkv.decode_runs(w.k_cache, cfg.num_seqs, cfg.q_heads, max_len, cfg.part_tokens)

    def write():
        pkv.paged_kv_write(w.new_k, w.new_v, w.slot_mapping, w.k_cache, w.v_cache)

    def decode():
        pkv.paged_attn_decode(w.q, w.k_cache, w.v_cache, w.block_table, w.seq_lens, cfg.scale,
                              max_len, out=out, part_tokens=cfg.part_tokens, workspace=ws)

    for _ in range(args.warmup):
        write()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    t0 = time.perf_counter()
    for i in range(K):
        write()
        ev[i][0].record()
        decode()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm_ms = [a.elapsed_time(b) for a, b in ev]
    decode_ms = float(np.mean(warm_ms))
    step_ms = wall * 1e3 / K
    print(f"# {K} steps: {step_ms:.4f} ms/step, decode {decode_ms:.4f} ms", file=sys.stderr,
          flush=True)

    # Cold figure, outside the timed steps: before each decode a 1 GiB write
    # evicts the L2 and the Infinity Cache.
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    for i in range(K):
        write()
        flush.fill_(i & 255)
        ev[i][0].record()
        decode()
        ev[i][1].record()
    torch.cuda.synchronize()
    cold_ms = [a.elapsed_time(b) for a, b in ev]
    del flush

    # The same decode over a second copy of the pools, allocated after the
    # first.  Where the driver places later allocations moves this gather by
    # a few percent; the headline keeps the pools as first allocated, as a
    # server allocating its cache at start-up would.
    k2, v2 = w.k_cache.clone(), w.v_cache.clone()
    torch.cuda.synchronize()
    for i in range(K):
        ev[i][0].record()
        pkv.paged_attn_decode(w.q, k2, v2, w.block_table, w.seq_lens, cfg.scale, max_len, out=out,
                              part_tokens=cfg.part_tokens, workspace=ws)
        ev[i][1].record()
    torch.cuda.synchronize()
    second_ms = [a.elapsed_time(b) for a, b in ev]
    del k2, v2

    nb = step_bytes(cfg, lay.seq_lens)
    step_total = nb["decode"] + nb["kv_write"]
    value = step_total / (step_ms * 1e-3) / 1e9
    # HBM has to deliver each stored row once: with a shared prefix the
    # roofline counts the prefix once (the effective figure counts it per
    # sequence).
    roof_bytes = nb["decode"] - nb["shared_repeat"]
    achieved = roof_bytes / (decode_ms * 1e-3) / 1e9
    warm = percentiles(warm_ms)
    cold = percentiles(cold_ms)
    second = percentiles(second_ms)
    decode_stats = {
        "warm_ms": warm, "cold_ms": cold, "second_allocation_ms": second,
        "second_allocation_GBps_mean": round(roof_bytes / (float(np.mean(second_ms)) * 1e-3) / 1e9,
                                             1),
        "warm_GBps_median": round(roof_bytes / (warm["p50"] * 1e-3) / 1e9, 1),
        "cold_GBps_median": round(roof_bytes / (cold["p50"] * 1e-3) / 1e9, 1),
        "flush_bytes": FLUSH_BYTES,
    }

    ops = time_cache_ops(pkv, w, cfg, dev)

    cpu = None
    if args.cpu_sample > 0:
        print(f"# cpu baseline: oracle on {args.cpu_sample} sequences", file=sys.stderr,
              flush=True)
        q, kc, vc = (host_array(t) for t in (w.q, w.k_cache, w.v_cache))
        cpu = cpu_baseline(cfg, q, kc, vc, lay.block_table, lay.seq_lens, args.cpu_sample)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded, drawn on the device)",
        "config": {
            "workload": cfg.name,
            "num_seqs": cfg.num_seqs,
            "q_heads": cfg.q_heads,
            "kv_heads": cfg.kv_heads,
            "head_dim": cfg.head_dim,
            "block_size": cfg.block_size,
            "seq_lens": [int(lay.seq_lens.min()), int(lay.seq_lens.max())],
            "pool_blocks": lay.num_blocks,
            "part_tokens": part,
            "runs": runs,
            "step": "paged_kv_write (one token per sequence) + paged_attn_decode",
        },
        "seqs_per_s": round(cfg.num_seqs / (step_ms * 1e-3), 1),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "decode_ms": round(decode_ms, 5),
        "decode_timing": decode_stats,
        "roofline": {
            "bound": "hbm",
            "kernel": "paged_attn_decode" + (" (stream + merge)" if runs > 1 else ""),
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "bytes_per_launch": roof_bytes,
            # the summaries were taken at each batch's own partition length
            # and block size
            "traffic": (profiled_traffic(cfg.name)
                        if args.part_tokens is None and args.block_size is None else None),
        },
        "cpu_baseline": cpu,
        "ops": ops,
        "allocator": allocator_report(cfg, lay),
    }
    if cfg.prefix_tokens:
        line["unique_bytes_per_launch"] = roof_bytes
        line["effective_decode_GBps"] = round(nb["decode"] / (decode_ms * 1e-3) / 1e9, 2)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
