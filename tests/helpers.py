"""Test helpers: moving seeded workloads to the GPU and comparing with the oracle."""

import sys

import numpy as np
import torch

import oracle

# Tolerances: fp32 caches max-abs 1e-5; bf16 caches max-abs 2e-2 and, per
# (sequence, head) row, max|err| / max(max|ref|, 1e-6) <= 1e-2.
F32_ATOL = 1e-5
BF16_ATOL = 2e-2
BF16_ROW_RTOL = 1e-2


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(arr, dtype, device="cuda"):
    """numpy array (float32, or uint16 bf16 bits, or ints) -> torch tensor on device."""
    if dtype == "bf16" and arr.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def to_host(t, dtype):
    """torch tensor -> numpy in the oracle's storage (uint16 bits for bf16)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def upload(w, device="cuda"):
    """Device copies of a host workload's arrays (dict of tensors)."""
    dt = w.cfg.dtype
    return {
        "q": to_device(w.q, dt, device),
        "k_cache": to_device(w.k_cache, dt, device),
        "v_cache": to_device(w.v_cache, dt, device),
        "new_k": to_device(w.new_k, dt, device),
        "new_v": to_device(w.new_v, dt, device),
        "slot_mapping": to_device(w.slot_mapping, None, device),
        "block_table": to_device(w.block_table, None, device),
        "seq_lens": to_device(w.seq_lens, None, device),
    }


def out_to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(got, ref, dtype, rows=None):
    """Assert the decode tolerance; returns (max_abs, max_row_rel).

    ``got`` is the device output, ``ref`` the oracle's float64 array; with
    ``rows`` only those sequence indices are compared.
    """
    g = out_to_f64(got)
    if rows is not None:
        g, ref = g[rows], ref[rows]
    assert np.all(np.isfinite(g)), "non-finite values in the GPU output"
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    D = ref.shape[-1]
    row_err = err.reshape(-1, D).max(axis=1) if err.size else np.zeros(0)
    row_ref = np.abs(ref).reshape(-1, D).max(axis=1) if err.size else np.zeros(0)
    row_rel = row_err / np.maximum(row_ref, 1e-6)
    max_rel = float(row_rel.max()) if row_rel.size else 0.0
    if dtype == "f32":
        assert max_abs <= F32_ATOL, f"fp32 max-abs {max_abs:.3e} > {F32_ATOL}"
    else:
        assert max_abs <= BF16_ATOL, f"bf16 max-abs {max_abs:.3e} > {BF16_ATOL}"
        assert max_rel <= BF16_ROW_RTOL, f"bf16 row max-rel {max_rel:.3e} > {BF16_ROW_RTOL}"
    return max_abs, max_rel


def oracle_decode(w, k_cache=None, v_cache=None, seq_lens=None, block_table=None, seqs=None):
    cfg = w.cfg
    return oracle.decode_attention(
        w.q, w.k_cache if k_cache is None else k_cache, w.v_cache if v_cache is None else v_cache,
        w.block_table if block_table is None else block_table,
        w.seq_lens if seq_lens is None else seq_lens, cfg.scale, cfg.dtype, seqs=seqs)


def drop_bad_blocks(block_table, seq_lens, block_size, num_blocks):
    """The table and lengths of the sequences with every block whose table
    entry lies outside the pool taken out (the decode rule for such entries:
    their positions do not count).  Attention does not depend on the order of
    positions, so the oracle on the result is the expected output.  Only the
    last block of a sequence is partial, so a dropped middle block removes
    block_size positions and a dropped last block the positions it held."""
    table = np.full_like(block_table, -1)
    lens = np.array(seq_lens, dtype=np.int32).copy()
    for s, L in enumerate(np.asarray(seq_lens).tolist()):
        nb = -(-int(L) // block_size)
        keep = []
        for j in range(nb):
            e = int(block_table[s, j])
            if 0 <= e < num_blocks:
                keep.append(e)
            else:
                lens[s] -= min(block_size, int(L) - j * block_size)
        table[s, :len(keep)] = keep
    return table, lens
