"""The oracle's pins catch plausible mistakes: each case plants one mistake
(a dropped term, a wrong index, a swapped operand) in a copy of ``oracle/``
in a scratch directory and runs the pins of that module against the copy;
the run must fail.  The repository's own oracle is never touched."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (module, text to replace (first occurrence), replacement, pin file)
MUTATIONS = {
    "decode scale dropped": (
        "attention.py", "x = scale64 * (K[:, g, :] @ qs[h])", "x = (K[:, g, :] @ qs[h])",
        "test_oracle_attention.py"),
    "decode head mapping h mod kv_heads": (
        "attention.py", "            g = h // G\n            x = scale64 * (K[:, g, :] @ qs[h])",
        "            g = h % Hkv\n            x = scale64 * (K[:, g, :] @ qs[h])",
        "test_oracle_attention.py"),
    "decode weights applied to K": (
        "attention.py", "out[s, h] = (p @ V[:, g, :]) / p.sum()",
        "out[s, h] = (p @ K[:, g, :]) / p.sum()", "test_oracle_attention.py"),
    "decode last token dropped": (
        "attention.py",
        "        K = widen(gather_sequence(k_cache, block_table[s], L, BS), dtype)\n"
        "        V = widen(gather_sequence(v_cache, block_table[s], L, BS), dtype)",
        "        K = widen(gather_sequence(k_cache, block_table[s], max(L - 1, 1), BS), dtype)\n"
        "        V = widen(gather_sequence(v_cache, block_table[s], max(L - 1, 1), BS), dtype)",
        "test_oracle_attention.py"),
    "decode normaliser perturbed": (
        "attention.py", "out[s, h] = (p @ V[:, g, :]) / p.sum()",
        "out[s, h] = (p @ V[:, g, :]) / (p.sum() + 1e-3)", "test_oracle_attention.py"),
    "gather offset shifted": (
        "attention.py", "    offset = t % block_size", "    offset = (t + 1) % block_size",
        "test_oracle_attention.py"),
    "gather block index off at block end": (
        "attention.py", "    logical = t // block_size",
        "    logical = t // block_size + (t % block_size == block_size - 1)",
        "test_oracle_attention.py"),
    "merge without max rescale": (
        "attention.py", "    w = np.exp(m - M)\n", "    w = np.ones_like(m)\n",
        "test_oracle_attention.py"),
    "partition sum wrong on one partition": (
        "attention.py", "        l[p] = e.sum()\n", "        l[p] = e.sum() + (p == 1)\n",
        "test_oracle_attention.py"),
    "extend query does not see itself": (
        "extend.py", "visible = np.arange(L)[None, :] <= pos[:, None]",
        "visible = np.arange(L)[None, :] < pos[:, None]", "test_oracle_extend.py"),
    "extend positions ignore the context": (
        "extend.py", "pos = L - n + np.arange(n)", "pos = np.arange(n)", "test_oracle_extend.py"),
    "extend head mapping h mod kv_heads": (
        "extend.py", "            g = h // G\n            x = scale64 * (Q[:, h, :] @ K[:, g, :].T)",
        "            g = h % Hkv\n            x = scale64 * (Q[:, h, :] @ K[:, g, :].T)",
        "test_oracle_extend.py"),
    "extend flops halved": (
        "extend.py", "    return total * q_heads * 4 * head_dim",
        "    return total * q_heads * 2 * head_dim", "test_oracle_extend.py"),
    "slot write swaps K and V": (
        "cache_ops.py", "        k_cache[block, offset] = k[i]\n        v_cache[block, offset] = v[i]",
        "        k_cache[block, offset] = v[i]\n        v_cache[block, offset] = k[i]",
        "test_oracle_bf16_and_ops.py"),
    "slot decode swapped": (
        "cache_ops.py", "        block, offset = divmod(slot, block_size)",
        "        offset, block = divmod(slot, block_size)", "test_oracle_bf16_and_ops.py"),
    "block move writes K rows into V": (
        "cache_ops.py", "    out_v[dst] = v_rows\n", "    out_v[dst] = k_rows\n",
        "test_oracle_bf16_and_ops.py"),
    "block move reads the block after the source": (
        "cache_ops.py", "    k_rows = src_k[src].copy()\n",
        "    k_rows = src_k[np.minimum(src + 1, src_k.shape[0] - 1)].copy()\n",
        "test_oracle_bf16_and_ops.py"),
    "block copy skips V": (
        "cache_ops.py", "    k_cache[dst] = k_src\n    v_cache[dst] = v_src",
        "    k_cache[dst] = k_src", "test_oracle_bf16_and_ops.py"),
    "blocks_for rounds down": (
        "block_manager.py", "    return -(-length // block_size)", "    return length // block_size",
        "test_oracle_block_manager.py"),
    "freed block never returns to the pool": (
        "block_manager.py", "            self.fill[b] = 0\n            self.free.append(b)",
        "            self.fill[b] = 0", "test_oracle_block_manager.py"),
    "shared block written without a copy": (
        "block_manager.py", "                if self.refcount[b] > 1:",
        "                if self.refcount[b] > 99:", "test_oracle_block_manager.py"),
    "copy-on-write keeps the old reference": (
        "block_manager.py",
        "                    self.fill[nb] = self.fill[b]\n                    self.refcount[b] -= 1",
        "                    self.fill[nb] = self.fill[b]", "test_oracle_block_manager.py"),
    "fork does not share": (
        "block_manager.py", "        for b in self.tables[child]:\n            self.refcount[b] += 1",
        "        self.tables[child] = [self._take() for _ in self.tables[child]]",
        "test_oracle_block_manager.py"),
    "prefix hit does not take a reference": (
        "block_manager.py", "            self.refcount[b] += 1\n            self.tables[seq].append(b)",
        "            self.tables[seq].append(b)", "test_oracle_block_manager.py"),
    "prefix entry outlives its block": (
        "block_manager.py", "            if key is not None:\n                del self.cache[key]",
        "            pass", "test_oracle_block_manager.py"),
    "swap-in fills every block": (
        "block_manager.py", "            self.fill[b] = min(BS, length - j * BS)",
        "            self.fill[b] = BS", "test_oracle_block_manager.py"),
    "waste counts the used slots": (
        "block_manager.py", '"unused_slots": slots - used,', '"unused_slots": used,',
        "test_oracle_block_manager.py"),
    "bf16 widening shift wrong": (
        "bf16.py", "        word = a.astype(np.uint32) << np.uint32(16)",
        "        word = a.astype(np.uint32) << np.uint32(15)", "test_oracle_bf16_and_ops.py"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_a_planted_mistake_fails_the_pins(name, tmp_path):
    module, old, new, pins = MUTATIONS[name]
    # scratch repository: the oracle (mutated), the pins and the input
    # generators; the package and the built library come from ROOT
    for d in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    target = tmp_path / "oracle" / module
    src = target.read_text()
    assert old in src, f"mutation pattern no longer in oracle/{module}"
    target.write_text(src.replace(old, new, 1))
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", os.path.join("tests", pins)],
                       cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"the pins passed with '{name}' planted:\n{r.stdout[-1500:]}"
