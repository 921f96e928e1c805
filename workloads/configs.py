"""The five decode workloads, as frozen records.

The pages name no dataset or benchmark; these synthetic batches stand in for
the serving workloads they describe (block size 16 as the pages' example,
scattered physical placement, shared prefixes, long contexts).

    c1_tiny_f32      4 sequences, lengths {35, 16, 1, 100}, 8/8 heads, D 64,
                     fp32 N(0,1), block 16, a 32-block pool, scale 1/8.
    c2_mha_bf16      64 sequences, lengths U{1..2048}, 32/32 heads, D 128,
                     bf16 N(0,1), block 16, pool 1.25x the need.
    c3_gqa4k_bf16    256 sequences, lengths U{3072..4096}, 32/8 heads, D 128,
                     bf16 N(0, sd 0.5), block 16, pool 1.25x the need.
    c4_prefix_bf16   128 sequences sharing a 1024-token prefix (64 blocks,
                     reference count 128) + private suffix U{1..512},
                     32/8 heads, D 128, bf16 N(0,1), block 16.
    c5_long_bf16     16 sequences, lengths U{65536..131072}, 64/8 heads,
                     D 128, bf16 N(0,1), block 32, split into 512-token
                     partitions.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    q_heads: int
    kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "f32" or "bf16"
    std: float                      # standard deviation of q, K and V draws
    seed: int
    seq_lens: tuple = ()            # fixed lengths (overrides len_range)
    len_range: tuple = (1, 1)       # inclusive uniform range of lengths
    prefix_tokens: int = 0          # shared prefix length (0: no sharing)
    max_len: int = 0                # table width = ceil(max_len / block_size)
    pool_blocks: int = 0            # fixed pool size (0: pool_factor x need)
    pool_factor: float = 1.25
    part_tokens: int = 0            # split-K partition length (0: library picks)

    @property
    def group(self):
        return self.q_heads // self.kv_heads

    @property
    def table_width(self):
        return -(-self.max_len // self.block_size)

    @property
    def scale(self):
        return self.head_dim ** -0.5

    @property
    def elem_bytes(self):
        return 4 if self.dtype == "f32" else 2


CONFIGS = {
    "c1_tiny_f32": DecodeConfig(
        name="c1_tiny_f32", num_seqs=4, q_heads=8, kv_heads=8, head_dim=64,
        block_size=16, dtype="f32", std=1.0, seed=317_001,
        seq_lens=(35, 16, 1, 100), max_len=112, pool_blocks=32),
    "c2_mha_bf16": DecodeConfig(
        name="c2_mha_bf16", num_seqs=64, q_heads=32, kv_heads=32, head_dim=128,
        block_size=16, dtype="bf16", std=1.0, seed=317_002,
        len_range=(1, 2048), max_len=2048),
    "c3_gqa4k_bf16": DecodeConfig(
        name="c3_gqa4k_bf16", num_seqs=256, q_heads=32, kv_heads=8, head_dim=128,
        block_size=16, dtype="bf16", std=0.5, seed=317_003,
        len_range=(3072, 4096), max_len=4096),
    "c4_prefix_bf16": DecodeConfig(
        name="c4_prefix_bf16", num_seqs=128, q_heads=32, kv_heads=8, head_dim=128,
        block_size=16, dtype="bf16", std=1.0, seed=317_004,
        len_range=(1, 512), prefix_tokens=1024, max_len=1536),
    "c5_long_bf16": DecodeConfig(
        name="c5_long_bf16", num_seqs=16, q_heads=64, kv_heads=8, head_dim=128,
        block_size=32, dtype="bf16", std=1.0, seed=317_005,
        len_range=(65536, 131072), max_len=131072, part_tokens=512),
}


def get_config(name):
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None


def scaled(cfg, **changes):
    """A copy of ``cfg`` with some fields changed (smaller parity cases)."""
    return replace(cfg, **changes)
