"""The five synthetic workloads of the paged KV-cache hot path.

Each entry fixes the shapes, the element type and the length distributions;
``layout.py`` turns an entry into block tables with a seeded generator.  The
seed of workload k is k.
"""

from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    key: str                 # short name used by tests and the bench
    title: str               # what the workload is
    seed: int
    num_heads: int           # query heads Hq
    num_kv_heads: int        # KV heads Hkv
    head_dim: int
    dtype: str               # "f32" or "bf16"
    block_size: int = 16
    # decode part
    num_decode: int = 0
    decode_lens: Optional[Tuple[int, ...]] = None     # fixed lengths, or
    decode_range: Optional[Tuple[int, int]] = None    # inclusive uniform
    pool_blocks: Optional[int] = None  # fixed pool size (else 1.1x need)
    shared_prefix_blocks: int = 0      # blocks every decode table shares
    suffix_range: Optional[Tuple[int, int]] = None    # tokens after prefix
    # chunked-prefill part
    num_prefill: int = 0
    chunk_len: int = 0
    history_range: Optional[Tuple[int, int]] = None
    history_pinned: Tuple[int, ...] = field(default_factory=tuple)


CONFIGS = {
    "tiny": Config(
        key="tiny", seed=1,
        title="tiny decode: 4 seqs, ctx {7,16,33,100}, 8q/2kv, D=64, fp32",
        num_heads=8, num_kv_heads=2, head_dim=64, dtype="f32",
        num_decode=4, decode_lens=(7, 16, 33, 100), pool_blocks=64),
    "small": Config(
        key="small", seed=2,
        title="small-model decode: 64 seqs, ctx U[128,4096], 16q/8kv, "
              "D=128, bf16",
        num_heads=16, num_kv_heads=8, head_dim=128, dtype="bf16",
        num_decode=64, decode_range=(128, 4096)),
    "decode8b": Config(
        key="decode8b", seed=3,
        title="8B-shaped decode step: 256 seqs, ctx U[512,8192], 32q/8kv, "
              "D=128, bf16, store 256 rows then decode",
        num_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        num_decode=256, decode_range=(512, 8192)),
    "prefix": Config(
        key="prefix", seed=4,
        title="prefix-sharing decode: 128 seqs, shared 128-block prefix + "
              "U[1,512] private suffix, 32q/8kv, D=128, bf16",
        num_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        num_decode=128, shared_prefix_blocks=128, suffix_range=(1, 512)),
    "mixed": Config(
        key="mixed", seed=5,
        title="mixed chunked prefill + decode: 8 x 512-row chunks over "
              "U[0,8192] history + 192 decode rows ctx U[256,8192], "
              "32q/8kv, D=128, bf16",
        num_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
        num_decode=192, decode_range=(256, 8192),
        num_prefill=8, chunk_len=512, history_range=(0, 8192),
        history_pinned=(0, 8192)),
}


def get_config(key):
    if key not in CONFIGS:
        raise KeyError(f"unknown workload {key!r}; have {sorted(CONFIGS)}")
    return CONFIGS[key]
