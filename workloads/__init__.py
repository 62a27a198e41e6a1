"""Seeded synthetic inputs for the paged KV-cache hot path.

This is the only module that both the oracle side (tests, CPU baseline) and
the HIP side (tests, bench) use.  It holds no arithmetic of the method: it
draws lengths, shuffles a pool of physical block ids into per-sequence block
tables, and fills tensors with normal random values.  It does not compute slot
mappings, cumulative lengths, padded block-table matrices or anything
attention computes; each side does that with its own code.

Distributions (all seeded; numpy ``Generator(PCG64(seed))`` for layouts,
``torch.Generator`` seeded the same way for values):
* lengths "uniform in [a, b]" are integers drawn inclusively;
* a block pool of NB ids is shuffled once and handed out in order, so a
  sequence's blocks are scattered over the pool;
* q, k, v and the whole cache pool are N(0, 1); bfloat16 values are float32
  normals rounded to nearest-even by the dtype cast.
"""

from .specs import CONFIGS, get_config  # noqa: F401
from .layout import (  # noqa: F401
    DecodeLayout, PrefillLayout, decode_layout, config_decode_layout,
    prefill_layout, mixed_layout, valid_slot_mask,
)
from .values import (  # noqa: F401
    make_values, fill_pool, poison_unused, host_bits, torch_dtype,
    make_codes, fill_pool_codes,
)
