"""paged_kv_cache_slot_amd: the paged KV-cache hot path on MI355X (gfx950).

* ``ops``      -- torch-tensor calls into libpa (store_kv, decode,
                  prefill_varlen); every step runs in hand-written HIP
                  kernels, with no CPU fallback.
* ``metadata`` -- host-side slot mappings, cu_seqlens and padded block
                  tables for a batch.
* ``build``    -- compiles libpa.so for gfx950.
"""

from . import metadata  # noqa: F401
from ._lib import PaError, load as load_library  # noqa: F401


def __getattr__(name):
    # ops imports torch; keep ``import paged_kv_cache_slot_amd`` light.
    if name == "ops":
        import importlib
        return importlib.import_module(__name__ + ".ops")
    raise AttributeError(name)
