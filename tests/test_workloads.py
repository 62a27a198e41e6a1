"""The seeded workloads have the shapes and structure their titles state."""

import numpy as np
import pytest

import workloads as wl


def _check_tables(tables, lens, bs, nb, shared=0):
    seen = {}
    for i, (t, n) in enumerate(zip(tables, lens)):
        assert len(t) == -(-int(n) // bs)
        assert np.all((t >= 0) & (t < nb))
        for j, blk in enumerate(t.tolist()):
            if j < shared:
                continue
            assert blk not in seen, "private block used twice"
            seen[blk] = i


@pytest.mark.parametrize("key", ["tiny", "small", "decode8b", "prefix"])
def test_decode_layouts(key):
    cfg = wl.get_config(key)
    lay = wl.config_decode_layout(cfg)
    assert len(lay.lens) == cfg.num_decode
    if cfg.decode_lens:
        assert lay.lens.tolist() == list(cfg.decode_lens)
        assert lay.num_blocks == cfg.pool_blocks
    elif cfg.decode_range:
        lo, hi = cfg.decode_range
        assert lay.lens.min() >= lo and lay.lens.max() <= hi
    _check_tables(lay.tables, lay.lens, cfg.block_size, lay.num_blocks,
                  cfg.shared_prefix_blocks)
    if cfg.shared_prefix_blocks:
        first = lay.tables[0][:cfg.shared_prefix_blocks]
        for t in lay.tables:
            assert np.array_equal(t[:cfg.shared_prefix_blocks], first)
        suffix = lay.lens - cfg.shared_prefix_blocks * cfg.block_size
        assert suffix.min() >= 1 and suffix.max() <= 512
    # same seed, same layout
    again = wl.config_decode_layout(cfg)
    assert np.array_equal(again.lens, lay.lens)


def test_mixed_layout():
    cfg = wl.get_config("mixed")
    pre, dec = wl.mixed_layout(cfg)
    assert pre.history.tolist()[:2] == [0, 8192]
    assert np.all(pre.chunk == 512)
    assert pre.history.max() <= 8192 and pre.history.min() >= 0
    assert len(dec.lens) == 192
    assert dec.lens.min() >= 256 and dec.lens.max() <= 8192
    both = list(pre.tables) + list(dec.tables)
    lens = list(pre.history + pre.chunk) + list(dec.lens)
    _check_tables(both, lens, 16, pre.num_blocks)


def test_valid_mask_and_poison():
    import torch
    lay = wl.decode_layout([5, 16, 17], 16, seed=3, num_blocks=6)
    mask = wl.valid_slot_mask(lay.num_blocks, 16, lay.tables, lay.lens)
    assert mask.sum() == 5 + 16 + 17
    k, v = wl.fill_pool(6, 16, 2, 8, "bf16", seed=1)
    wl.poison_unused(k, v, mask)
    assert torch.isnan(k[~torch.as_tensor(mask)].float()).all()
    assert not torch.isnan(k[torch.as_tensor(mask)].float()).any()
