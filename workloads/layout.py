"""Seeded block-table layouts.

A layout says which physical blocks each sequence owns, in logical order, and
how many tokens it holds.  The pool of ``num_blocks`` ids is shuffled once
and dealt out in order, so blocks of one sequence are scattered.  The number
of blocks a sequence of n tokens owns is ceil(n / block_size) -- that is the
shape of the input, not something the kernels compute.
"""

from dataclasses import dataclass
from typing import List, Optional

import numpy as np

from .specs import Config


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _nblocks(n, bs):
    return -(-int(n) // bs)


@dataclass
class DecodeLayout:
    """Decode batch: sequence b holds ``lens[b]`` tokens (the newest one
    included) in blocks ``tables[b]``."""
    lens: np.ndarray            # int64 [B]
    tables: List[np.ndarray]    # int64, len(tables[b]) == ceil(lens[b]/bs)
    num_blocks: int
    block_size: int


@dataclass
class PrefillLayout:
    """Chunked-prefill batch: sequence b has ``history[b]`` cached tokens and
    ``chunk[b]`` tokens computed this round; ``tables[b]`` covers both."""
    history: np.ndarray         # int64 [P]
    chunk: np.ndarray           # int64 [P]
    tables: List[np.ndarray]
    num_blocks: int
    block_size: int


def _deal(rng, counts, num_blocks, shared_blocks=0):
    """Shuffle range(num_blocks) and deal ``counts[i]`` private ids to each
    table after ``shared_blocks`` ids common to all tables."""
    need = shared_blocks + int(sum(counts))
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} blocks < {need} needed")
    pool = rng.permutation(num_blocks).astype(np.int64)
    shared = pool[:shared_blocks]
    pos = shared_blocks
    tables = []
    for c in counts:
        tables.append(np.concatenate([shared, pool[pos:pos + c]]))
        pos += c
    return tables


def _pool_size(total, fixed):
    if fixed is not None:
        return int(fixed)
    return int(np.ceil(1.1 * total))


def decode_layout(lens, block_size, seed, num_blocks=None, shared_prefix=0):
    """Explicit decode layout.  ``shared_prefix`` blocks (full, at the start
    of every table) are common to all sequences; ``lens`` then counts the
    whole sequence, prefix included."""
    rng = _rng(seed)
    lens = np.asarray(lens, dtype=np.int64)
    prefix_tokens = shared_prefix * block_size
    if shared_prefix and np.any(lens <= prefix_tokens):
        raise ValueError("every sequence must extend past the shared prefix")
    counts = [_nblocks(n - prefix_tokens, block_size) for n in lens]
    nb = _pool_size(shared_prefix + sum(counts), num_blocks)
    tables = _deal(rng, counts, nb, shared_prefix)
    return DecodeLayout(lens=lens, tables=tables, num_blocks=nb,
                        block_size=block_size)


def _draw_decode_lens(cfg: Config, rng):
    if cfg.decode_lens is not None:
        return np.asarray(cfg.decode_lens, dtype=np.int64)
    if cfg.suffix_range is not None:
        lo, hi = cfg.suffix_range
        suffix = rng.integers(lo, hi, size=cfg.num_decode, endpoint=True)
        return cfg.shared_prefix_blocks * cfg.block_size + suffix
    lo, hi = cfg.decode_range
    return rng.integers(lo, hi, size=cfg.num_decode, endpoint=True)


def config_decode_layout(cfg: Config) -> DecodeLayout:
    """The decode layout of a decode-only workload."""
    if cfg.num_prefill:
        raise ValueError("use mixed_layout for a workload with prefill rows")
    rng = _rng(cfg.seed)
    lens = _draw_decode_lens(cfg, rng)
    return decode_layout(lens, cfg.block_size, seed=cfg.seed + 1000,
                         num_blocks=cfg.pool_blocks,
                         shared_prefix=cfg.shared_prefix_blocks)


def prefill_layout(history, chunk, block_size, seed, num_blocks=None):
    """Explicit chunked-prefill layout: tables cover history + chunk."""
    rng = _rng(seed)
    history = np.asarray(history, dtype=np.int64)
    chunk = np.asarray(chunk, dtype=np.int64)
    counts = [_nblocks(h + c, block_size) for h, c in zip(history, chunk)]
    nb = _pool_size(sum(counts), num_blocks)
    tables = _deal(rng, counts, nb)
    return PrefillLayout(history=history, chunk=chunk, tables=tables,
                         num_blocks=nb, block_size=block_size)


def mixed_layout(cfg: Config):
    """Chunked-prefill sequences and decode sequences sharing one pool.

    History lengths are uniform in ``history_range`` with the first entries
    pinned to ``history_pinned`` (so both ends of the range occur).  Returns
    (PrefillLayout, DecodeLayout) with one common ``num_blocks``.
    """
    rng = _rng(cfg.seed)
    lo, hi = cfg.history_range
    history = rng.integers(lo, hi, size=cfg.num_prefill, endpoint=True)
    for i, h in enumerate(cfg.history_pinned[:cfg.num_prefill]):
        history[i] = h
    chunk = np.full(cfg.num_prefill, cfg.chunk_len, dtype=np.int64)
    dlens = _draw_decode_lens(cfg, rng)
    bs = cfg.block_size
    pcounts = [_nblocks(h + c, bs) for h, c in zip(history, chunk)]
    dcounts = [_nblocks(n, bs) for n in dlens]
    nb = _pool_size(sum(pcounts) + sum(dcounts), cfg.pool_blocks)
    tables = _deal(_rng(cfg.seed + 1000), pcounts + dcounts, nb)
    pre = PrefillLayout(history=history.astype(np.int64), chunk=chunk,
                        tables=tables[:cfg.num_prefill], num_blocks=nb,
                        block_size=bs)
    dec = DecodeLayout(lens=dlens.astype(np.int64),
                       tables=tables[cfg.num_prefill:], num_blocks=nb,
                       block_size=bs)
    return pre, dec


def valid_slot_mask(num_blocks, block_size, tables, lens):
    """Boolean [num_blocks, block_size]: True where some sequence keeps a
    token (block i of a table holds tokens i*bs .. i*bs+bs-1 of that
    sequence, up to its length).  Used to poison everything else."""
    mask = np.zeros((num_blocks, block_size), dtype=bool)
    for table, n in zip(tables, lens):
        n = int(n)
        for i, blk in enumerate(np.asarray(table).tolist()):
            filled = min(block_size, n - i * block_size)
            if filled <= 0:
                break
            mask[blk, :filled] = True
    return mask
