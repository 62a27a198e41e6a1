"""Host-side metadata of a paged KV cache, as int32 arrays for the kernels.

This is the control-plane side of the hot path: it turns per-sequence block
tables and lengths into the tensors the C ABI takes.  Source: "3.6
ModelRunner, CUDA Graph, and benchmarks", section 2 (prepare_prefill /
prepare_decode) and section 5 (padding), and the "Warmup Guide -- Inference
Serving Internals", Chapter 3 (slot = block id * block size + offset).
Vectorised with numpy; nothing here runs on the GPU.
"""

import collections

import numpy as np


def block_table_matrix(tables, width=None, pad=-1):
    """Right-pad per-sequence block tables into one int32 matrix."""
    n = len(tables)
    w = max((len(t) for t in tables), default=0) if width is None else width
    out = np.full((n, max(w, 1)), pad, dtype=np.int32)
    for i, t in enumerate(tables):
        t = np.asarray(t, dtype=np.int64)
        if len(t) > w:
            raise ValueError("table longer than the matrix width")
        out[i, :len(t)] = t
    return out


def slots_for_positions(table, positions, block_size):
    """Physical slots of logical token positions of one sequence."""
    table = np.asarray(table, dtype=np.int64)
    positions = np.asarray(positions, dtype=np.int64)
    blocks = table[positions // block_size]
    return blocks * block_size + positions % block_size


def decode_inputs(tables, lens, block_size, width=None):
    """Decode batch: the token being decoded is position len-1 of each
    sequence (its context length counts it).

    Returns dict(slot_mapping int32 [B], context_lens int32 [B],
    block_tables int32 [B, W] padded with -1, max_context_len int).
    """
    lens = np.asarray(lens, dtype=np.int64)
    slots = np.empty(len(lens), dtype=np.int64)
    for i, (t, n) in enumerate(zip(tables, lens)):
        slots[i] = slots_for_positions(t, [n - 1], block_size)[0] if n > 0 \
            else -1
    return {
        "slot_mapping": slots.astype(np.int32),
        "context_lens": lens.astype(np.int32),
        "block_tables": block_table_matrix(tables, width),
        "max_context_len": int(lens.max()) if len(lens) else 0,
    }


def shared_prefix_inputs(tables, lens, block_size):
    """Sharing groups of a decode batch, for decode_shared_prefix: runs of
    consecutive sequences whose leading full blocks are the same physical
    blocks.  A sequence that shares k >= 1 full blocks with the next one
    opens a group with a k-block prefix; following sequences join while
    they share at least those k blocks with the group's first sequence.

    Returns dict(prefix_lens int32 [B] (k * block_size for members, 0
    otherwise), groups int32 [G, 2] (first, count), max_prefix_len,
    max_suffix_len, max_group_size).
    """
    lens = np.asarray(lens, dtype=np.int64)
    rows = [np.asarray(t, dtype=np.int64) for t in tables]
    full = lens // block_size

    def common(a, b):
        n = int(min(full[a], full[b]))
        diff = np.nonzero(rows[a][:n] != rows[b][:n])[0]
        return int(diff[0]) if len(diff) else n

    prefix = np.zeros(len(rows), dtype=np.int64)
    groups = []
    i = 0
    while i < len(rows):
        k = common(i, i + 1) if i + 1 < len(rows) else 0
        if k == 0:
            i += 1
            continue
        j = i + 1
        while j + 1 < len(rows) and common(i, j + 1) >= k:
            j += 1
        prefix[i:j + 1] = k * block_size
        groups.append((i, j - i + 1))
        i = j + 1
    g = np.asarray(groups, dtype=np.int32).reshape(-1, 2)
    return {
        "prefix_lens": prefix.astype(np.int32),
        "groups": g,
        "max_prefix_len": int(prefix.max()) if len(prefix) else 0,
        "max_suffix_len": int((lens - prefix).max()) if len(lens) else 0,
        "max_group_size": int(g[:, 1].max()) if len(g) else 0,
    }


def prefill_inputs(tables, num_cached, num_scheduled, block_size, width=None):
    """Chunked-prefill batch: sequence b computes tokens
    [num_cached[b], num_cached[b] + num_scheduled[b]) this step.

    Returns dict(slot_mapping int32 [total_q], cu_seqlens_q / cu_seqlens_k
    int32 [B+1], max_seqlen_q, max_seqlen_k, block_tables int32 [B, W],
    needs_block_tables bool).
    """
    cached = np.asarray(num_cached, dtype=np.int64)
    sched = np.asarray(num_scheduled, dtype=np.int64)
    ends = cached + sched
    cu_q = np.concatenate([[0], np.cumsum(sched)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(ends)]).astype(np.int32)
    parts = [slots_for_positions(t, np.arange(c, e), block_size)
             for t, c, e in zip(tables, cached, ends) if len(t)]
    slots = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    return {
        "slot_mapping": slots.astype(np.int32),
        "cu_seqlens_q": cu_q,
        "cu_seqlens_k": cu_k,
        "max_seqlen_q": int(sched.max()) if len(sched) else 0,
        "max_seqlen_k": int(ends.max()) if len(ends) else 0,
        "block_tables": block_table_matrix(tables, width),
        "needs_block_tables": bool(cu_k[-1] > cu_q[-1]),
    }


class BlockPool:
    """Physical blocks with reference counts: prefix sharing, fork and
    copy-on-write ("Warmup Guide -- Inference Serving Internals", Chapters 3
    and 4).

    A block named by several block tables is stored once; its count says how
    many tables name it.  Appending a token that falls into a block others
    also hold first moves the appender onto a private copy of that block:
    the pool hands out a fresh block, records (shared, fresh) as a copy for
    ``pa_copy_blocks`` to carry out, and lowers the shared block's count.
    Blocks whose count drops to zero return to the free list.

    Tables are Python lists of block ids; this class is host bookkeeping only.
    """

    def __init__(self, num_blocks, order=None):
        ids = np.arange(num_blocks) if order is None else np.asarray(order)
        self.refs = np.zeros(num_blocks, dtype=np.int64)
        self._free = collections.deque(int(b) for b in ids)

    @property
    def num_free(self):
        return len(self._free)

    def _take(self):
        if not self._free:
            raise MemoryError("no free block")
        blk = self._free.popleft()
        self.refs[blk] = 1
        return blk

    def share(self, table):
        """A second table naming the same blocks (a prefix hit or a fork)."""
        if len(table):
            np.add.at(self.refs, np.asarray(table, dtype=np.int64), 1)
        return list(table)

    def release(self, table):
        """Drop one table's hold on its blocks."""
        for blk in table:
            self.refs[blk] -= 1
            if self.refs[blk] == 0:
                self._free.append(int(blk))

    def append_slots(self, tables, lens, block_size):
        """Room for one new token at the end of every sequence of a batch.

        ``tables`` (lists, updated in place) and ``lens`` (token counts before
        the append) describe the batch.  Returns (slot_mapping int32 [B],
        copies int32 [C, 2]): the slot each new token is stored at, and the
        (source, destination) block copies that must run before the store.
        """
        slots = np.empty(len(tables), dtype=np.int32)
        copies = []
        for i, (table, n) in enumerate(zip(tables, lens)):
            n = int(n)
            off = n % block_size
            if off == 0:                      # last block full, or no block
                table.append(self._take())
            elif self.refs[table[-1]] > 1:    # shared partial block: copy it
                shared = table[-1]
                fresh = self._take()
                self.refs[shared] -= 1
                copies.append((shared, fresh))
                table[-1] = fresh
            slots[i] = table[-1] * block_size + off
        pairs = np.asarray(copies, dtype=np.int32).reshape(-1, 2)
        return slots, pairs
