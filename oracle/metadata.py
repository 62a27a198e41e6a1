"""Oracle: host-side metadata of a paged KV cache (plain Python loops).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Written from:
* "Warmup Guide -- Inference Serving Internals", Chapter 3 (PagedAttention):
  fixed-size blocks, a per-sequence block table of physical block ids, the
  ceil-division block count, and the rule that appending a token takes a new
  block exactly when the current length is a multiple of the block size.
* "3.6 ModelRunner, CUDA Graph, and benchmarks", section 2: how a batch of
  sequences becomes the slot mapping, cu_seqlens_q / cu_seqlens_k,
  max_seqlen_q / max_seqlen_k, context lengths and the -1 padded block-table
  matrix; section 4: the bytes of one KV block.
* "10 Serving Engines", section 10.2.3 worked example: bytes of KV cache per
  token for the Llama 3 8B shape.
* "Warmup Guide -- Inference Serving Internals", Chapter 4 (prefix sharing and
  copy-on-write): ref-counted blocks that several block tables name, and the
  rule that a write into a shared block first copies that one block.

Everything is done one token at a time with Python integers, so that each
line can be checked against the description by eye.
"""


def blocks_needed(num_tokens, block_size):
    """Number of blocks that hold ``num_tokens`` tokens: ceil division.

    Warmup Guide, Chapter 3: a sequence of n tokens occupies ceil(n / bs)
    blocks; 8 tokens in 4-slot blocks take 2 blocks.
    """
    if num_tokens < 0 or block_size <= 0:
        raise ValueError("num_tokens must be >= 0 and block_size > 0")
    count = 0
    while count * block_size < num_tokens:
        count += 1
    return count


def append_takes_new_block(length, block_size):
    """True when appending one token to a sequence of ``length`` tokens must
    first take a new block.

    Warmup Guide, Chapter 3: the last block is exactly full when the length
    is a multiple of the block size (an empty sequence has no block yet).
    """
    return length % block_size == 0


def grow_block_table(block_table, length, num_new, free_blocks, block_size):
    """Append ``num_new`` tokens one at a time, taking blocks from
    ``free_blocks`` (a list used as a stack, popped from the front) only when
    the append rule says so.  Returns the new (block_table, length).

    Warmup Guide, Chapter 3 (append) -- used by the tests to build tables that
    are consistent with the allocator.
    """
    table = list(block_table)
    for _ in range(num_new):
        if append_takes_new_block(length, block_size):
            if not free_blocks:
                raise MemoryError("block pool exhausted")
            table.append(free_blocks.pop(0))
        length += 1
    return table, length


def slot_of(block_table, position, block_size):
    """Physical slot of logical token ``position``: the block the block table
    names for that position, times the block size, plus the offset inside the
    block.  ModelRunner page, section 2 (prepare_prefill)."""
    block_id = block_table[position // block_size]
    return block_id * block_size + position % block_size


def prefill_metadata(seqs, block_size):
    """Tensorize a prefill (or chunked-prefill) batch.

    ``seqs`` is a list of dicts with keys ``block_table`` (list of physical
    block ids, may be empty for sequences that own no cache), ``num_cached``
    (tokens already in the cache) and ``num_scheduled`` (tokens computed this
    step).

    ModelRunner page, section 2 (prepare_prefill): the query side holds only
    the tokens of this step, [start, end); the key side covers [0, end);
    cu_seqlens_q / cu_seqlens_k are running sums of those two lengths; the
    slot of each token of this step follows the block table; a sequence
    without a block table writes no slots; block tables are needed as soon as
    the key total exceeds the query total (a prefix-cache hit or a chunked
    resume).
    """
    slot_mapping = []
    cu_q = [0]
    cu_k = [0]
    max_q = 0
    max_k = 0
    for seq in seqs:
        start = seq["num_cached"]
        end = start + seq["num_scheduled"]
        cu_q.append(cu_q[-1] + (end - start))
        cu_k.append(cu_k[-1] + end)
        max_q = max(max_q, end - start)
        max_k = max(max_k, end)
        if not seq["block_table"]:
            continue
        for pos in range(start, end):
            slot_mapping.append(slot_of(seq["block_table"], pos, block_size))
    return {
        "slot_mapping": slot_mapping,
        "cu_seqlens_q": cu_q,
        "cu_seqlens_k": cu_k,
        "max_seqlen_q": max_q,
        "max_seqlen_k": max_k,
        "needs_block_tables": cu_k[-1] > cu_q[-1],
    }


def decode_metadata(seqs, block_size):
    """Tensorize a decode batch (one new token per sequence).

    ``seqs`` is a list of dicts with keys ``block_table`` and ``length`` (the
    sequence length *including* the token being decoded; the allocator has
    already appended a block if that token crossed a boundary).

    ModelRunner page, section 2 (prepare_decode): the context length counts
    the new token; the new token is the last_block_num_tokens-th token of the
    last block, so its slot is last_block_id * bs + last_block_num_tokens - 1;
    the block tables are right-padded with -1 into one rectangular matrix.
    """
    slot_mapping = []
    context_lens = []
    for seq in seqs:
        table = seq["block_table"]
        length = seq["length"]
        last_block_num_tokens = length - (len(table) - 1) * block_size
        if not 1 <= last_block_num_tokens <= block_size:
            raise ValueError("block table does not match the sequence length")
        context_lens.append(length)
        slot_mapping.append(table[-1] * block_size + last_block_num_tokens - 1)
    width = max((len(s["block_table"]) for s in seqs), default=0)
    block_tables = []
    for seq in seqs:
        row = list(seq["block_table"])
        while len(row) < width:
            row.append(-1)
        block_tables.append(row)
    return {
        "slot_mapping": slot_mapping,
        "context_lens": context_lens,
        "block_tables": block_tables,
    }


def shared_prefix_groups(seqs, block_size):
    """Groups of consecutive decode sequences that share leading blocks.

    Warmup Guide, Chapter 4 (prefix sharing): sequences that start with the
    same tokens hold the same physical blocks for them (reference-counted,
    stored once); only full blocks are shared -- a write into a shared block
    copies it first.  This reading groups a batch for a decode that reads
    each shared block once per group:

    * a sequence's full blocks are its first length // block_size blocks;
    * two sequences share the leading full blocks whose ids are equal
      position by position, up to the first difference;
    * scanning the batch in order, a sequence that shares k >= 1 blocks with
      the next one starts a group with prefix k; the group takes every
      following consecutive sequence that shares at least those k blocks
      with the group's first sequence; every member's shared length is
      k * block_size tokens.  Sequences in no group have shared length 0.

    Returns (prefix_lens list [B], groups list of (first, count)).
    """
    def full_blocks(seq):
        return seq["length"] // block_size

    def shared(a, b):
        n = min(full_blocks(a), full_blocks(b))
        k = 0
        while k < n and a["block_table"][k] == b["block_table"][k]:
            k += 1
        return k

    prefix_lens = [0] * len(seqs)
    groups = []
    i = 0
    while i < len(seqs):
        k = shared(seqs[i], seqs[i + 1]) if i + 1 < len(seqs) else 0
        if k == 0:
            i += 1
            continue
        last = i + 1
        while last + 1 < len(seqs) and shared(seqs[i], seqs[last + 1]) >= k:
            last += 1
        for b in range(i, last + 1):
            prefix_lens[b] = k * block_size
        groups.append((i, last - i + 1))
        i = last + 1
    return prefix_lens, groups


def pad_decode_batch(meta, bucket):
    """Pad a decode batch to a captured-graph bucket size.

    ModelRunner page, section 5 (run_model): padding rows get slot -1 (the
    store skips them) and context length 0 (attention reads nothing); their
    block-table rows may hold anything and are never read.
    """
    n = len(meta["context_lens"])
    if bucket < n:
        raise ValueError("bucket smaller than the batch")
    width = len(meta["block_tables"][0]) if meta["block_tables"] else 0
    return {
        "slot_mapping": list(meta["slot_mapping"]) + [-1] * (bucket - n),
        "context_lens": list(meta["context_lens"]) + [0] * (bucket - n),
        "block_tables": [list(r) for r in meta["block_tables"]]
        + [[-1] * width for _ in range(bucket - n)],
    }


def internal_waste(length, block_size):
    """Unused slots in a sequence's last block (Warmup Guide, Chapter 3:
    bounded by block_size - 1)."""
    return blocks_needed(length, block_size) * block_size - length


def kv_block_bytes(num_layers, block_size, num_kv_heads, head_dim, itemsize,
                   tensor_parallel=1):
    """Bytes of one KV block across all layers: K and V, every layer, every
    slot of the block, this rank's KV heads, every head dimension.
    ModelRunner page, section 4 (block_bytes)."""
    if num_kv_heads % tensor_parallel:
        raise ValueError("KV heads must divide evenly over ranks")
    heads = num_kv_heads // tensor_parallel
    return 2 * num_layers * block_size * heads * head_dim * itemsize


def kv_bytes_per_token(num_layers, num_kv_heads, head_dim, itemsize):
    """Bytes of KV cache one token occupies across all layers (K and V).
    Warmup Guide, Chapter 2 (the KV size formula, per token and per
    sequence) and "10 Serving Engines", section 10.2.3."""
    return 2 * num_layers * num_kv_heads * head_dim * itemsize


class RefCountedPool:
    """A pool of physical blocks with a reference count per block.

    Warmup Guide, Chapter 4: a block several sequences share is one physical
    block named by several block tables, with a reference count; a sequence
    about to write into a block that others also hold first takes a fresh
    block, copies the shared block into it, lowers the shared block's count
    and writes into its private copy.  Freed blocks (count 0) return to the
    free list.  Free blocks are handed out from the front of the list.
    """

    def __init__(self, free_blocks):
        self.free = list(free_blocks)
        self.ref = {}

    def allocate(self):
        if not self.free:
            raise MemoryError("block pool exhausted")
        block = self.free.pop(0)
        self.ref[block] = 1
        return block

    def share(self, block_table):
        """A new sequence points at the same physical blocks (a prefix hit,
        or a fork): every block's count goes up by one."""
        for block in block_table:
            self.ref[block] += 1
        return list(block_table)

    def release(self, block_table):
        """A sequence ends: its blocks' counts go down; blocks no one holds
        any more return to the free list."""
        for block in block_table:
            self.ref[block] -= 1
            if self.ref[block] == 0:
                del self.ref[block]
                self.free.append(block)

    def append(self, block_table, length, block_size):
        """Make room for the token at position ``length`` of a sequence.

        A full last block (Chapter 3's rule) means a fresh block and no copy.
        Otherwise the token goes into the last block; if another sequence
        holds that block too, it is copied first (copy-on-write).  Returns
        (block_table, length + 1, slot of the new token, copy) where copy is
        (source block, destination block) or None.
        """
        table = list(block_table)
        copy = None
        if append_takes_new_block(length, block_size):
            table.append(self.allocate())
        else:
            last = table[-1]
            if self.ref[last] > 1:
                fresh = self.allocate()
                copy = (last, fresh)
                self.ref[last] -= 1
                table[-1] = fresh
        slot = slot_of(table, length, block_size)
        return table, length + 1, slot, copy
