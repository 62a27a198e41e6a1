"""Host-side metadata of a paged KV cache, as int32 arrays for the kernels.

This is the control-plane side of the hot path: it turns per-sequence block
tables and lengths into the tensors the C ABI takes.  Source: "3.6
ModelRunner, CUDA Graph, and benchmarks", section 2 (prepare_prefill /
prepare_decode) and section 5 (padding), and the "Warmup Guide -- Inference
Serving Internals", Chapter 3 (slot = block id * block size + offset).
Vectorised with numpy; nothing here runs on the GPU.
"""

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


def prefill_inputs(tables, num_cached, num_scheduled, block_size, width=None):
    """Chunked-prefill batch: sequence b computes tokens
    [num_cached[b], num_cached[b] + num_scheduled[b]) this round.

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
