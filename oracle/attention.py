"""Oracle: slot scatter, block-table gather and attention in float64.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Cache layout (ModelRunner page, section 4): one layer's K cache and V cache
are each an array [num_blocks, block_size, num_kv_heads, head_dim]; viewed
flat they are [num_slots, num_kv_heads, head_dim] with
slot = block_id * block_size + offset.

Element types.  ``"f32"`` arrays are numpy float32.  ``"bf16"`` arrays are
numpy uint16 holding the raw bfloat16 bits (numpy has no bfloat16); a bfloat16
is the top half of a float32, so shifting the bits left by 16 and viewing the
result as float32 converts it exactly.  All arithmetic is float64.

Attention (not spelled out on the pages, which only name the kernels):
out = softmax(scale * q K^T) V over the keys a query row may see, computed
directly with a max-subtracted exponent.  Readings taken where the pages are
silent:
* GQA: query head h reads KV head h // G with G = Hq / Hkv (contiguous
  groups).  Parity unpinned by the pages for this mapping.
* Causal alignment when the key side is longer than the query side (chunked
  prefill or a prefix hit): bottom-right, i.e. query row i of a sequence with
  Lq query rows and Lk keys sits at absolute position Lk - Lq + i and sees
  keys 0 .. Lk - Lq + i.  The ModelRunner page, section 2, has query
  positions continue from the number of cached tokens while keys start at 0.
* A decode row attends to its own new token: the context length counts it and
  the store runs before attention (ModelRunner page, section 2).
* A row with context length 0 (batch padding, section 5) gives zeros.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Exact bfloat16 -> float64: place the 16 bits in the high half of a
    float32 and widen."""
    bits = np.asarray(bits, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def to_f64(arr, dtype):
    """Widen an input array of the given element type to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def store_kv(k_cache, v_cache, k, v, slot_mapping):
    """Scatter new K/V rows into copies of the caches, bit for bit.

    ModelRunner page, section 2 (slot_mapping) and section 5 (padding): row t
    of k and v is written whole (all KV heads, all dims) to flat slot
    slot_mapping[t]; a negative slot (padding) writes nothing.  Returns new
    (k_cache, v_cache) arrays; the inputs are not modified.  Works on the raw
    element bits, so the comparison with a GPU cache can be bytewise.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    num_blocks, block_size, hkv, d = k_out.shape
    flat_k = k_out.reshape(num_blocks * block_size, hkv, d)
    flat_v = v_out.reshape(num_blocks * block_size, hkv, d)
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        if slot >= num_blocks * block_size:
            raise IndexError(f"slot {slot} outside the cache")
        flat_k[slot] = k[t]
        flat_v[slot] = v[t]
    return k_out, v_out


def copy_blocks(k_cache, v_cache, pairs):
    """Copy whole blocks, bit for bit: for each (source, destination) pair
    block ``destination`` of both caches becomes a copy of block
    ``source``.  Warmup Guide, Chapter 4: copy-on-write copies the one
    shared block a sequence is about to write into.  A pair with an id
    outside the pool is skipped.  Returns new arrays; the inputs are not
    modified.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    num_blocks = k_out.shape[0]
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks):
            continue
        k_out[dst] = k_cache[src]
        v_out[dst] = v_cache[src]
    return k_out, v_out


def gather_sequence_kv(k_cache, v_cache, block_table, length, dtype):
    """Gather one sequence's first ``length`` tokens of K and V through its
    block table into contiguous float64 arrays [length, Hkv, D].

    Warmup Guide, Chapter 3: logical token t lives in the block the table
    names at index t // bs, at offset t % bs.  Only the first
    ceil(length / bs) table entries are read; anything after them (-1
    padding or stale ids, ModelRunner page, sections 2 and 5) is never
    touched.
    """
    block_size = k_cache.shape[1]
    hkv, d = k_cache.shape[2], k_cache.shape[3]
    keys = np.empty((length, hkv, d), dtype=np.float64)
    values = np.empty((length, hkv, d), dtype=np.float64)
    for t in range(length):
        block_id = int(block_table[t // block_size])
        offset = t % block_size
        if block_id < 0 or block_id >= k_cache.shape[0]:
            raise IndexError(f"block id {block_id} outside the pool")
        keys[t] = to_f64(k_cache[block_id, offset], dtype)
        values[t] = to_f64(v_cache[block_id, offset], dtype)
    return keys, values


def attend(q_rows, keys, values, scale, visible):
    """softmax(scale * q K^T) V for a group of query rows sharing K and V.

    q_rows [R, D], keys / values [N, D] (float64), ``visible[r]`` = number of
    leading keys row r may see (0 <= visible[r] <= N).  Returns
    (out [R, D], probs [R, N]) with probs zero on hidden keys.  A row that sees
    no key gives a zero output and a zero probability row.
    """
    rows = q_rows.shape[0]
    n = keys.shape[0]
    out = np.zeros((rows, values.shape[1]), dtype=np.float64)
    probs = np.zeros((rows, n), dtype=np.float64)
    if n == 0:
        return out, probs
    logits = scale * (q_rows @ keys.T)
    for r in range(rows):
        m = int(visible[r])
        if m == 0:
            continue
        row = logits[r, :m]
        e = np.exp(row - row.max())
        p = e / e.sum()
        probs[r, :m] = p
        out[r] = p @ values[:m]
    return out, probs


def decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale,
                     dtype, return_probs=False, seqs=None):
    """Decode attention: one query row per sequence against its paged
    context.

    q [B, Hq, D]; caches [NB, bs, Hkv, D]; block_tables [B, W] (-1 padded);
    context_lens [B] (counts the new token; 0 -> zero row).  Returns float64
    out [B, Hq, D] (and, if asked, a list of per-sequence probability arrays
    [Hq, L_b]).  ``seqs`` restricts the work to the listed sequences (other
    rows stay zero), for sampled checks at full size.
    """
    q64 = to_f64(q, dtype)
    b_count, hq, d = q64.shape
    hkv = k_cache.shape[2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    out = np.zeros((b_count, hq, d), dtype=np.float64)
    all_probs = [None] * b_count
    for b in (range(b_count) if seqs is None else seqs):
        length = int(context_lens[b])
        probs_b = np.zeros((hq, length), dtype=np.float64)
        if length > 0:
            keys, values = gather_sequence_kv(k_cache, v_cache,
                                              block_tables[b], length, dtype)
            for h in range(hq):
                g = h // group
                o, p = attend(q64[b, h][None, :], keys[:, g, :],
                              values[:, g, :], scale, [length])
                out[b, h] = o[0]
                probs_b[h] = p[0]
        all_probs[b] = probs_b
    if return_probs:
        return out, all_probs
    return out


def prefill_attention(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k,
                      block_tables, scale, causal, dtype, seqs=None,
                      rows=None):
    """Varlen (chunked) prefill attention with K/V read through block tables.

    q [total_q, Hq, D] packed end to end (ModelRunner page, section 2):
    sequence b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and
    Lk = cu_seqlens_k[b+1] - cu_seqlens_k[b] keys, read from the cache through
    block_tables[b].  With ``causal``, query row i of the sequence sees keys
    0 .. Lk - Lq + i (bottom-right); requires Lq <= Lk.  Without it every row
    sees all Lk keys.

    Returns float64 out [total_q, Hq, D].  ``seqs`` restricts the work to
    some sequences; ``rows`` (a dict b -> list of local row indices)
    restricts it further to some rows.
    """
    q64 = to_f64(q, dtype)
    total_q, hq, d = q64.shape
    hkv = k_cache.shape[2]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = hq // hkv
    out = np.zeros((total_q, hq, d), dtype=np.float64)
    num_seqs = len(cu_seqlens_q) - 1
    for b in (range(num_seqs) if seqs is None else seqs):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        lq = q1 - q0
        lk = int(cu_seqlens_k[b + 1]) - int(cu_seqlens_k[b])
        if lq == 0:
            continue
        if causal and lq > lk:
            raise ValueError("causal prefill needs Lq <= Lk")
        keys, values = gather_sequence_kv(k_cache, v_cache, block_tables[b],
                                          lk, dtype)
        local = list(range(lq)) if rows is None or b not in rows else rows[b]
        if causal:
            visible = [lk - lq + i + 1 for i in local]
        else:
            visible = [lk] * len(local)
        for h in range(hq):
            g = h // group
            o, _ = attend(q64[q0 + np.asarray(local, dtype=np.int64), h],
                          keys[:, g, :], values[:, g, :], scale, visible)
            out[q0 + np.asarray(local, dtype=np.int64), h] = o
    return out
