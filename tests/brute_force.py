"""A second, independent implementation of paged attention in pure Python.

Lists, ``math.exp`` and ``math.fsum`` only -- no numpy -- for tiny inputs.
It pins the numpy oracle: the two are written differently (this one walks
block tables by hand and sums with exact-rounded fsum) and must agree to
1e-12.  Test helper only.
"""

import math


def _row(cache, slot, head, block_size):
    block, off = divmod(slot, block_size)
    return [float(x) for x in cache[block][off][head]]


def brute_attend(q, key_rows, value_rows, scale):
    """softmax(scale * q.k) v over the given rows (lists of floats)."""
    if not key_rows:
        return [0.0] * len(q)
    logits = [scale * math.fsum(a * b for a, b in zip(q, k)) for k in key_rows]
    top = max(logits)
    weights = [math.exp(s - top) for s in logits]
    total = math.fsum(weights)
    dim = len(value_rows[0])
    return [math.fsum(w * v[j] for w, v in zip(weights, value_rows)) / total
            for j in range(dim)]


def brute_decode(q, k_cache, v_cache, block_tables, context_lens, scale):
    """q[b][h][d] nested lists; caches nested [NB][bs][Hkv][D]."""
    block_size = len(k_cache[0])
    hkv = len(k_cache[0][0])
    out = []
    for b, qb in enumerate(q):
        hq = len(qb)
        group = hq // hkv
        length = context_lens[b]
        rows = []
        for h in range(hq):
            g = h // group
            keys, vals = [], []
            for t in range(length):
                blk = block_tables[b][t // block_size]
                slot = blk * block_size + t % block_size
                keys.append(_row(k_cache, slot, g, block_size))
                vals.append(_row(v_cache, slot, g, block_size))
            rows.append(brute_attend(qb[h], keys, vals, scale))
        out.append(rows)
    return out


def brute_prefill(q, k_cache, v_cache, cu_q, cu_k, block_tables, scale,
                  causal):
    """q[row][h][d] packed rows; returns the same nesting."""
    block_size = len(k_cache[0])
    hkv = len(k_cache[0][0])
    out = [None] * len(q)
    for b in range(len(cu_q) - 1):
        lq = cu_q[b + 1] - cu_q[b]
        lk = cu_k[b + 1] - cu_k[b]
        for i in range(lq):
            r = cu_q[b] + i
            hq = len(q[r])
            group = hq // hkv
            last = lk - lq + i if causal else lk - 1
            rows = []
            for h in range(hq):
                g = h // group
                keys, vals = [], []
                for t in range(last + 1):
                    blk = block_tables[b][t // block_size]
                    slot = blk * block_size + t % block_size
                    keys.append(_row(k_cache, slot, g, block_size))
                    vals.append(_row(v_cache, slot, g, block_size))
                rows.append(brute_attend(q[r][h], keys, vals, scale))
            out[r] = rows
    return out


def brute_store(k_cache, v_cache, k, v, slot_mapping):
    """Element-by-element scatter on nested lists (deep copies)."""
    import copy
    kc = copy.deepcopy(k_cache)
    vc = copy.deepcopy(v_cache)
    block_size = len(kc[0])
    for t, slot in enumerate(slot_mapping):
        if slot < 0:
            continue
        blk, off = divmod(slot, block_size)
        for h in range(len(k[t])):
            for d in range(len(k[t][h])):
                kc[blk][off][h][d] = k[t][h][d]
                vc[blk][off][h][d] = v[t][h][d]
    return kc, vc


def f32_round(x):
    """Nearest float32 to a Python float (ties to even), via the IEEE
    single-precision packing of the struct module."""
    import struct
    return struct.unpack("f", struct.pack("f", x))[0]


def nearest_code(a, values):
    """Code of the magnitude ``a`` (>= 0, already saturated) by exhaustive
    search over ``values`` -- values[c] is the value of code c, c = 0..126,
    the non-negative finite codes -- nearest value first, and between two
    equally near codes the even one (an even code has an even last
    mantissa bit)."""
    best, best_d = None, None
    for c, val in enumerate(values):
        d = abs(a - val)
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best


def brute_store_fp8(k_codes, v_codes, k, v, slot_mapping, k_inv_scale,
                    v_inv_scale, values, max_value):
    """Quantising scatter, one element at a time, on nested lists.

    Row t goes to flat slot slot_mapping[t] (block slot // bs, offset
    slot % bs; a negative slot writes nothing).  Element x becomes the code
    of p = float32(x * inv_scale): sign bit 0x80 if p is negative (also -0),
    magnitude min(|p|, max_value) matched by ``nearest_code``.  ``values``
    lists the non-negative finite code values (taken from a library's
    decoding, not from the oracle)."""
    import copy
    kc = copy.deepcopy(k_codes)
    vc = copy.deepcopy(v_codes)
    block_size = len(kc[0])
    for t, slot in enumerate(slot_mapping):
        if slot < 0:
            continue
        blk, off = divmod(slot, block_size)
        for cache, rows, inv in ((kc, k, k_inv_scale), (vc, v, v_inv_scale)):
            for h in range(len(rows[t])):
                for d in range(len(rows[t][h])):
                    p = f32_round(rows[t][h][d] * inv)
                    sign = 0x80 if math.copysign(1.0, p) < 0 else 0
                    mag = min(abs(p), max_value)
                    cache[blk][off][h][d] = sign | nearest_code(mag, values)
    return kc, vc
