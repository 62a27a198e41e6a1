"""Planted mistakes in the oracle must each fail at least one pin.

Each mutation below is a copy of one oracle function with one plausible
mistake (a dropped term, a wrong sign or index, a swapped operand, a wrong
alignment).  It is swapped in with monkeypatch, on the CPU, and the full pin
set is run: if every pin still passed, the pins would not be able to tell the
mistake from the real thing.
"""

import numpy as np
import pytest

import oracle.attention as oa
import oracle.metadata as om
from tests import oracle_pins


def _attend_factory(drop_scale=False, no_normalize=False, no_max=False,
                    use_keys_as_values=False):
    def attend(q_rows, keys, values, scale, visible):
        rows = q_rows.shape[0]
        n = keys.shape[0]
        out = np.zeros((rows, values.shape[1]))
        probs = np.zeros((rows, n))
        if n == 0:
            return out, probs
        s = 1.0 if drop_scale else scale
        logits = s * (q_rows @ keys.T)
        with np.errstate(all="ignore"):
            for r in range(rows):
                m = int(visible[r])
                if m == 0:
                    continue
                row = logits[r, :m]
                e = np.exp(row if no_max else row - row.max())
                p = e if no_normalize else e / e.sum()
                probs[r, :m] = p
                src = keys if use_keys_as_values else values
                out[r] = p @ src[:m]
        return out, probs
    return attend


def _gather_off_by_one(k_cache, v_cache, block_table, length, dtype):
    bs = k_cache.shape[1]
    keys = np.empty((length,) + k_cache.shape[2:])
    values = np.empty((length,) + k_cache.shape[2:])
    for t in range(length):
        blk = int(block_table[t // bs])
        off = (t + 1) % bs                      # planted: wrong offset
        keys[t] = oa.to_f64(k_cache[blk, off], dtype)
        values[t] = oa.to_f64(v_cache[blk, off], dtype)
    return keys, values


def _gather_physical_order(k_cache, v_cache, block_table, length, dtype):
    bs = k_cache.shape[1]
    used = sorted(int(b) for b in block_table[:-(-length // bs)])
    keys = np.empty((length,) + k_cache.shape[2:])
    values = np.empty((length,) + k_cache.shape[2:])
    for t in range(length):
        blk = used[t // bs]                     # planted: physical order
        keys[t] = oa.to_f64(k_cache[blk, t % bs], dtype)
        values[t] = oa.to_f64(v_cache[blk, t % bs], dtype)
    return keys, values


def _decode_gqa_modulo(q, k_cache, v_cache, block_tables, context_lens,
                       scale, dtype, return_probs=False, seqs=None):
    q64 = oa.to_f64(q, dtype)
    bcount, hq, d = q64.shape
    hkv = k_cache.shape[2]
    out = np.zeros((bcount, hq, d))
    probs_all = [None] * bcount
    for b in range(bcount):
        length = int(context_lens[b])
        probs = np.zeros((hq, length))
        if length:
            keys, values = oa.gather_sequence_kv(k_cache, v_cache,
                                                 block_tables[b], length,
                                                 dtype)
            for h in range(hq):
                g = h % hkv                         # planted: wrong mapping
                o, p = oa.attend(q64[b, h][None], keys[:, g], values[:, g],
                                 scale, [length])
                out[b, h] = o[0]
                probs[h] = p[0]
        probs_all[b] = probs
    return (out, probs_all) if return_probs else out


def _prefill_top_left(q, k_cache, v_cache, cu_q, cu_k, block_tables, scale,
                      causal, dtype, seqs=None, rows=None):
    q64 = oa.to_f64(q, dtype)
    total, hq, d = q64.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    out = np.zeros((total, hq, d))
    for b in range(len(cu_q) - 1):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        lq, lk = q1 - q0, int(cu_k[b + 1]) - int(cu_k[b])
        if lq == 0:
            continue
        keys, values = oa.gather_sequence_kv(k_cache, v_cache,
                                             block_tables[b], lk, dtype)
        vis = [i + 1 for i in range(lq)] if causal else [lk] * lq  # planted
        for h in range(hq):
            o, _ = oa.attend(q64[q0:q1, h], keys[:, h // group],
                             values[:, h // group], scale, vis)
            out[q0:q1, h] = o
    return out


_ORIG_DECODE_META = om.decode_metadata
_ORIG_PREFILL_META = om.prefill_metadata


def _decode_meta_no_minus_one(seqs, block_size):
    meta = _ORIG_DECODE_META(seqs, block_size)
    meta["slot_mapping"] = [s + 1 for s in meta["slot_mapping"]]  # planted
    return meta


def _prefill_meta_cu_k_wrong(seqs, block_size):
    meta = _ORIG_PREFILL_META(seqs, block_size)
    cu_k = [0]
    for s in seqs:                                   # planted: k = q lengths
        cu_k.append(cu_k[-1] + s["num_scheduled"])
    meta["cu_seqlens_k"] = cu_k
    meta["needs_block_tables"] = cu_k[-1] > meta["cu_seqlens_q"][-1]
    return meta


def _store_no_skip(k_cache, v_cache, k, v, slot_mapping):
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    nb, bs = k_out.shape[:2]
    fk = k_out.reshape(nb * bs, *k_out.shape[2:])
    fv = v_out.reshape(nb * bs, *v_out.shape[2:])
    for t, slot in enumerate(list(slot_mapping)):
        fk[slot] = k[t]                              # planted: no skip
        fv[slot] = v[t]
    return k_out, v_out


def _blocks_floor(num_tokens, block_size):
    return num_tokens // block_size                  # planted: floor


_ORIG_POOL_APPEND = om.RefCountedPool.append


def _pool_append_never_copies(self, block_table, length, block_size):
    table = list(block_table)
    if om.append_takes_new_block(length, block_size):
        table.append(self.allocate())
    # planted: writes into a shared block without copying it
    return table, length + 1, om.slot_of(table, length, block_size), None


def _pool_append_no_decrement(self, block_table, length, block_size):
    table = list(block_table)
    copy = None
    if om.append_takes_new_block(length, block_size):
        table.append(self.allocate())
    elif self.ref[table[-1]] > 1:
        fresh = self.allocate()
        copy = (table[-1], fresh)                    # planted: no decrement
        table[-1] = fresh
    return table, length + 1, om.slot_of(table, length, block_size), copy


def _pool_share_no_count(self, block_table):
    return list(block_table)                         # planted: no ref bump


def _copy_blocks_reversed(k_cache, v_cache, pairs):
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for src, dst in pairs:
        if min(src, dst) < 0 or max(src, dst) >= k_out.shape[0]:
            continue
        k_out[src] = k_cache[dst]                    # planted: reversed
        v_out[src] = v_cache[dst]
    return k_out, v_out


_orig_shared_groups = om.shared_prefix_groups


def _shared_groups_counts_partial(seqs, block_size):
    """Counts the partially filled last block as shareable."""
    rounded = [{"block_table": s["block_table"],
                "length": -(-s["length"] // block_size) * block_size} for s in seqs]
    return _orig_shared_groups(rounded, block_size)


def _shared_groups_greedy_shrink(seqs, block_size):
    """Lets the group's shared length shrink as members join."""
    lens, groups = _orig_shared_groups(seqs, block_size)
    if len(groups) > 1 and groups[0][0] + groups[0][1] == groups[1][0]:
        first, count = groups[0]
        merged = (first, count + groups[1][1])
        k = min(lens[first], lens[groups[1][0]])
        for b in range(first, first + merged[1]):
            lens[b] = k
        groups = [merged] + groups[2:]
    return lens, groups


import oracle.fp8 as of8  # noqa: E402

_orig_e4m3_encode = of8.e4m3_encode
_orig_e4m3_value = of8.e4m3_value


def _e4m3_round_half_up(v):
    """Rounds halfway cases away from zero instead of to even."""
    code = _orig_e4m3_encode(v)
    a = abs(float(v))
    if a != a or a >= 448.0:
        return code
    nxt = _orig_e4m3_value((code & 0x7F) + 1) if (code & 0x7F) < 0x7E else None
    here = abs(_orig_e4m3_value(code))
    if nxt is not None and a - here == nxt - a:
        return (code & 0x80) | ((code & 0x7F) + 1)
    return code


def _e4m3_no_saturation(v):
    """Lets values past 448 become the NaN code."""
    if abs(float(v)) > 464.0:
        return (0x80 if v < 0 else 0) | 0x7F
    return _orig_e4m3_encode(v)


def _e4m3_subnormal_exponent(code):
    """Gives subnormals the exponent of the smallest normal binade."""
    if (code >> 3) & 0xF == 0 and code & 7:
        s = -1.0 if code & 0x80 else 1.0
        return s * (1 + (code & 7) / 8.0) * 2.0 ** -7
    return _orig_e4m3_value(code)


_orig_dequantize = of8.dequantize
_orig_quantize = of8.quantize
_orig_fp8_decode = of8.decode_attention


def _dequantize_no_scale(codes, scale):
    """Forgets the per-cache scale."""
    return _orig_dequantize(codes, 1.0)


def _quantize_divides(x, inv_scale):
    """Divides by the inverse scale instead of multiplying."""
    return _orig_quantize(x, 1.0 / inv_scale)


def _fp8_decode_swapped_scales(q, k_codes, v_codes, block_tables, context_lens,
                               scale, k_scale, v_scale, *args, **kwargs):
    """Applies the V scale to K and the K scale to V."""
    return _orig_fp8_decode(q, k_codes, v_codes, block_tables, context_lens,
                            scale, v_scale, k_scale, *args, **kwargs)


_orig_fp8_store = of8.store_kv


def _fp8_store_swapped_scales(k_cache, v_cache, k, v, slot_mapping,
                              k_inv_scale, v_inv_scale, src_dtype):
    """Quantises K with the V inverse scale and V with the K one."""
    return _orig_fp8_store(k_cache, v_cache, k, v, slot_mapping, v_inv_scale,
                           k_inv_scale, src_dtype)


def _fp8_store_slot_split(k_cache, v_cache, k, v, slot_mapping, k_inv_scale,
                          v_inv_scale, src_dtype):
    """Splits the flat slot with the head count instead of the block size."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    split = k_out.shape[2]                      # planted: Hkv, not bs
    k32 = oa.to_f64(k, src_dtype).astype(np.float32)
    v32 = oa.to_f64(v, src_dtype).astype(np.float32)
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0:
            continue
        k_out[slot // split % k_out.shape[0], slot % split] = \
            of8.quantize(k32[t], k_inv_scale)
        v_out[slot // split % k_out.shape[0], slot % split] = \
            of8.quantize(v32[t], v_inv_scale)
    return k_out, v_out


def _fp8_store_no_skip(k_cache, v_cache, k, v, slot_mapping, k_inv_scale,
                       v_inv_scale, src_dtype):
    """Writes the rows of -1 slots too (numpy wraps -1 to the last slot)."""
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    bs = k_out.shape[1]
    k32 = oa.to_f64(k, src_dtype).astype(np.float32)
    v32 = oa.to_f64(v, src_dtype).astype(np.float32)
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)                        # planted: no skip of < 0
        k_out[slot // bs, slot % bs] = of8.quantize(k32[t], k_inv_scale)
        v_out[slot // bs, slot % bs] = of8.quantize(v32[t], v_inv_scale)
    return k_out, v_out


MUTATIONS = {
    "drop_scale": (oa, "attend", _attend_factory(drop_scale=True)),
    "no_normalize": (oa, "attend", _attend_factory(no_normalize=True)),
    "no_max_subtract": (oa, "attend", _attend_factory(no_max=True)),
    "keys_as_values": (oa, "attend", _attend_factory(use_keys_as_values=True)),
    "gather_offset": (oa, "gather_sequence_kv", _gather_off_by_one),
    "gather_physical_order": (oa, "gather_sequence_kv",
                              _gather_physical_order),
    "gqa_modulo": (oa, "decode_attention", _decode_gqa_modulo),
    "causal_top_left": (oa, "prefill_attention", _prefill_top_left),
    "decode_slot": (om, "decode_metadata", _decode_meta_no_minus_one),
    "prefill_cu_k": (om, "prefill_metadata", _prefill_meta_cu_k_wrong),
    "store_no_skip": (oa, "store_kv", _store_no_skip),
    "blocks_floor": (om, "blocks_needed", _blocks_floor),
    "cow_never_copies": (om.RefCountedPool, "append", _pool_append_never_copies),
    "cow_no_decrement": (om.RefCountedPool, "append", _pool_append_no_decrement),
    "share_no_count": (om.RefCountedPool, "share", _pool_share_no_count),
    "copy_blocks_reversed": (oa, "copy_blocks", _copy_blocks_reversed),
    "shared_counts_partial": (om, "shared_prefix_groups",
                              _shared_groups_counts_partial),
    "shared_group_shrinks": (om, "shared_prefix_groups",
                             _shared_groups_greedy_shrink),
    "e4m3_round_half_up": (of8, "e4m3_encode", _e4m3_round_half_up),
    "e4m3_no_saturation": (of8, "e4m3_encode", _e4m3_no_saturation),
    "e4m3_subnormal_exponent": (of8, "e4m3_value", _e4m3_subnormal_exponent),
    "fp8_dequantize_no_scale": (of8, "dequantize", _dequantize_no_scale),
    "fp8_quantize_divides": (of8, "quantize", _quantize_divides),
    "fp8_decode_swapped_scales": (of8, "decode_attention",
                                  _fp8_decode_swapped_scales),
    "fp8_store_swapped_scales": (of8, "store_kv", _fp8_store_swapped_scales),
    "fp8_store_slot_split": (of8, "store_kv", _fp8_store_slot_split),
    "fp8_store_no_skip": (of8, "store_kv", _fp8_store_no_skip),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    module, attr, bad = MUTATIONS[name]
    monkeypatch.setattr(module, attr, bad)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check()
        except Exception as exc:  # noqa: BLE001 - any failure counts
            failed.append((check.__name__, type(exc).__name__))
    assert failed, f"planted mistake {name!r} passed every pin"
