"""Pins of the oracle: checks against facts that do not come from the oracle.

Each ``check_*`` function raises AssertionError when the oracle disagrees with
what the pages print, a closed form, an invariant of the mathematics, or the
independent pure-Python brute force.  ``test_oracle_pins.py`` runs them on the
oracle as it is (all must pass); ``test_oracle_mutations.py`` runs them on
copies of the oracle with a planted mistake (at least one must fail).
"""

import json
import math
import os

import numpy as np

import oracle.attention as oa
import oracle.fp8 as of8
import oracle.metadata as om
from tests import brute_force as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bf16_bits(x):
    """float -> bfloat16 bits, round to nearest even (test-side helper)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


# ----------------------------------------------------------------- metadata

def check_worked_example():
    """ModelRunner page, section 2 figure: bs=4, table [7,2,5], 10 tokens of
    which 4 are cached -> slots 8..11, 20, 21; cu_q [0,6]; cu_k [0,10];
    block tables needed."""
    g = _golden("prefill_worked_example.json")
    seq = {"block_table": g["block_table"], "num_cached": g["num_cached"],
           "num_scheduled": g["num_tokens"] - g["num_cached"]}
    meta = om.prefill_metadata([seq], g["block_size"])
    exp = g["expected"]
    assert meta["slot_mapping"] == exp["slot_mapping"], meta["slot_mapping"]
    assert meta["cu_seqlens_q"] == exp["cu_seqlens_q"]
    assert meta["cu_seqlens_k"] == exp["cu_seqlens_k"]
    assert meta["needs_block_tables"] == exp["needs_block_tables"]
    assert meta["max_seqlen_q"] == 6 and meta["max_seqlen_k"] == 10


def check_no_history_needs_no_tables():
    """ModelRunner page, section 2: with no cached tokens Q and K have the
    same length and no block tables are attached."""
    seqs = [{"block_table": [3, 1], "num_cached": 0, "num_scheduled": 5},
            {"block_table": [0], "num_cached": 0, "num_scheduled": 2}]
    meta = om.prefill_metadata(seqs, 4)
    assert meta["cu_seqlens_q"] == [0, 5, 7]
    assert meta["cu_seqlens_k"] == [0, 5, 7]
    assert not meta["needs_block_tables"]
    assert meta["slot_mapping"] == [12, 13, 14, 15, 4, 0, 1]


def check_allocation_rules():
    """Warmup Guide, Chapter 3: blocks_needed(8, 4) == 2, the 9th token takes
    a third block, a new block iff len % bs == 0, waste <= bs - 1."""
    g = _golden("allocation.json")
    for n, bs, want in g["printed_on_page"]["blocks_needed"]:
        assert om.blocks_needed(n, bs) == want
    for n, bs, want in g["closed_form_ceil_division"]:
        assert om.blocks_needed(n, bs) == want == math.ceil(n / bs)
    free = list(range(100, 110))
    table, length = om.grow_block_table([], 0, 8, free, 4)
    assert len(table) == 2 and length == 8
    table, length = om.grow_block_table(table, length, 1, free, 4)
    assert len(table) == 3, "the 9th token must take a third block"
    # token numbers (1-based) that took a new block, appending one at a time
    took = []
    table, length = [], 0
    free = list(range(50))
    for token in range(1, 17):
        before = len(table)
        table, length = om.grow_block_table(table, length, 1, free, 4)
        if len(table) > before:
            took.append(token)
    assert took == [1, 5, 9, 13], took
    for n in range(0, 200):
        for bs in (1, 2, 4, 16):
            assert 0 <= om.internal_waste(n, bs) <= bs - 1


def check_prefix_sharing_example():
    """Warmup Guide, Chapter 4 figure: a prompt in blocks [P0][P1] shared by
    requests A, B, C (ref count 3); each continuation goes to a private
    block; the prefix is stored once (5 physical blocks, no copies)."""
    g = _golden("prefix_sharing.json")
    bs = g["block_size"]
    pool = om.RefCountedPool(range(32))
    prompt, length = [], 0
    for _ in range(g["prompt_tokens"]):
        prompt, length, _, copy = pool.append(prompt, length, bs)
        assert copy is None
    tables = {"A": prompt}
    for name in g["requests"][1:]:
        tables[name] = pool.share(prompt)
    copies = 0
    for name in g["requests"]:
        tables[name], _, slot, copy = pool.append(tables[name], length, bs)
        copies += copy is not None
        assert slot == tables[name][-1] * bs, (name, slot)
    exp = g["expected"]
    for blk in prompt:
        assert pool.ref[blk] == exp["prefix_ref_count"], pool.ref
    lasts = [tables[n][-1] for n in g["requests"]]
    assert len(set(lasts)) == len(lasts)
    for blk in lasts:
        assert pool.ref[blk] == exp["continuation_ref_count"]
    for name in g["requests"]:
        assert tables[name][:exp["tables_share_first_blocks"]] == prompt
    used = {b for t in tables.values() for b in t}
    assert len(used) == exp["physical_blocks_used"], used
    assert copies == exp["copies"]


def check_shared_prefix_groups():
    """Sharing groups for the read-once decode (Warmup Guide, Chapter 4):
    the figure's three requests form one group whose shared length is the
    two prompt blocks; by hand from the rule: only full blocks count, a
    group keeps the first pair's shared length, a shorter share starts a
    new group, and a sequence sharing nothing stays alone."""
    g = _golden("prefix_sharing.json")
    bs = g["block_size"]
    nshared = g["expected"]["tables_share_first_blocks"]
    prompt = list(range(nshared))
    seqs = [{"block_table": prompt + [10 + i], "length": g["prompt_tokens"] + 1 + i}
            for i in range(len(g["requests"]))]
    lens, groups = om.shared_prefix_groups(seqs, bs)
    assert groups == [(0, len(g["requests"]))], groups
    assert lens == [nshared * bs] * len(g["requests"]), lens

    def run(tables, lengths, b=4):
        return om.shared_prefix_groups(
            [{"block_table": t, "length": n} for t, n in zip(tables, lengths)], b)

    # equal ids past the shorter sequence's full blocks do not count
    assert run([[1, 2, 3], [1, 2, 4], [5, 6]], [12, 10, 8]) == \
        ([8, 8, 0], [(0, 2)])
    # a partially filled last block is never shared, even with equal ids
    assert run([[1, 2], [1, 2]], [6, 7]) == ([4, 4], [(0, 2)])
    # the group keeps the first pair's 3 blocks; a 2-block share starts anew
    assert run([[1, 2, 3], [1, 2, 3], [1, 2, 9], [1, 7, 8]], [12, 12, 12, 12]) == \
        ([12, 12, 4, 4], [(0, 2), (2, 2)])
    # nothing shared
    assert run([[1], [2], [3]], [4, 4, 4]) == ([0, 0, 0], [])
    # a single sequence never forms a group
    assert run([[1, 2]], [8]) == ([0], [])


def check_e4m3_codes_against_library():
    """E4M3 values of all 256 codes equal torch's float8_e4m3fn decoding
    (an independent implementation of the OCP format)."""
    import torch
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    mine = np.array([of8.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(lib), np.isnan(mine))
    ok = ~np.isnan(lib)
    assert np.array_equal(lib[ok], mine[ok])


def check_e4m3_encode_against_library():
    """Encoding equals torch's round-to-nearest-even float32 -> e4m3fn cast
    of the value saturated to +-448, over normals, subnormals, exact ties
    (midpoints between neighbouring codes) and out-of-range values."""
    import torch
    rng = np.random.default_rng(21)
    vals = np.array([of8.e4m3_value(c) for c in range(256)])
    vals = vals[np.isfinite(vals)]
    srt = np.unique(vals)
    mids = (srt[1:] + srt[:-1]) / 2
    x = np.concatenate([
        rng.normal(size=4000) * rng.choice([1e-3, 0.05, 1, 30, 400], 4000),
        mids, vals, [600.0, -1e30, 449.0, 464.0, 500.0, -0.0, 0.0]]).astype(np.float32)
    mine = of8.quantize(x, 1.0)
    lib = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    assert np.array_equal(mine, lib), np.nonzero(mine != lib)[0][:10]


def check_e4m3_hand_values():
    """Values worked out by hand from the format: 1 = 0x38, 448 = 0x7E (the
    largest finite), larger values saturate to it, -0 keeps its sign,
    2^-9 is the smallest subnormal; halfway cases go to the even mantissa
    (2^-10 -> 0, 3 * 2^-10 -> 2 steps, 1 + 1/16 -> 1, 1 + 3/16 -> 1.25);
    1.125 * 2^-4 = 0x19; the scale divides before rounding."""
    enc = of8.e4m3_encode
    assert enc(1.0) == 0x38 and enc(448.0) == 0x7E and enc(1e6) == 0x7E
    assert enc(-1e6) == 0xFE and enc(-0.0) == 0x80 and enc(0.0) == 0x00
    assert enc(2.0 ** -9) == 0x01 and enc(2.0 ** -10) == 0x00
    assert enc(3 * 2.0 ** -10) == 0x02
    assert enc(1 + 1 / 16) == 0x38 and enc(1 + 3 / 16) == 0x3A
    assert enc(1.125 * 2.0 ** -4) == 0x19
    assert of8.quantize(np.float32([3.0]), 0.5)[0] == enc(1.5)
    assert of8.e4m3_value(0x7E) == 448.0 and math.isnan(of8.e4m3_value(0xFF))


def check_fp8_dequantize_closed_form():
    """code * scale for codes whose values the E4M3 definition fixes (bias
    7, subnormals m/8 * 2^-6): 0x38 = 1, 0x40 = 2, 0xB8 = -1, 0x01 = 2^-9,
    0x7E = 448; with scale 0.25."""
    got = of8.dequantize(np.array([0x38, 0x40, 0xB8, 0x01, 0x7E]), 0.25)
    want = np.array([0.25, 0.5, -0.25, 2.0 ** -11, 112.0])
    assert np.array_equal(got, want), got


def check_fp8_decode_equals_dequantized():
    """Decode over an E4M3 cache equals plain decode over float32 caches
    holding code * scale (exact in float32), for random codes and scales."""
    rng = np.random.default_rng(23)
    nb, bs, hkv, d, hq = 6, 4, 2, 8, 4
    kc = rng.integers(0, 256, size=(nb, bs, hkv, d)).astype(np.uint8)
    vc = rng.integers(0, 256, size=(nb, bs, hkv, d)).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x10            # no NaN codes
    vc[(vc & 0x7F) == 0x7F] = 0x21
    q = rng.normal(size=(3, hq, d)).astype(np.float32)
    tables = [[0, 3], [5, 1, 2], [4]]
    lens = [7, 10, 3]
    bt = np.full((3, 3), -1)
    for i, t in enumerate(tables):
        bt[i, :len(t)] = t
    ks, vs = 0.0625, 0.015625
    got = of8.decode_attention(q, kc, vc, bt, lens, 0.3, ks, vs, "f32")
    kf = of8.dequantize(kc, ks).astype(np.float32)
    vf = of8.dequantize(vc, vs).astype(np.float32)
    want = oa.decode_attention(q, kf, vf, bt, lens, 0.3, "f32")
    assert np.max(np.abs(got - want)) < 1e-12


def check_copy_on_write_partial_block():
    """Warmup Guide, Chapter 4: appending into a partially filled block that
    another sequence also holds copies that one block first, lowers its ref
    count and writes into the private copy; the last holder then writes in
    place; a released sequence's unshared blocks return to the pool."""
    bs = 4
    pool = om.RefCountedPool(range(8))
    a, length = [], 0
    for _ in range(6):                    # 6 tokens: P0 full, P1 holds 2
        a, length, _, copy = pool.append(a, length, bs)
        assert copy is None
    p0, p1 = a
    b = pool.share(a)
    assert pool.ref[p0] == 2 and pool.ref[p1] == 2
    a, la, slot_a, copy_a = pool.append(a, length, bs)
    assert copy_a is not None and copy_a[0] == p1 and copy_a[1] not in (p0, p1)
    assert a == [p0, copy_a[1]] and slot_a == copy_a[1] * bs + 2
    assert pool.ref[p1] == 1 and pool.ref[copy_a[1]] == 1
    b, lb, slot_b, copy_b = pool.append(b, length, bs)
    assert copy_b is None and b == [p0, p1] and slot_b == p1 * bs + 2
    assert la == lb == 7
    free_before = len(pool.free)
    pool.release(a)
    assert pool.ref[p0] == 1 and copy_a[1] in pool.free
    assert len(pool.free) == free_before + 1


def check_copy_blocks_against_brute():
    """Block copy, element by element: each destination block of both caches
    equals its source block; pairs with an id outside the pool and all other
    blocks are left alone."""
    rng = np.random.default_rng(11)
    kc = rng.integers(0, 2**16, size=(9, 4, 2, 8), dtype=np.uint16)
    vc = rng.integers(0, 2**16, size=(9, 4, 2, 8), dtype=np.uint16)
    pairs = [(1, 5), (7, 2), (-1, 3), (4, 9), (0, 8)]
    ko, vo = oa.copy_blocks(kc, vc, pairs)
    dst_of = {5: 1, 2: 7, 8: 0}
    for blk in range(9):
        src = dst_of.get(blk, blk)
        for s in range(4):
            for h in range(2):
                for d in range(8):
                    assert ko[blk, s, h, d] == kc[src, s, h, d]
                    assert vo[blk, s, h, d] == vc[src, s, h, d]


def check_decode_slot_closed_form():
    """ModelRunner page, section 2 (prepare_decode): the new token's slot is
    last_block * bs + last_block_num_tokens - 1.  For tables built by the
    append rule this equals table[(L-1)//bs]*bs + (L-1)%bs, the prefill rule
    of the same section applied to position L-1."""
    rng = np.random.default_rng(11)
    for bs in (1, 4, 16):
        for _ in range(50):
            length = int(rng.integers(1, 300))
            free = [int(x) for x in rng.permutation(1000)]
            table, n = om.grow_block_table([], 0, length, free, bs)
            assert n == length
            meta = om.decode_metadata([{"block_table": table,
                                        "length": length}], bs)
            pos = length - 1
            want = table[pos // bs] * bs + pos % bs
            assert meta["slot_mapping"] == [want]
            assert meta["context_lens"] == [length]
    # the worked-example sequence decoding its 11th token: block 5, 3rd slot
    meta = om.decode_metadata([{"block_table": [7, 2, 5], "length": 11}], 4)
    assert meta["slot_mapping"] == [22]


def check_decode_padding():
    """ModelRunner page, sections 2 and 5: block tables right-padded with -1;
    a batch of 37 replayed in bucket 48 gets 11 rows of slot -1 and context
    length 0."""
    seqs = [{"block_table": list(range(i + 1)), "length": 4 * i + 1}
            for i in range(37)]
    meta = om.decode_metadata(seqs, 4)
    assert all(len(r) == 37 for r in meta["block_tables"])
    assert meta["block_tables"][0] == [0] + [-1] * 36
    padded = om.pad_decode_batch(meta, 48)
    assert padded["slot_mapping"][37:] == [-1] * 11
    assert padded["context_lens"][37:] == [0] * 11
    assert padded["slot_mapping"][:37] == meta["slot_mapping"]


def check_kv_bytes():
    """ModelRunner page, section 4 (Qwen3-0.6B block bytes) and "10 Serving
    Engines", section 10.2.3 (Llama 3 8B bytes per token)."""
    g = _golden("kv_bytes.json")
    q = g["qwen3_0_6b_block"]
    b = om.kv_block_bytes(q["num_layers"], q["block_size"], q["num_kv_heads"],
                          q["head_dim"], q["itemsize"], q["tensor_parallel"])
    assert b == q["block_bytes"]
    assert b == q["block_mib"] * 2 ** 20
    assert b // q["block_size"] == q["token_kib"] * 1024
    assert 2 ** 30 // b == q["blocks_per_gib"]
    assert abs(q["blocks_per_gib"] * q["block_size"]
               - q["tokens_per_gib_approx"]) < 100
    assert om.kv_bytes_per_token(q["num_layers"], q["num_kv_heads"],
                                 q["head_dim"], q["itemsize"]) == 114688
    l3 = g["llama3_8b_token"]
    per_tok = om.kv_bytes_per_token(l3["num_layers"], l3["num_kv_heads"],
                                    l3["head_dim"], l3["itemsize"])
    assert per_tok == l3["bytes_per_token"]
    payload = l3["requests"] * l3["tokens_per_request"] * per_tok
    assert round(payload / 1e9, 1) == l3["payload_gb_approx"]


# ------------------------------------------------------------------- values

def check_bf16_widening():
    """bfloat16 is the top 16 bits of a float32: known patterns."""
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x3F81, 0x7F80, 0x0001],
                    dtype=np.uint16)
    got = oa.bf16_bits_to_f64(bits)
    assert got[0] == 1.0 and got[1] == -2.0 and got[2] == 0.0
    assert got[3] == 1.0 + 2.0 ** -7
    assert math.isinf(got[4])
    assert got[5] == 2.0 ** -133


def _e4m3_values_from_library():
    """Values of the non-negative finite E4M3 codes 0..126, decoded by
    torch's float8_e4m3fn (an implementation of the OCP format independent
    of the oracle)."""
    import torch
    return torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn) \
        .to(torch.float64).tolist()


def check_fp8_store_against_brute():
    """The quantising store equals an element-by-element brute force (float32
    product, nearest code by exhaustive search over the library's code
    values, ties to the even code, saturation at 448) for bf16 and float32
    rows, with different K and V scales (not powers of two, so the float32
    product rounds), slots in random order, two -1 slots that must write
    nothing ("3.6 ModelRunner, CUDA Graph, and benchmarks", section 5) and
    a gain that pushes some elements far past 448.  A slot past the cache
    raises.  Sources: the cache-precision flag of "10 Serving Engines"
    section 10.2.2 (format readings in oracle/fp8.py)."""
    values = _e4m3_values_from_library()
    rng = np.random.default_rng(29)
    nb, bs, hkv, d, t = 5, 4, 2, 8, 9
    k_inv = float(np.float32(1.0) / np.float32(0.07))
    v_inv = float(np.float32(1.0) / np.float32(0.3))
    assert k_inv != v_inv
    for src in ("f32", "bf16"):
        kc = rng.integers(0, 256, size=(nb, bs, hkv, d)).astype(np.uint8)
        vc = rng.integers(0, 256, size=(nb, bs, hkv, d)).astype(np.uint8)
        k = (rng.standard_normal((t, hkv, d)) *
             rng.choice([0.01, 1.0, 8.0, 60.0], size=(t, hkv, 1))).astype(np.float32)
        v = (rng.standard_normal((t, hkv, d)) *
             rng.choice([0.01, 1.0, 8.0, 200.0], size=(t, hkv, 1))).astype(np.float32)
        k[0, 0, :3] = [0.0, -0.0, 1e-9]
        if src == "bf16":
            k, v = _bf16_bits(k), _bf16_bits(v)
        k32 = oa.to_f64(k, src)
        v32 = oa.to_f64(v, src)
        assert np.max(np.abs(k32)) * k_inv > 448 and np.max(np.abs(v32)) * v_inv > 448
        slots = [int(s) for s in rng.permutation(nb * bs)[:t]]
        slots[1] = -1
        slots[6] = -1
        nk, nv = of8.store_kv(kc, vc, k, v, slots, k_inv, v_inv, src)
        bk, bv = bf.brute_store_fp8(kc.tolist(), vc.tolist(), k32.tolist(),
                                    v32.tolist(), slots, k_inv, v_inv,
                                    values, 448.0)
        assert nk.tolist() == bk, "K codes differ from the brute force"
        assert nv.tolist() == bv, "V codes differ from the brute force"
        # the -1 rows left every slot they might have named untouched
        named = {s for s in slots if s >= 0}
        for s in range(nb * bs):
            if s not in named:
                assert nk[s // bs, s % bs].tobytes() == kc[s // bs, s % bs].tobytes()
                assert nv[s // bs, s % bs].tobytes() == vc[s // bs, s % bs].tobytes()
    try:
        of8.store_kv(kc, vc, k[:1], v[:1], [nb * bs], k_inv, v_inv, "bf16")
    except IndexError:
        pass
    else:
        raise AssertionError("a slot past the cache must raise")


# -------------------------------------------------------------------- store

def _tiny_pool(rng, nb, bs, hkv, d, dtype):
    k = rng.standard_normal((nb, bs, hkv, d)).astype(np.float32)
    v = rng.standard_normal((nb, bs, hkv, d)).astype(np.float32)
    if dtype == "bf16":
        return _bf16_bits(k), _bf16_bits(v)
    return k, v


def check_store_against_brute():
    """The scatter equals an element-by-element brute force; slot -1 writes
    nothing (ModelRunner page, section 5); untouched slots keep their bytes."""
    rng = np.random.default_rng(5)
    for dtype in ("f32", "bf16"):
        nb, bs, hkv, d = 6, 4, 2, 8
        kc, vc = _tiny_pool(rng, nb, bs, hkv, d, dtype)
        t = 7
        k, v = _tiny_pool(rng, 1, t, hkv, d, dtype)
        k, v = k[0], v[0]
        slots = [int(s) for s in rng.permutation(nb * bs)[:t]]
        slots[2] = -1
        slots[5] = -1
        nk, nv = oa.store_kv(kc, vc, k, v, slots)
        bk, bv = bf.brute_store(kc.tolist(), vc.tolist(), k.tolist(),
                                v.tolist(), slots)
        assert nk.tolist() == bk and nv.tolist() == bv
        assert nk.tobytes() != kc.tobytes()
        # slots never named keep their exact bytes (incl. the last slot,
        # which a wrapped negative index would hit)
        flat_old = kc.reshape(nb * bs, -1)
        flat_new = nk.reshape(nb * bs, -1)
        named = {s for s in slots if s >= 0}
        for s in range(nb * bs):
            if s not in named:
                assert flat_old[s].tobytes() == flat_new[s].tobytes()


# ---------------------------------------------------------------- attention

def _paged_from_contiguous(rng, keys, values, bs, nb, dtype):
    """Scatter contiguous per-sequence K/V [L, Hkv, D] into a pool through a
    random table (test-side scatter, written independently of the oracle).
    Unused slots hold NaN so that reading them shows."""
    length, hkv, d = keys.shape
    nblk = -(-length // bs)
    table = [int(x) for x in rng.permutation(nb)[:nblk]]
    if dtype == "bf16":
        nan_bits = np.uint16(0x7FC0)
        kc = np.full((nb, bs, hkv, d), nan_bits, dtype=np.uint16)
    else:
        kc = np.full((nb, bs, hkv, d), np.nan, dtype=np.float32)
    vc = kc.copy()
    for t in range(length):
        kc[table[t // bs], t % bs] = keys[t]
        vc[table[t // bs], t % bs] = values[t]
    return kc, vc, table


def _softmax_direct(q, keys, values, scale):
    s = [scale * sum(a * b for a, b in zip(q, k)) for k in keys]
    top = max(s)
    w = [math.exp(x - top) for x in s]
    tot = sum(w)
    return [sum(wi * v[j] for wi, v in zip(w, values)) / tot
            for j in range(len(values[0]))]


def check_decode_against_brute(cases=None):
    """numpy oracle == pure-Python brute force to 1e-12 on tiny shapes, with
    -1 / stale padding and a zero-length row."""
    rng = np.random.default_rng(7)
    cases = cases or [
        dict(bs=1, hq=2, hkv=1, d=8, lens=[1, 3, 5], dtype="f32"),
        dict(bs=2, hq=4, hkv=2, d=8, lens=[2, 7, 0], dtype="bf16"),
        dict(bs=4, hq=4, hkv=1, d=8, lens=[9, 4, 13], dtype="f32"),
        dict(bs=16, hq=8, hkv=2, d=8, lens=[17, 33, 1], dtype="bf16"),
    ]
    for c in cases:
        bs, hq, hkv, d = c["bs"], c["hq"], c["hkv"], c["d"]
        lens = c["lens"]
        need = sum(-(-n // bs) for n in lens)
        nb = need + 3
        kc, vc = _tiny_pool(rng, nb, bs, hkv, d, c["dtype"])
        perm = [int(x) for x in rng.permutation(nb)]
        width = max(-(-n // bs) for n in lens) + 2
        tables, pos = [], 0
        for n in lens:
            k = -(-n // bs)
            row = perm[pos:pos + k]
            pos += k
            # padding: -1 then a stale (valid-looking) id
            row = row + [-1] * (width - k - 1) + [perm[-1]]
            tables.append(row)
        q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
        if c["dtype"] == "bf16":
            q = _bf16_bits(q)
        scale = 1.0 / math.sqrt(d)
        got, probs = oa.decode_attention(q, kc, vc, tables, lens, scale,
                                         c["dtype"], return_probs=True)
        q64 = oa.to_f64(q, c["dtype"])
        kc64 = oa.to_f64(kc, c["dtype"]).tolist()
        vc64 = oa.to_f64(vc, c["dtype"]).tolist()
        want = bf.brute_decode(q64.tolist(), kc64, vc64, tables, lens, scale)
        assert np.max(np.abs(got - np.array(want))) < 1e-12, c
        for b, n in enumerate(lens):
            if n == 0:
                assert np.all(got[b] == 0.0)
            else:
                assert np.allclose(probs[b].sum(axis=1), 1.0, atol=1e-12)


def check_prefill_against_brute():
    """Varlen prefill oracle == brute force, causal and not, with an empty
    chunk, a no-history sequence and chunked resumes."""
    rng = np.random.default_rng(8)
    bs, hq, hkv, d = 4, 4, 2, 8
    lq = [3, 0, 5, 1]
    lk = [3, 6, 12, 9]
    need = sum(-(-n // bs) for n in lk)
    nb = need + 2
    for dtype in ("f32", "bf16"):
        kc, vc = _tiny_pool(rng, nb, bs, hkv, d, dtype)
        perm = [int(x) for x in rng.permutation(nb)]
        width = max(-(-n // bs) for n in lk)
        tables, pos = [], 0
        for n in lk:
            k = -(-n // bs)
            tables.append(perm[pos:pos + k] + [-1] * (width - k))
            pos += k
        cu_q = [0]
        cu_k = [0]
        for a, b in zip(lq, lk):
            cu_q.append(cu_q[-1] + a)
            cu_k.append(cu_k[-1] + b)
        q = rng.standard_normal((cu_q[-1], hq, d)).astype(np.float32)
        if dtype == "bf16":
            q = _bf16_bits(q)
        scale = 0.3
        q64 = oa.to_f64(q, dtype)
        kc64 = oa.to_f64(kc, dtype).tolist()
        vc64 = oa.to_f64(vc, dtype).tolist()
        for causal in (True, False):
            got = oa.prefill_attention(q, kc, vc, cu_q, cu_k, tables, scale,
                                       causal, dtype)
            want = bf.brute_prefill(q64.tolist(), kc64, vc64, cu_q, cu_k,
                                    tables, scale, causal)
            assert np.max(np.abs(got - np.array(want))) < 1e-12, causal


def check_one_key_returns_v():
    """A one-key context returns V exactly: its only weight is e^0/e^0 = 1."""
    rng = np.random.default_rng(3)
    for dtype in ("f32", "bf16"):
        kc, vc = _tiny_pool(rng, 4, 4, 2, 8, dtype)
        q = rng.standard_normal((1, 4, 8)).astype(np.float32)
        if dtype == "bf16":
            q = _bf16_bits(q)
        out = oa.decode_attention(q, kc, vc, [[2]], [1], 0.7, dtype)
        v0 = oa.to_f64(vc[2, 0], dtype)
        for h in range(4):
            assert np.array_equal(out[0, h], v0[h // 2])


def check_uniform_weights_give_mean():
    """q = 0, or all keys equal, makes every weight 1/L: the output is the
    mean of V over the context."""
    rng = np.random.default_rng(4)
    bs, hkv, d, length = 4, 1, 8, 11
    values = rng.standard_normal((length, hkv, d))
    keys = rng.standard_normal((length, hkv, d))
    same = np.repeat(keys[:1], length, axis=0)
    for q_scale, ks in ((0.0, keys), (1.0, same)):
        kc, vc, table = _paged_from_contiguous(rng, ks.astype(np.float32),
                                               values.astype(np.float32),
                                               bs, 8, "f32")
        q = (q_scale * rng.standard_normal((1, 2, d))).astype(np.float32)
        out = oa.decode_attention(q, kc, vc, [table], [length], 0.5, "f32")
        mean = values.astype(np.float32).astype(np.float64).mean(axis=0)[0]
        for h in range(2):
            assert np.max(np.abs(out[0, h] - mean)) < 1e-12


def check_two_key_logistic():
    """Two keys with q.k0 = a, q.k1 = b: weight of key 1 is
    1 / (1 + exp(scale * (a - b))) -- pins where the scale goes."""
    d = 4
    q = np.array([[[1.0, 0.0, 0.0, 0.0]]], dtype=np.float32)
    kc = np.zeros((1, 2, 1, d), dtype=np.float32)
    vc = np.zeros((1, 2, 1, d), dtype=np.float32)
    kc[0, 0, 0, 0] = 2.0     # a = 2
    kc[0, 1, 0, 0] = -1.0    # b = -1
    vc[0, 0, 0] = [1.0, 0.0, 0.0, 0.0]
    vc[0, 1, 0] = [0.0, 1.0, 0.0, 0.0]
    for scale in (0.25, 1.0, 3.0):
        out = oa.decode_attention(q, kc, vc, [[0]], [2], scale, "f32")
        w1 = 1.0 / (1.0 + math.exp(scale * 3.0))
        assert abs(out[0, 0, 1] - w1) < 1e-14
        assert abs(out[0, 0, 0] - (1.0 - w1)) < 1e-14


def check_large_logits_pick_argmax():
    """scale * |logit| >> 1 with a unique maximum: the output is V at the
    argmax (a max-subtracted softmax stays finite)."""
    rng = np.random.default_rng(9)
    length, d = 9, 8
    keys = rng.standard_normal((length, 1, d))
    values = rng.standard_normal((length, 1, d))
    q = rng.standard_normal((1, 1, d))
    kc, vc, table = _paged_from_contiguous(rng, keys.astype(np.float32),
                                           values.astype(np.float32), 4, 5,
                                           "f32")
    out = oa.decode_attention(q.astype(np.float32), kc, vc, [table], [length],
                              1e4, "f32")
    best = int(np.argmax(keys[:, 0].astype(np.float32).astype(np.float64)
                         @ q[0, 0].astype(np.float32).astype(np.float64)))
    assert np.all(np.isfinite(out))
    assert np.max(np.abs(out[0, 0] - values[best, 0].astype(np.float32))) < 1e-9


def check_paged_equals_contiguous():
    """Scattering a sequence's tokens over random physical blocks changes
    nothing: compare with softmax computed directly on the contiguous arrays
    (Warmup Guide, Chapter 3: order is logical, not physical)."""
    rng = np.random.default_rng(10)
    for bs in (1, 4, 16):
        length, hkv, hq, d = 37, 2, 4, 8
        keys = rng.standard_normal((length, hkv, d)).astype(np.float32)
        values = rng.standard_normal((length, hkv, d)).astype(np.float32)
        q = rng.standard_normal((1, hq, d)).astype(np.float32)
        nb = -(-length // bs) + 5
        kc, vc, table = _paged_from_contiguous(rng, keys, values, bs, nb,
                                               "f32")
        out = oa.decode_attention(q, kc, vc, [table], [length], 0.4, "f32")
        for h in range(hq):
            g = h // (hq // hkv)
            want = _softmax_direct(q[0, h].astype(np.float64).tolist(),
                                   keys[:, g].astype(np.float64).tolist(),
                                   values[:, g].astype(np.float64).tolist(),
                                   0.4)
            assert np.max(np.abs(out[0, h] - np.array(want))) < 1e-12


def check_chunked_equals_unchunked():
    """"10 Serving Engines", section 10.3: chunking changes when prompt work
    runs, not the attention it computes -- a prompt prefilled in one causal
    pass equals the same prompt prefilled in chunks over its own history."""
    rng = np.random.default_rng(12)
    bs, hq, hkv, d, length = 4, 4, 2, 8, 23
    keys = rng.standard_normal((length, hkv, d)).astype(np.float32)
    values = rng.standard_normal((length, hkv, d)).astype(np.float32)
    kc, vc, table = _paged_from_contiguous(rng, keys, values, bs, 9, "f32")
    q = rng.standard_normal((length, hq, d)).astype(np.float32)
    whole = oa.prefill_attention(q, kc, vc, [0, length], [0, length],
                                 [table], 0.35, True, "f32")
    cuts = [0, 5, 6, 14, 23]
    for a, b in zip(cuts[:-1], cuts[1:]):
        part = oa.prefill_attention(q[a:b], kc, vc, [0, b - a], [0, b],
                                    [table], 0.35, True, "f32")
        assert np.max(np.abs(part - whole[a:b])) < 1e-12


def check_decode_equals_last_prefill_row():
    """A decode row at context L equals the last row of a causal prefill over
    the same L tokens, whatever the chunk length."""
    rng = np.random.default_rng(13)
    bs, hq, hkv, d, length = 4, 8, 2, 8, 19
    keys = rng.standard_normal((length, hkv, d)).astype(np.float32)
    values = rng.standard_normal((length, hkv, d)).astype(np.float32)
    kc, vc, table = _paged_from_contiguous(rng, keys, values, bs, 8, "f32")
    qrows = rng.standard_normal((length, hq, d)).astype(np.float32)
    dec = oa.decode_attention(qrows[-1:], kc, vc, [table], [length], 0.5,
                              "f32")
    for lq in (1, 3, length):
        pre = oa.prefill_attention(qrows[length - lq:], kc, vc, [0, lq],
                                   [0, length], [table], 0.5, True, "f32")
        assert np.max(np.abs(pre[-1] - dec[0])) < 1e-12


def check_gqa_equals_repeated_mha():
    """GQA with G = Hq/Hkv equals MHA whose KV heads are repeated G times in
    contiguous groups (reading: query head h uses KV head h // G)."""
    rng = np.random.default_rng(14)
    bs, hq, hkv, d, length = 4, 8, 2, 8, 13
    g = hq // hkv
    keys = rng.standard_normal((length, hkv, d)).astype(np.float32)
    values = rng.standard_normal((length, hkv, d)).astype(np.float32)
    kc, vc, table = _paged_from_contiguous(rng, keys, values, bs, 6, "f32")
    kr = np.repeat(keys, g, axis=1)
    vr = np.repeat(values, g, axis=1)
    kc2, vc2, table2 = _paged_from_contiguous(rng, kr, vr, bs, 6, "f32")
    q = rng.standard_normal((1, hq, d)).astype(np.float32)
    a = oa.decode_attention(q, kc, vc, [table], [length], 0.5, "f32")
    b = oa.decode_attention(q, kc2, vc2, [table2], [length], 0.5, "f32")
    assert np.max(np.abs(a - b)) < 1e-12


ALL_CHECKS = [
    check_worked_example,
    check_no_history_needs_no_tables,
    check_allocation_rules,
    check_decode_slot_closed_form,
    check_decode_padding,
    check_prefix_sharing_example,
    check_shared_prefix_groups,
    check_copy_on_write_partial_block,
    check_e4m3_codes_against_library,
    check_e4m3_encode_against_library,
    check_e4m3_hand_values,
    check_fp8_dequantize_closed_form,
    check_fp8_decode_equals_dequantized,
    check_fp8_store_against_brute,
    check_copy_blocks_against_brute,
    check_kv_bytes,
    check_bf16_widening,
    check_store_against_brute,
    check_decode_against_brute,
    check_prefill_against_brute,
    check_one_key_returns_v,
    check_uniform_weights_give_mean,
    check_two_key_logistic,
    check_large_logits_pick_argmax,
    check_paged_equals_contiguous,
    check_chunked_equals_unchunked,
    check_decode_equals_last_prefill_row,
    check_gqa_equals_repeated_mha,
]
