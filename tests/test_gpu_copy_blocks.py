"""pa_copy_blocks on the GPU against the oracle, and a fork followed by a
copy-on-write decode step through the whole path (block copy, store,
decode)."""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oa
import oracle.metadata as om
import workloads as wl
from paged_kv_cache_slot_amd import metadata as pm
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import TOL, bits_equal, dev_i32, f64, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_copy_blocks_bit_exact(dtype):
    """Disjoint random (source, destination) pairs plus pairs the call must
    skip (ids outside the pool, source == destination): the caches after the
    call equal the oracle's block copy byte for byte."""
    nb, bs, hkv, d = 3000, 16, 8, 128
    say("copy_blocks bit-exact", dtype)
    kc, vc = wl.fill_pool(nb, bs, hkv, d, dtype, 61, "cuda")
    h_kc, h_vc = wl.host_bits(kc), wl.host_bits(vc)
    rng = np.random.default_rng(62)
    ids = rng.permutation(nb)
    pairs = [(int(s), int(t)) for s, t in zip(ids[:400], ids[400:800])]
    pairs += [(-1, int(ids[900])), (int(ids[901]), nb), (int(ids[902]), int(ids[902])),
              (nb + 5, -3)]
    ops.copy_blocks(kc, vc, dev_i32(pairs))
    torch.cuda.synchronize()
    ek, ev = oa.copy_blocks(h_kc, h_vc, pairs)
    assert bits_equal(wl.host_bits(kc), ek)
    assert bits_equal(wl.host_bits(vc), ev)


def test_copy_blocks_single_pair_and_empty():
    """One pair on a tiny pool, then an empty list (no-op)."""
    say("copy_blocks single / empty")
    kc, vc = wl.fill_pool(4, 16, 2, 64, "f32", 63, "cuda")
    h_kc, h_vc = wl.host_bits(kc), wl.host_bits(vc)
    ops.copy_blocks(kc, vc, dev_i32([[3, 0]]))
    ops.copy_blocks(kc, vc, torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    ek, ev = oa.copy_blocks(h_kc, h_vc, [(3, 0)])
    assert bits_equal(wl.host_bits(kc), ek) and bits_equal(wl.host_bits(vc), ev)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fork_then_copy_on_write_decode(dtype):
    """Parents of various lengths (partial and exactly full last blocks) are
    forked; one decode step then appends a different token to every parent
    and every child.  A shared partial last block is copied for the first
    writer; the last holder writes in place; shared full blocks are never
    written.  Block tables, slots and copies from the product pool equal the
    oracle pool's; caches and outputs match the oracle."""
    bs, hkv, hq, d = 16, 2, 8, 64
    lens = [7, 16, 33, 100, 47, 64]
    say("fork + copy-on-write decode", dtype)
    nb = 128
    pool = pm.BlockPool(nb)
    ref = om.RefCountedPool(range(nb))
    parents, ref_parents = [], []
    for n in lens:                       # grow each parent to its length
        t, r = [], []
        for pos in range(n):
            pool.append_slots([t], [pos], bs)
            r, _, _, _ = ref.append(r, pos, bs)
        parents.append(t)
        ref_parents.append(r)
    children = [pool.share(t) for t in parents]
    ref_children = [ref.share(r) for r in ref_parents]
    tables = parents + children
    ref_tables = ref_parents + ref_children
    before = [list(t) for t in tables]
    slots, pairs = pool.append_slots(tables, lens + lens, bs)
    want_slots, want_pairs = [], []
    for i, n in enumerate(lens + lens):
        ref_tables[i], _, slot, copy = ref.append(ref_tables[i], n, bs)
        want_slots.append(slot)
        if copy is not None:
            want_pairs.append(copy)
    assert slots.tolist() == want_slots
    assert [tuple(p) for p in pairs.tolist()] == want_pairs
    assert [list(t) for t in tables] == [list(t) for t in ref_tables]
    n_partial = sum(1 for n in lens if n % bs)
    assert len(want_pairs) == n_partial      # one copy per shared partial block

    b = len(tables)
    kc, vc = wl.fill_pool(nb, bs, hkv, d, dtype, 64, "cuda")
    q = wl.make_values((b, hq, d), dtype, 65, "cuda")
    k_new = wl.make_values((b, hkv, d), dtype, 66, "cuda")
    v_new = wl.make_values((b, hkv, d), dtype, 67, "cuda")
    h_kc, h_vc = wl.host_bits(kc), wl.host_bits(vc)
    h_q, h_kn, h_vn = (wl.host_bits(x) for x in (q, k_new, v_new))

    new_lens = np.asarray(lens + lens) + 1
    meta = pm.decode_inputs(tables, new_lens, bs)
    assert meta["slot_mapping"].tolist() == want_slots
    ops.copy_blocks(kc, vc, dev_i32(pairs))
    ops.store_kv(k_new, v_new, kc, vc, dev_i32(meta["slot_mapping"]))
    out = ops.decode(q, kc, vc, dev_i32(meta["block_tables"]),
                     dev_i32(meta["context_lens"]), meta["max_context_len"])
    torch.cuda.synchronize()

    ek, ev = oa.copy_blocks(h_kc, h_vc, want_pairs)
    ek, ev = oa.store_kv(ek, ev, h_kn, h_vn, want_slots)
    assert bits_equal(wl.host_bits(kc), ek) and bits_equal(wl.host_bits(vc), ev)
    # blocks every table still shares were never written
    shared = {blk for t in before for blk in t[:-1]}
    for blk in shared:
        assert bits_equal(ek[blk], h_kc[blk]) and bits_equal(ev[blk], h_vc[blk])
    om_meta = om.decode_metadata(
        [{"block_table": t, "length": int(n)} for t, n in zip(ref_tables, new_lens)],
        bs)
    want = oa.decode_attention(h_q, ek, ev, om_meta["block_tables"],
                               om_meta["context_lens"], 1 / math.sqrt(d), dtype)
    err = float(np.max(np.abs(f64(out) - want)))
    assert err <= TOL[dtype], err
    # parent and child differ only in their last token: different outputs
    assert not np.array_equal(f64(out)[: len(lens)], f64(out)[len(lens):])
