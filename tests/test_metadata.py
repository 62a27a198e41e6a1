"""The package's vectorised metadata builder equals the oracle's loop
version, bit for bit, on random batches and on the pages' worked example."""

import numpy as np
import pytest

import oracle.metadata as om
from paged_kv_cache_slot_amd import metadata as pm
from tests.oracle_pins import _golden


def _random_tables(rng, lens, bs, pool):
    perm = [int(x) for x in rng.permutation(pool)]
    tables, pos = [], 0
    for n in lens:
        c = -(-int(n) // bs)
        tables.append(perm[pos:pos + c])
        pos += c
    return tables


def test_worked_example():
    g = _golden("prefill_worked_example.json")
    got = pm.prefill_inputs([g["block_table"]], [g["num_cached"]],
                            [g["num_tokens"] - g["num_cached"]],
                            g["block_size"])
    exp = g["expected"]
    assert got["slot_mapping"].tolist() == exp["slot_mapping"]
    assert got["cu_seqlens_q"].tolist() == exp["cu_seqlens_q"]
    assert got["cu_seqlens_k"].tolist() == exp["cu_seqlens_k"]
    assert got["needs_block_tables"] == exp["needs_block_tables"]


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_decode_matches_oracle(bs):
    rng = np.random.default_rng(bs)
    for _ in range(20):
        lens = rng.integers(1, 400, size=int(rng.integers(1, 12)))
        tables = _random_tables(rng, lens, bs, 4000)
        got = pm.decode_inputs(tables, lens, bs)
        want = om.decode_metadata(
            [{"block_table": t, "length": int(n)} for t, n in zip(tables, lens)],
            bs)
        assert got["slot_mapping"].tolist() == want["slot_mapping"]
        assert got["context_lens"].tolist() == want["context_lens"]
        assert got["block_tables"].tolist() == want["block_tables"]
        assert got["slot_mapping"].dtype == np.int32


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_prefill_matches_oracle(bs):
    rng = np.random.default_rng(100 + bs)
    for _ in range(20):
        n = int(rng.integers(1, 8))
        cached = rng.integers(0, 300, size=n)
        sched = rng.integers(0, 200, size=n)
        tables = _random_tables(rng, cached + sched, bs, 6000)
        got = pm.prefill_inputs(tables, cached, sched, bs)
        want = om.prefill_metadata(
            [{"block_table": t, "num_cached": int(c), "num_scheduled": int(s)}
             for t, c, s in zip(tables, cached, sched)], bs)
        for key in ("slot_mapping", "cu_seqlens_q", "cu_seqlens_k"):
            assert got[key].tolist() == want[key], key
        for key in ("max_seqlen_q", "max_seqlen_k", "needs_block_tables"):
            assert got[key] == want[key], key


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_pool_matches_oracle(seed):
    """Random fork / append / release traffic: the product pool and the
    oracle's ref-counted pool produce the same tables, slots, block copies
    and counts."""
    rng = np.random.default_rng(seed)
    bs, nb = 4, 64
    pool = pm.BlockPool(nb)
    ref = om.RefCountedPool(range(nb))
    seqs = []                 # (product table, oracle table, length)
    for _ in range(200):
        op = rng.integers(0, 10)
        if op < 2 or not seqs:                       # new sequence
            seqs.append(([], [], 0))
        elif op < 4:                                 # fork
            t, r, n = seqs[rng.integers(0, len(seqs))]
            seqs.append((pool.share(t), ref.share(r), n))
        elif op < 5 and len(seqs) > 1:               # finish
            t, r, n = seqs.pop(rng.integers(0, len(seqs)))
            pool.release(t)
            ref.release(r)
        else:                                        # one decode step
            picks = rng.choice(len(seqs), size=min(len(seqs), 3),
                               replace=False)
            if pool.num_free < 2 * len(picks):
                continue
            tables = [seqs[i][0] for i in picks]
            lens = [seqs[i][2] for i in picks]
            slots, pairs = pool.append_slots(tables, lens, bs)
            want_pairs = []
            for k, i in enumerate(picks):
                t, r, n = seqs[i]
                r, n2, slot, copy = ref.append(r, n, bs)
                assert slot == slots[k]
                if copy is not None:
                    want_pairs.append(list(copy))
                seqs[i] = (t, r, n2)
            assert pairs.tolist() == want_pairs
        for t, r, _ in seqs:
            assert t == r
        for blk, count in ref.ref.items():
            assert pool.refs[blk] == count
        assert pool.num_free == len(ref.free)


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_shared_prefix_inputs_match_oracle(seed):
    """Random batches with planted runs of sharers (prefixes of various
    lengths, partial last blocks, equal ids past a sequence's full blocks):
    the product's sharing groups equal the oracle's exactly."""
    rng = np.random.default_rng(seed)
    bs = 16
    tables, lens = [], []
    nxt = 1000
    while len(tables) < 40:
        run = int(rng.integers(1, 6))
        k = int(rng.integers(0, 6))
        prefix = list(range(nxt, nxt + k))
        nxt += k
        for _ in range(run):
            extra = int(rng.integers(0, 4))
            t = prefix[:int(rng.integers(max(k - 1, 0), k + 1))] + \
                list(range(nxt, nxt + extra + 1))
            nxt += extra + 1
            n = (len(t) - 1) * bs + int(rng.integers(1, bs + 1))
            tables.append(t)
            lens.append(n)
    got = pm.shared_prefix_inputs(tables, lens, bs)
    want_lens, want_groups = om.shared_prefix_groups(
        [{"block_table": t, "length": n} for t, n in zip(tables, lens)], bs)
    assert got["prefix_lens"].tolist() == want_lens
    assert [tuple(g) for g in got["groups"].tolist()] == want_groups
    assert got["max_group_size"] == max((c for _, c in want_groups), default=0)
    assert got["max_prefix_len"] == max(want_lens)
    assert got["max_suffix_len"] == max(n - p for n, p in zip(lens, want_lens))
