"""pa_decode_shared_prefix on the GPU against the oracle's plain decode.

The call reads each group's shared leading blocks once for the whole group
and merges partial results; its output must equal decode attention over
every sequence's whole context.  Slots outside any context are NaN."""

import numpy as np
import pytest
import torch

import workloads as wl
from paged_kv_cache_slot_amd import metadata as pm
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import (TOL, DecodeCase, bits_equal, dev_i32, f64,
                               sample_seqs, say)

pytestmark = pytest.mark.gpu


def _grouped_layout(spec, seed, bs=16):
    """spec: list of (shared_blocks, [context lengths]) -- each entry with
    shared_blocks > 0 is a run of consecutive sequences whose first
    shared_blocks blocks are the same physical blocks (the first member's);
    shared_blocks == 0 entries are independent sequences."""
    lens = [n for _, ls in spec for n in ls]
    lay = wl.decode_layout(lens, bs, seed=seed)
    tables = [np.array(t) for t in lay.tables]
    i = 0
    for k, ls in spec:
        if k:
            for j in range(i + 1, i + len(ls)):
                assert len(tables[j]) >= k and len(tables[i]) >= k
                tables[j][:k] = tables[i][:k]
        i += len(ls)
    return wl.DecodeLayout(lens=lay.lens, tables=tables,
                           num_blocks=lay.num_blocks, block_size=bs)


def _run(case, seqs=None, expect_groups=None):
    case.run_store()
    sp = pm.shared_prefix_inputs(case.tables, case.lens, case.bs)
    if expect_groups is not None:
        assert [tuple(g) for g in sp["groups"].tolist()] == expect_groups
    out = ops.decode_shared_prefix(
        case.q, case.kc, case.vc, case.block_tables, case.context_lens,
        dev_i32(sp["prefix_lens"]),
        dev_i32(sp["groups"].reshape(-1, 2)), sp["max_suffix_len"],
        sp["max_prefix_len"], sp["max_group_size"], scale=case.scale)
    torch.cuda.synchronize()
    ek, ev = case.oracle_store()
    assert bits_equal(wl.host_bits(case.kc), ek), "store mismatch"
    want = case.oracle_decode(ek, ev, seqs=seqs)
    got = f64(out)
    rows = list(range(len(case.lens))) if seqs is None else seqs
    assert np.all(np.isfinite(got[rows]))
    err = float(np.max(np.abs(got[rows] - want[rows])))
    assert err <= TOL[case.dtype], f"max abs err {err}"
    return sp


SPEC = [
    (3, [60, 49, 100, 200]),        # 4 members share 3 blocks (48 tokens)
    (0, [33]),
    (5, [81, 300, 97]),             # 3 members share 5 blocks
    (0, [1, 17]),
    (2, [40, 33]),
]


@pytest.mark.parametrize("dtype,d,hq,hkv", [
    ("bf16", 128, 32, 8), ("bf16", 64, 8, 1), ("bf16", 128, 8, 8),
    ("f32", 64, 8, 2), ("f32", 128, 8, 4),
])
def test_groups_and_singles(dtype, d, hq, hkv):
    """Three groups (2-5 shared blocks) between independent sequences, every
    supported dtype / head_dim and GQA ratios 1, 4, 8."""
    say("shared prefix groups", dtype, d, hq, hkv)
    case = DecodeCase(_grouped_layout(SPEC, 71), hq, hkv, d, dtype, seed=72)
    _run(case, expect_groups=[(0, 4), (5, 3), (10, 2)])


def test_long_prefix_many_chunks():
    """Six sequences sharing 60 blocks (960 tokens): the shared keys run as
    several chunk partials; suffixes 1..300 tokens."""
    say("shared prefix long")
    spec = [(60, [961, 1000, 1100, 1260, 970, 985])]
    case = DecodeCase(_grouped_layout(spec, 73), 32, 8, 128, "bf16", seed=74)
    sp = _run(case, expect_groups=[(0, 6)])
    assert sp["max_prefix_len"] == 960


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_suffixes_merge_pass(dtype):
    """Suffixes longer than one 512-token partition: the suffix partials
    and the prefix partials meet in the merge pass (short suffixes merge
    the prefix partials inside the partition kernel instead)."""
    say("shared prefix long suffixes", dtype)
    spec = [(20, [1000, 2100, 340, 800]), (0, [1500]), (6, [97, 700])]
    case = DecodeCase(_grouped_layout(spec, 79), 32, 8, 128, dtype, seed=80)
    sp = _run(case, expect_groups=[(0, 4), (5, 2)])
    assert sp["max_suffix_len"] > 512


def test_empty_suffix_member():
    """A member whose whole context is the shared prefix (its new token is
    the last slot of the last shared block): its suffix is empty and only
    the prefix partials reach the merge."""
    say("shared prefix empty suffix")
    spec = [(4, [64, 70, 90])]
    case = DecodeCase(_grouped_layout(spec, 75), 8, 2, 128, "bf16", seed=76)
    _run(case, expect_groups=[(0, 3)])


def test_no_groups_equals_decode():
    """No sharing at all: every prefix length is 0, no groups; the call is
    the plain decode (partitions + merge)."""
    say("shared prefix none")
    lay = wl.decode_layout([5, 16, 17, 700, 1500], 16, seed=77)
    case = DecodeCase(lay, 16, 2, 64, "f32", seed=78)
    sp = _run(case, expect_groups=[])
    assert sp["max_prefix_len"] == 0


def test_prefix_workload_full_size_sampled():
    """The prefix-sharing workload as the bench runs it: 128 sequences
    sharing a 128-block prefix, suffixes U[1,512]; the oracle checks
    sampled sequences."""
    cfg = wl.get_config("prefix")
    say("shared prefix full-size sampled")
    lay = wl.config_decode_layout(cfg)
    case = DecodeCase(lay, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim,
                      cfg.dtype, seed=cfg.seed)
    _run(case, seqs=sample_seqs(lay.lens, 10, cfg.seed),
         expect_groups=[(0, 128)])


def test_large_values_prefix_partials():
    """V values near 2^20 (bf16): the prefix pass's partials and the suffix
    partitions' partials reach 2^15 and are stored scaled; the merge must
    undo it.  Checked relative to the output size."""
    say("shared prefix large values")
    case = DecodeCase(_grouped_layout(SPEC, seed=93), 32, 8, 128, "bf16",
                      seed=94)
    case.vc.mul_(2.0 ** 20)
    case.v_new.mul_(2.0 ** 20)
    case.h_vc = wl.host_bits(case.vc)
    case.h_vn = wl.host_bits(case.v_new)
    case.run_store()
    sp = pm.shared_prefix_inputs(case.tables, case.lens, case.bs)
    assert len(sp["groups"]) > 0
    out = ops.decode_shared_prefix(
        case.q, case.kc, case.vc, case.block_tables, case.context_lens,
        dev_i32(sp["prefix_lens"]),
        dev_i32(sp["groups"].reshape(-1, 2)), sp["max_suffix_len"],
        sp["max_prefix_len"], sp["max_group_size"], scale=case.scale)
    torch.cuda.synchronize()
    ek, ev = case.oracle_store()
    want = case.oracle_decode(ek, ev)
    got = f64(out)
    assert np.all(np.isfinite(got))
    big = np.max(np.abs(want))
    assert big > 65504
    err = float(np.max(np.abs(got - want)))
    assert err <= big * 2.0 ** -7, (err, big)


@pytest.mark.parametrize("spec,seed", [
    ([(3, [60, 49, 100, 200]), (0, [33]), (5, [81, 300, 97]), (0, [1, 17]),
      (2, [40, 33])], 95),
    ([(20, [1000, 2100, 340, 800]), (0, [1500]), (6, [97, 700])], 97),
])
def test_suffix_schedule_from_prefix_pass(spec, seed):
    """The prefix pass's last workgroup writes the suffix pass's schedule
    (the last array of the workspace): a permutation of the (partition,
    sequence) items whose suffix tokens never increase, one or several
    512-token partitions.  The output still matches the oracle."""
    say("shared prefix suffix schedule", seed)
    hq, hkv, d = 32, 8, 128
    case = DecodeCase(_grouped_layout(spec, seed), hq, hkv, d, "bf16",
                      seed=seed + 1)
    case.run_store()
    sp = pm.shared_prefix_inputs(case.tables, case.lens, case.bs)
    b = len(case.lens)
    ng = int(sp["groups"].shape[0])
    need = ops.shared_prefix_workspace_bytes(
        b, hq, hkv, d, sp["max_suffix_len"], sp["max_prefix_len"], ng,
        sp["max_group_size"])
    ws = torch.full((need,), 0xEE, dtype=torch.uint8, device=case.q.device)
    out = ops.decode_shared_prefix(
        case.q, case.kc, case.vc, case.block_tables, case.context_lens,
        dev_i32(sp["prefix_lens"]), dev_i32(sp["groups"].reshape(-1, 2)),
        sp["max_suffix_len"], sp["max_prefix_len"], sp["max_group_size"],
        scale=case.scale, workspace=ws)
    torch.cuda.synchronize()
    part = 512
    nparts = max(1, -(-int(sp["max_suffix_len"]) // part))
    n = b * nparts
    off = need - (n * 4 + 255) // 256 * 256
    order = ws[off:off + n * 4].cpu().numpy().view(np.int32)
    assert sorted(order.tolist()) == list(range(n)), order
    lens = np.asarray(case.lens, dtype=np.int64)
    start = np.asarray(sp["prefix_lens"], dtype=np.int64)
    start -= start % case.bs
    item = np.arange(n)
    toks = np.clip(lens[item % b] - start[item % b] - (item // b) * part, 0, part)
    bins = (toks + case.bs - 1) // case.bs
    assert np.all(np.diff(bins[order]) <= 0), bins[order]
    ek, ev = case.oracle_store()
    want = case.oracle_decode(ek, ev)
    err = float(np.max(np.abs(f64(out) - want)))
    assert err <= TOL["bf16"], f"max abs err {err}"


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (64, 8, 128), (32, 8, 64)])
def test_group_spans_partial_mtile(hq, hkv, d):
    """40 members sharing 10 blocks: G x 40 packed rows per KV head (160 or
    320) fill one or two M-tiles of the group-mode kernel and part of the
    next; suffixes of 1..120 tokens.  Sampled members against the oracle."""
    say("shared prefix partial M-tile", hq, hkv, d)
    rng = np.random.default_rng(99)
    lens = [160 + int(x) for x in rng.integers(1, 121, size=40)]
    case = DecodeCase(_grouped_layout([(10, lens)], 98), hq, hkv, d, "bf16",
                      seed=97)
    _run(case, seqs=[0, 1, 17, 31, 38, 39], expect_groups=[(0, 40)])
