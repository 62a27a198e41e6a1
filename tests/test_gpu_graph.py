"""The entry points can be captured in a HIP graph: a call makes no host
synchronisation, no allocation and no memset node.  One graph holds a decode
step (store, then decode through the partition kernel and the merge) and a
chunked prefill with more work items
than a workgroup has threads (plan kernel, then attention).  It is replayed
several times with q changed in place before each replay and eager calls in
between; every replay must equal the eager calls on the same inputs bit for
bit (both run the same kernels on the same data)."""

import numpy as np
import pytest
import torch

import workloads as wl
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import DecodeCase, PrefillCase, bits_equal, say

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    say("graph capture: decode step + chunked prefill")
    rng = np.random.default_rng(91)
    # 64 sequences x 8 KV heads x 8 partitions of 512 tokens = 4,096
    # workgroups: the partition kernel (its waves rank their own items) and
    # the merge run.
    lens = rng.integers(512, 4096, 64, endpoint=True).tolist()
    lens[0] = 4096
    dec = DecodeCase(wl.decode_layout(lens, 16, seed=92), 32, 8, 128, "bf16",
                     seed=93)
    # 40 sequences x 16 M-tiles = 640 items: the prefill plan kernel runs.
    hist = rng.integers(0, 300, 40).tolist()
    chunk = rng.integers(1, 100, 40).tolist()
    chunk[5] = 1024
    pre = PrefillCase(wl.prefill_layout(hist, chunk, 16, seed=94), 32, 8, 128,
                      "bf16", seed=95)
    dm, pm = dec.meta, pre.meta
    dws = torch.empty(max(ops.decode_workspace_bytes(
        len(lens), 32, 8, 128, dm["max_context_len"]), 1),
        dtype=torch.uint8, device="cuda")
    pws = torch.empty(max(ops.prefill_workspace_bytes(
        len(hist), 32, 8, 128, pm["max_seqlen_q"], pm["max_seqlen_k"]), 1),
        dtype=torch.uint8, device="cuda")
    dout = torch.empty_like(dec.q)
    pout = torch.empty_like(pre.q)

    def calls():
        dec.run_store()
        dec.run_decode(out=dout, workspace=dws)
        pre.run_store()
        pre.run_prefill(out=pout, workspace=pws)

    calls()                       # once eagerly: one-time set-up stays outside
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    for r in range(3):
        dec.q.copy_(wl.make_values(tuple(dec.q.shape), "bf16", 200 + r, "cuda"))
        pre.q.copy_(wl.make_values(tuple(pre.q.shape), "bf16", 300 + r, "cuda"))
        dout.fill_(float("nan"))
        pout.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_d, got_p = wl.host_bits(dout).copy(), wl.host_bits(pout).copy()
        assert np.isfinite(dout.float().cpu().numpy()).all(), f"replay {r}"
        assert np.isfinite(pout.float().cpu().numpy()).all(), f"replay {r}"
        dout.fill_(float("nan"))
        pout.fill_(float("nan"))
        calls()
        torch.cuda.synchronize()
        assert bits_equal(got_d, wl.host_bits(dout)), f"decode, replay {r}"
        assert bits_equal(got_p, wl.host_bits(pout)), f"prefill, replay {r}"


def test_graph_shared_prefix():
    """The shared-prefix decode (prefix pass on MFMA, then the suffix
    partitions, which merge the prefix partials) captured in a graph:
    replays must equal eager calls bit for bit."""
    from paged_kv_cache_slot_amd import metadata as pm
    from tests.gpu_harness import dev_i32
    from tests.test_gpu_shared_prefix import _grouped_layout
    say("graph capture: shared-prefix decode")
    rng = np.random.default_rng(97)
    spec = [(40, (640 + rng.integers(1, 300, 12)).tolist()), (0, [90, 700]),
            (9, (144 + rng.integers(1, 80, 5)).tolist())]
    case = DecodeCase(_grouped_layout(spec, 98), 32, 8, 128, "bf16", seed=99)
    sp = pm.shared_prefix_inputs(case.tables, case.lens, case.bs)
    assert sp["groups"].shape[0] == 2
    pl, gr = dev_i32(sp["prefix_lens"]), dev_i32(sp["groups"].reshape(-1, 2))
    ws = torch.empty(max(ops.shared_prefix_workspace_bytes(
        len(case.lens), 32, 8, 128, sp["max_suffix_len"], sp["max_prefix_len"],
        sp["groups"].shape[0], sp["max_group_size"]), 1),
        dtype=torch.uint8, device="cuda")
    out = torch.empty_like(case.q)

    def calls():
        case.run_store()
        ops.decode_shared_prefix(case.q, case.kc, case.vc, case.block_tables,
                                 case.context_lens, pl, gr, sp["max_suffix_len"],
                                 sp["max_prefix_len"], sp["max_group_size"],
                                 scale=case.scale, out=out, workspace=ws)

    calls()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for r in range(3):
        case.q.copy_(wl.make_values(tuple(case.q.shape), "bf16", 400 + r, "cuda"))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = wl.host_bits(out).copy()
        assert np.isfinite(out.float().cpu().numpy()).all(), f"replay {r}"
        out.fill_(float("nan"))
        calls()
        torch.cuda.synchronize()
        assert bits_equal(got, wl.host_bits(out)), f"replay {r}"


def test_graph_small_row_routes():
    """Decode calls that run on the small-row kernel, captured together:
    a large bf16 batch (one partition per sequence), a bf16 batch split
    into 2 partitions of 4,096 tokens (partials and a merge), and the 8-bit
    cache's store and decode.  Each call's plan kernel zeroes its own ticket
    counter, so every replay restarts the persistent workgroups; replays
    (with q changed in place) equal eager calls bit for bit."""
    import math
    from paged_kv_cache_slot_amd import metadata as pm
    from tests.gpu_harness import dev_i32
    say("graph capture: small-row decode routes")
    rng = np.random.default_rng(97)
    lens1 = rng.integers(1, 3000, 259, endpoint=True).tolist()
    big = DecodeCase(wl.decode_layout(lens1, 16, seed=98), 32, 8, 128, "bf16",
                     seed=99)
    lens2 = rng.integers(1, 8192, 192, endpoint=True).tolist()
    lens2[0] = 8192
    split = DecodeCase(wl.decode_layout(lens2, 16, seed=100), 32, 8, 128,
                       "bf16", seed=101)
    lay3 = wl.decode_layout(rng.integers(1, 3000, 259, endpoint=True).tolist(),
                            16, seed=102)
    kc8, vc8 = wl.fill_pool_codes(lay3.num_blocks, 16, 8, 128, 103, "cuda")
    q8 = wl.make_values((259, 32, 128), "bf16", 104, "cuda")
    kn8 = wl.make_values((259, 8, 128), "bf16", 105, "cuda")
    vn8 = wl.make_values((259, 8, 128), "bf16", 106, "cuda")
    m3 = pm.decode_inputs(lay3.tables, lay3.lens, 16)
    slot8, bt8 = dev_i32(m3["slot_mapping"]), dev_i32(m3["block_tables"])
    cl8 = dev_i32(m3["context_lens"])

    def ws(b, mcl):
        return torch.empty(max(ops.decode_workspace_bytes(b, 32, 8, 128, mcl),
                               1), dtype=torch.uint8, device="cuda")
    w1, w2 = ws(259, big.max_context_len), ws(192, split.max_context_len)
    w3 = ws(259, m3["max_context_len"])
    o1, o2, o3 = (torch.empty_like(x) for x in (big.q, split.q, q8))

    def calls():
        big.run_store()
        big.run_decode(out=o1, workspace=w1)
        split.run_store()
        split.run_decode(out=o2, workspace=w2)
        ops.store_kv_fp8(kn8, vn8, kc8, vc8, slot8, 1 / 16, 1 / 8)
        ops.decode_fp8(q8, kc8, vc8, bt8, cl8, m3["max_context_len"], 1 / 16,
                       1 / 8, scale=1 / math.sqrt(128), out=o3, workspace=w3)

    calls()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    outs = (o1, o2, o3)
    for r in range(3):
        for x, sd in ((big.q, 400), (split.q, 500), (q8, 600)):
            x.copy_(wl.make_values(tuple(x.shape), "bf16", sd + r, "cuda"))
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [wl.host_bits(o).copy() for o in outs]
        for o in outs:
            assert np.isfinite(o.float().cpu().numpy()).all(), f"replay {r}"
            o.fill_(float("nan"))
        calls()
        torch.cuda.synchronize()
        for name, g, o in zip(("bf16", "bf16 split", "e4m3"), got, outs):
            assert bits_equal(g, wl.host_bits(o)), f"{name}, replay {r}"
