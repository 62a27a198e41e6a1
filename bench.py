"""Benchmark of the paged KV-cache hot path on one MI355X.

One step = one decode step of an 8B-shaped attention layer: pa_store_kv of
the 256 newest K/V rows (one per sequence), then pa_decode of 256 sequences
with contexts uniform in [512, 8192], 32 query / 8 KV heads, head_dim 128,
bf16, block size 16 -- on one HIP stream, inputs resident in HBM.

The same run also times the mixed step, which exercises every kernel of the
path: one pa_store_kv of 4,288 rows, pa_prefill_varlen of 8 chunks of 512
rows over 0..8192 cached tokens, and pa_decode of 192 rows; it is reported in
``mixed_step`` with its own MFMA roofline for the prefill kernel.

Prints one JSON line.  ``value`` is the step's algorithmic HBM throughput in
TB/s (KV bytes the decode must read + q/out/block ids + the store's bytes,
over the step time); ``tokens_per_s`` is sequences decoded per second for
this one layer.  ``roofline`` covers pa_decode (for this batch: the plan
kernel and the persistent small-row attention kernel, one query row per
sequence) timed with HIP events on its stream inside the timed region;
``cpu_baseline`` times the fp64 oracle on a bounded sample of the same
sequences on the host cores.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
WORKLOAD = "decode8b"
MIXED = "mixed"
PREFIX = "prefix"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget for the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="before timing, copy 1 GiB once with a plain copy "
                         "kernel, so HBM counters can be scaled against it")
    ap.add_argument("--mixed-steps", type=int, default=20,
                    help="timed steps of the mixed chunked-prefill + decode "
                         "workload (0 skips it)")
    ap.add_argument("--prefix-steps", type=int, default=20,
                    help="timed steps of the prefix-sharing decode workload "
                         "(0 skips it)")
    ap.add_argument("--tiny-steps", type=int, default=20,
                    help="timed steps of the tiny fp32 decode workload "
                         "(0 skips it)")
    ap.add_argument("--small-steps", type=int, default=20,
                    help="timed calls of the small-model decode workload "
                         "(0 skips it)")
    ap.add_argument("--fp8-steps", type=int, default=20,
                    help="timed steps of the 8B-shaped decode step over an "
                         "8-bit (E4M3) cache (0 skips it)")
    ap.add_argument("--verify-steps", type=int, default=20,
                    help="timed calls per Lq of the 8B-shaped verify step "
                         "(0 skips it)")
    ap.add_argument("--indirection-steps", type=int, default=20,
                    help="timed calls per placement of the block-table "
                         "indirection leg (0 skips it)")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the oracle check of each timed workload's "
                         "outputs")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="MiB read between timed steps (outside the timed "
                         "events) so that no step reads the previous step's "
                         "data from L2 / MALL; 0 disables")
    return ap.parse_args()


class Flusher:
    """Reads a scratch buffer between timed steps (outside their events), so
    that L2 and MALL hold none of the previous step's data.  A read leaves
    no dirty lines whose write-back would land in the next step."""

    def __init__(self, mb, dev):
        import torch
        self.buf = torch.ones((mb << 20) // 4, dtype=torch.float32,
                              device=dev) if mb > 0 else None
        self.sink = []

    def __call__(self):
        if self.buf is not None:
            self.sink = [self.buf.sum()]


def settle(fn, min_s=0.05):
    """More untimed warm-up after a leg's warm-up steps: calls in groups of
    four until min_s seconds of back-to-back work have run, so that a leg
    timed after seconds of host-side work (pool copies for the check, the
    oracle) does not start at idle clocks."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def f64(t):
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def stats_ms(ms):
    """median, p10, p90 and mean of per-step times (ms)."""
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4),
            "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4),
            "mean": round(float(a.mean()), 4)}


# HBM traffic per launch measured with rocprofv3 --pmc (FETCH_SIZE and
# WRITE_SIZE, one pass each, scaled against a plain 1 GiB copy) lives in the
# committed summaries under profiles/, each with the sha256 of the kernel
# sources it was taken on.  A summary whose hash no longer matches the
# sources describes an older kernel and yields null.
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "paged_kv_cache_slot_amd", "csrc")


def sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic(summary, sources):
    path = os.path.join(PROFILES, summary)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("counters-json:"):
                rec = json.loads(line[len("counters-json:"):])
                if rec.get("sources_sha256") == sources_sha256(sources):
                    return rec.get("traffic_bytes")
    return None


# The 8B-shaped decode runs on the small-row attention kernel (api.cpp
# routes large bf16 batches there).
DECODE_SOURCES = ("verify.hip", "pa_tile.h", "pa_device.h", "pa_internal.h",
                  "api.cpp")
PREFILL_SOURCES = ("prefill.hip", "pa_tile.h", "pa_device.h", "pa_internal.h")


def decode_bytes(lens, hq, hkv, d, elem, bs=16):
    row = 2 * hkv * d * elem
    kv = int(sum(int(n) for n in lens)) * row
    qo = len(lens) * hq * d * elem * 2
    ids = 4 * int(sum(-(-int(n) // bs) for n in lens)) + 4 * len(lens)
    return kv + qo + ids


def prefill_flops(lq, lk, hq, d):
    """Algorithmic FLOPs of causal prefill: 4 * D * Hq per unmasked (q, k)
    pair (QK^T and PV, multiply + add); row i of a chunk of Lq rows over Lk
    keys sees Lk - Lq + i + 1 keys."""
    pairs = sum(int(a) * (int(b) - int(a)) + int(a) * (int(a) + 1) // 2
                for a, b in zip(lq, lk))
    return 4 * d * hq * pairs


def cpu_prefill_baseline(h_q, h_kc, h_vc, cu_q, cu_k, tables, hq, d, scale,
                         budget_s):
    """Time the oracle's chunked prefill, one whole chunk at a time (its rows
    and its block table), in a fixed shuffled order, until ~budget_s pass."""
    import numpy as np
    import oracle.attention as oa
    order = np.random.default_rng(0).permutation(len(tables)).tolist()
    flops, done, t0 = 0, 0, time.perf_counter()
    for b in order:
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        lk = int(cu_k[b + 1] - cu_k[b])
        oa.prefill_attention(h_q[q0:q1], h_kc, h_vc, [0, q1 - q0], [0, lk],
                             [[int(x) for x in tables[b]]], scale, True, "bf16")
        flops += prefill_flops(np.array([q1 - q0]), np.array([lk]), hq, d)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, flops, time.perf_counter() - t0


def run_mixed(steps, warmup, dev, flush, cpu_s=0.0, check=True):
    """Mixed step: one pa_store_kv of every new row (8 x 512 chunk rows + 192
    decode rows), then pa_prefill_varlen of the chunks, then pa_decode of the
    decode rows, on one stream.  Returns a dict for the JSON line."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_slot_amd import metadata as pm
    from paged_kv_cache_slot_amd import ops

    cfg = wl.get_config(MIXED)
    pre, dec = wl.mixed_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    kc, vc = wl.fill_pool(pre.num_blocks, bs, hkv, d, "bf16", cfg.seed, dev)
    tq = int(pre.chunk.sum())
    nd = len(dec.lens)
    qp = wl.make_values((tq, hq, d), "bf16", cfg.seed + 1, dev)
    qd = wl.make_values((nd, hq, d), "bf16", cfg.seed + 2, dev)
    k_new = wl.make_values((tq + nd, hkv, d), "bf16", cfg.seed + 3, dev)
    v_new = wl.make_values((tq + nd, hkv, d), "bf16", cfg.seed + 4, dev)
    mp = pm.prefill_inputs(pre.tables, pre.history, pre.chunk, bs)
    md = pm.decode_inputs(dec.tables, dec.lens, bs)
    slots = torch.as_tensor(np.concatenate([mp["slot_mapping"],
                                            md["slot_mapping"]]), device=dev)
    cu_q = torch.as_tensor(mp["cu_seqlens_q"], device=dev)
    cu_k = torch.as_tensor(mp["cu_seqlens_k"], device=dev)
    btp = torch.as_tensor(mp["block_tables"], device=dev)
    btd = torch.as_tensor(md["block_tables"], device=dev)
    cl = torch.as_tensor(md["context_lens"], device=dev)
    scale = 1.0 / math.sqrt(d)
    # host copies for the oracle check, taken before any kernel runs
    host = [wl.host_bits(x) for x in (kc, vc, k_new, v_new, qp, qd)] \
        if check else None
    outp = torch.empty_like(qp)
    outd = torch.empty_like(qd)
    wsd = torch.empty(max(ops.decode_workspace_bytes(
        nd, hq, hkv, d, md["max_context_len"]), 1), dtype=torch.uint8,
        device=dev)
    wsp = torch.empty(max(ops.prefill_workspace_bytes(
        len(pre.chunk), hq, hkv, d, mp["max_seqlen_q"], mp["max_seqlen_k"]),
        1), dtype=torch.uint8, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ops.store_kv(k_new, v_new, kc, vc, slots)
        if ev is not None:
            ev[1].record()
        ops.prefill_varlen(qp, kc, vc, cu_q, cu_k, mp["max_seqlen_q"],
                           mp["max_seqlen_k"], btp, scale=scale, causal=True,
                           out=outp, workspace=wsp)
        if ev is not None:
            ev[2].record()
        ops.decode(qd, kc, vc, btd, cl, md["max_context_len"], scale=scale,
                   out=outd, workspace=wsd)
        if ev is not None:
            ev[3].record()

    for _ in range(warmup):
        step()
    settle(step)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for _ in range(steps)]
    for i in range(steps):
        flush()
        step(evs[i])
    torch.cuda.synchronize()
    import numpy as np
    st = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    pf_all = [e[1].elapsed_time(e[2]) for e in evs]
    pf = float(np.median(pf_all))
    dc = float(np.median([e[2].elapsed_time(e[3]) for e in evs]))
    total = float(np.median([e[0].elapsed_time(e[3]) for e in evs]))
    flops = prefill_flops(pre.chunk, pre.history + pre.chunk, hq, d)
    dbytes = decode_bytes(dec.lens, hq, hkv, d, 2)
    row = 2 * hkv * d * 2
    sbytes = 2 * (tq + nd) * row + 4 * (tq + nd)
    tflops = flops / (pf * 1e-3) / 1e12
    cpu = None
    if cpu_s > 0:
        # the oracle on the cache as the timed steps left it
        done, cflops, dt = cpu_prefill_baseline(
            wl.host_bits(qp), wl.host_bits(kc), wl.host_bits(vc),
            mp["cu_seqlens_q"], mp["cu_seqlens_k"], pre.tables, hq, d, scale,
            cpu_s)
        cpu = {"value": round(cflops / dt / 1e12, 6), "unit": "TFLOP/s",
               "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
               "sample": f"{done} of {len(pre.chunk)} chunks "
                         f"({cflops / 1e9:.1f} GFLOP), fp64 numpy oracle, "
                         f"{dt:.1f} s"}
    chk = None
    if check:
        chk = cpu_check_mixed(pre, dec, *host[:4], host[4], host[5],
                              f64(outp), f64(outd), scale,
                              {b: [0, 255, 511] for b in range(len(pre.chunk))},
                              sample_sequences(dec.lens, 10, 5))
    return {
        "workload": cfg.title,
        "steps": steps,
        "check": chk,
        "ms_per_step": round(total, 4),
        "store_us": round(st * 1e3, 2),
        "store_gbs": round(sbytes / (st * 1e-3) / 1e9, 1),
        "prefill_us": round(pf * 1e3, 2),
        "prefill_ms_stats": stats_ms(pf_all),
        "prefill_gflop": round(flops / 1e9, 2),
        "decode_us": round(dc * 1e3, 2),
        "decode_tbs": round(dbytes / (dc * 1e-3) / 1e12, 4),
        "decode_tokens_per_s": round(nd / (dc * 1e-3), 1),
        "roofline": {"kernel": "pa_prefill_varlen (prefill_kernel)",
                     "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": committed_traffic(
                         "prefill_mixed_hbm_counters.md", PREFILL_SOURCES),
                     "algorithmic_flops": flops},
        "cpu_baseline": cpu,
    }


def run_prefix(steps, warmup, dev, flush, cpu_s=0.0, check=True):
    """Prefix-sharing decode step: pa_store_kv of each sequence's new token
    (private suffix blocks), then pa_decode; 128 sequences share their first
    128 blocks.  Reports unique-byte (each physical block once) and
    logical-byte (per sequence) rates."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_slot_amd import metadata as pm
    from paged_kv_cache_slot_amd import ops

    cfg = wl.get_config(PREFIX)
    lay = wl.config_decode_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    b = len(lay.lens)
    kc, vc = wl.fill_pool(lay.num_blocks, bs, hkv, d, "bf16", cfg.seed, dev)
    q = wl.make_values((b, hq, d), "bf16", cfg.seed + 1, dev)
    k_new = wl.make_values((b, hkv, d), "bf16", cfg.seed + 2, dev)
    v_new = wl.make_values((b, hkv, d), "bf16", cfg.seed + 3, dev)
    meta = pm.decode_inputs(lay.tables, lay.lens, bs)
    slot = torch.as_tensor(meta["slot_mapping"], device=dev)
    bt = torch.as_tensor(meta["block_tables"], device=dev)
    cl = torch.as_tensor(meta["context_lens"], device=dev)
    scale = 1.0 / math.sqrt(d)
    host = [wl.host_bits(x) for x in (q, kc, vc, k_new, v_new)] \
        if check else None
    out = torch.empty_like(q)
    ws = torch.empty(max(ops.decode_workspace_bytes(
        b, hq, hkv, d, meta["max_context_len"]), 1), dtype=torch.uint8,
        device=dev)

    sp = pm.shared_prefix_inputs(lay.tables, lay.lens, bs)
    pl = torch.as_tensor(sp["prefix_lens"], device=dev)
    groups = torch.as_tensor(sp["groups"], device=dev)
    ng = int(sp["groups"].shape[0])
    wsp = torch.empty(max(ops.shared_prefix_workspace_bytes(
        b, hq, hkv, d, sp["max_suffix_len"], sp["max_prefix_len"], ng,
        sp["max_group_size"]), 1), dtype=torch.uint8, device=dev)
    out2 = torch.empty_like(q)

    def attend_plain():
        ops.decode(q, kc, vc, bt, cl, meta["max_context_len"], scale=scale,
                   out=out, workspace=ws)

    def attend_shared():
        ops.decode_shared_prefix(q, kc, vc, bt, cl, pl, groups,
                                 sp["max_suffix_len"], sp["max_prefix_len"],
                                 sp["max_group_size"], scale=scale, out=out2,
                                 workspace=wsp)

    def timed(attend):
        def step(ev):
            ev[0].record()
            ops.store_kv(k_new, v_new, kc, vc, slot)
            ev[1].record()
            attend()
            ev[2].record()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(steps + warmup)]
        for i in range(warmup):
            step(evs[steps + i])
        settle(lambda: step(evs[steps]))
        torch.cuda.synchronize()
        for i in range(steps):
            flush()
            step(evs[i])
        torch.cuda.synchronize()
        return float(np.median([e[1].elapsed_time(e[2]) for e in evs[:steps]]))

    dec = timed(attend_plain)
    shared = timed(attend_shared)
    diff = float((out.float() - out2.float()).abs().max())
    chk = chk2 = None
    if check:
        seqs = sample_sequences(lay.lens, 8, 4)
        chk = cpu_check_decode(lay.tables, lay.lens, *host, f64(out), scale,
                               "bf16", seqs)
        chk2 = cpu_check_decode(lay.tables, lay.lens, *host, f64(out2), scale,
                                "bf16", seqs)
    row = 2 * hkv * d * 2
    logical = decode_bytes(lay.lens, hq, hkv, d, 2)
    pre_tok = cfg.shared_prefix_blocks * bs
    uniq_tok = pre_tok + int(sum(int(n) - pre_tok for n in lay.lens))
    unique = logical - (int(sum(int(n) for n in lay.lens)) - uniq_tok) * row
    cpu = None
    if cpu_s > 0:
        # the oracle's plain decode: every sequence reads its whole context
        done, toks, dt = cpu_baseline(lay.tables, lay.lens, wl.host_bits(q),
                                      wl.host_bits(kc), wl.host_bits(vc), hq,
                                      scale, cpu_s)
        cpu = {"value": round(toks * row / dt / 1e12, 6), "unit": "TB/s",
               "bytes": "logical", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "tokens_per_s": round(done / dt, 2),
               "sample": f"{done} of {b} sequences ({toks} context tokens), "
                         f"fp64 numpy oracle, {dt:.1f} s"}
    return {
        "workload": cfg.title,
        "steps": steps,
        "cpu_baseline": cpu,
        "check": chk,
        "decode_us": round(dec * 1e3, 2),
        "unique_bytes": unique,
        "logical_bytes": logical,
        "unique_tbs": round(unique / (dec * 1e-3) / 1e12, 4),
        "logical_tbs": round(logical / (dec * 1e-3) / 1e12, 4),
        "decode_tokens_per_s": round(b / (dec * 1e-3), 1),
        "kernel": "pa_decode (every sequence reads its whole context)",
        "shared_prefix": {
            "kernel": "pa_decode_shared_prefix (shared blocks read once per "
                      "group: prefix partials on MFMA, then the suffix "
                      "partitions, which merge them)",
            "groups": ng,
            "decode_us": round(shared * 1e3, 2),
            "unique_tbs": round(unique / (shared * 1e-3) / 1e12, 4),
            "logical_tbs": round(logical / (shared * 1e-3) / 1e12, 4),
            "decode_tokens_per_s": round(b / (shared * 1e-3), 1),
            "speedup_vs_pa_decode": round(dec / shared, 3),
            "max_abs_diff_vs_pa_decode": round(diff, 6),
            "check": chk2,
        },
    }


def run_fp8(steps, warmup, dev, flush, check=True):
    """The 8B-shaped decode step over an 8-bit (E4M3) cache: pa_store_kv_fp8
    of the 256 new rows, then pa_decode_fp8.  Bytes count one byte per
    cached element."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_slot_amd import metadata as pm
    from paged_kv_cache_slot_amd import ops

    cfg = wl.get_config(WORKLOAD)
    lay = wl.config_decode_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    b = len(lay.lens)
    kc, vc = wl.fill_pool_codes(lay.num_blocks, bs, hkv, d, cfg.seed, dev)
    q = wl.make_values((b, hq, d), "bf16", cfg.seed + 1, dev)
    k_new = wl.make_values((b, hkv, d), "bf16", cfg.seed + 2, dev)
    v_new = wl.make_values((b, hkv, d), "bf16", cfg.seed + 3, dev)
    meta = pm.decode_inputs(lay.tables, lay.lens, bs)
    slot = torch.as_tensor(meta["slot_mapping"], device=dev)
    bt = torch.as_tensor(meta["block_tables"], device=dev)
    cl = torch.as_tensor(meta["context_lens"], device=dev)
    maxlen = meta["max_context_len"]
    out = torch.empty_like(q)
    ws = torch.empty(max(ops.decode_workspace_bytes(b, hq, hkv, d, maxlen), 1),
                     dtype=torch.uint8, device=dev)
    ks, vs = 1 / 16, 1 / 16
    host = [wl.host_bits(x) for x in (q, kc, vc, k_new, v_new)] \
        if check else None

    def step(ev):
        ev[0].record()
        ops.store_kv_fp8(k_new, v_new, kc, vc, slot, ks, vs)
        ev[1].record()
        ops.decode_fp8(q, kc, vc, bt, cl, maxlen, ks, vs, out=out,
                       workspace=ws)
        ev[2].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(steps + warmup)]
    for i in range(warmup):
        step(evs[steps + i])
    settle(lambda: step(evs[steps]))
    torch.cuda.synchronize()
    for i in range(steps):
        flush()
        step(evs[i])
    torch.cuda.synchronize()
    dec_all = [e[1].elapsed_time(e[2]) for e in evs[:steps]]
    step_all = [e[0].elapsed_time(e[2]) for e in evs[:steps]]
    dec = float(np.median(dec_all))
    stp = float(np.median(step_all))
    dbytes = decode_bytes(lay.lens, hq, hkv, d, 1) + \
        len(lay.lens) * hq * d * (2 - 1) * 2      # q and out stay bf16
    chk = None
    if check:
        chk = cpu_check_fp8_decode(lay.tables, lay.lens, *host, f64(out),
                                   1.0 / math.sqrt(d), ks, vs,
                                   sample_sequences(lay.lens, 6, 3))
    return {
        "workload": cfg.title + "; 8-bit E4M3 cache",
        "steps": steps,
        "check": chk,
        "decode_us": round(dec * 1e3, 2),
        "step_us": round(stp * 1e3, 2),
        "decode_ms_stats": stats_ms(dec_all),
        "algorithmic_bytes": dbytes,
        "decode_tbs": round(dbytes / (dec * 1e-3) / 1e12, 4),
        "frac_of_hbm_peak": round(dbytes / (dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(b / (stp * 1e-3), 1),
        "kernel": "pa_decode_fp8 (large batch: verify_plan_kernel + verify_kernel<..., E4M3>, codes widened to bfloat16 into LDS)",
    }


def run_tiny(steps, warmup, dev, flush, check=True):
    """Tiny decode step (4 sequences, contexts 7 / 16 / 33 / 100, 8 query /
    2 KV heads, D = 64, fp32): pa_store_kv of the 4 newest rows, then
    pa_decode.  Launch-bound; reported in microseconds."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_slot_amd import metadata as pm
    from paged_kv_cache_slot_amd import ops

    cfg = wl.get_config("tiny")
    lay = wl.config_decode_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    b = len(lay.lens)
    kc, vc = wl.fill_pool(lay.num_blocks, bs, hkv, d, "f32", cfg.seed, dev)
    q = wl.make_values((b, hq, d), "f32", cfg.seed + 1, dev)
    k_new = wl.make_values((b, hkv, d), "f32", cfg.seed + 2, dev)
    v_new = wl.make_values((b, hkv, d), "f32", cfg.seed + 3, dev)
    meta = pm.decode_inputs(lay.tables, lay.lens, bs)
    slot = torch.as_tensor(meta["slot_mapping"], device=dev)
    bt = torch.as_tensor(meta["block_tables"], device=dev)
    cl = torch.as_tensor(meta["context_lens"], device=dev)
    maxlen = meta["max_context_len"]
    out = torch.empty_like(q)
    ws = torch.empty(max(ops.decode_workspace_bytes(b, hq, hkv, d, maxlen), 1),
                     dtype=torch.uint8, device=dev)
    host = [wl.host_bits(x) for x in (q, kc, vc, k_new, v_new)] \
        if check else None

    def step(ev):
        ev[0].record()
        ops.store_kv(k_new, v_new, kc, vc, slot)
        ev[1].record()
        ops.decode(q, kc, vc, bt, cl, maxlen, out=out, workspace=ws)
        ev[2].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
           for _ in range(steps + warmup)]
    for i in range(warmup):
        step(evs[steps + i])
    settle(lambda: step(evs[steps]))
    torch.cuda.synchronize()
    for i in range(steps):
        flush()
        step(evs[i])
    torch.cuda.synchronize()
    step_all = [e[0].elapsed_time(e[2]) for e in evs[:steps]]
    dec_all = [e[1].elapsed_time(e[2]) for e in evs[:steps]]
    chk = None
    if check:
        chk = cpu_check_decode(lay.tables, lay.lens, *host, f64(out),
                               1.0 / math.sqrt(d), "f32", list(range(b)))
    return {
        "workload": cfg.title + "; store 4 rows then decode",
        "steps": steps,
        "check": chk,
        "step_us": round(float(np.median(step_all)) * 1e3, 2),
        "decode_us": round(float(np.median(dec_all)) * 1e3, 2),
        "step_ms_stats": stats_ms(step_all),
        "bound": "launch / latency (159,744 B of K/V)",
        "kernel": "pa_store_kv + pa_decode (one partition, no merge)",
    }


def run_small(steps, warmup, dev, flush, cpu_s=0.0, check=True):
    """Small-model decode: 64 sequences, contexts uniform in [128, 4096],
    16 query / 8 KV heads, D = 128, bf16.  Decode only: the cache is filled
    up front, so the timed call is pa_decode."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_slot_amd import metadata as pm
    from paged_kv_cache_slot_amd import ops

    cfg = wl.get_config("small")
    lay = wl.config_decode_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    b = len(lay.lens)
    kc, vc = wl.fill_pool(lay.num_blocks, bs, hkv, d, "bf16", cfg.seed, dev)
    q = wl.make_values((b, hq, d), "bf16", cfg.seed + 1, dev)
    meta = pm.decode_inputs(lay.tables, lay.lens, bs)
    bt = torch.as_tensor(meta["block_tables"], device=dev)
    cl = torch.as_tensor(meta["context_lens"], device=dev)
    maxlen = meta["max_context_len"]
    out = torch.empty_like(q)
    ws = torch.empty(max(ops.decode_workspace_bytes(b, hq, hkv, d, maxlen), 1),
                     dtype=torch.uint8, device=dev)
    host = [wl.host_bits(x) for x in (q, kc, vc)] if check else None

    def call(ev):
        ev[0].record()
        ops.decode(q, kc, vc, bt, cl, maxlen, out=out, workspace=ws)
        ev[1].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
           for _ in range(steps + warmup)]
    for i in range(warmup):
        call(evs[steps + i])
    settle(lambda: call(evs[steps]))
    torch.cuda.synchronize()
    for i in range(steps):
        flush()
        call(evs[i])
    torch.cuda.synchronize()
    dec_all = [e[0].elapsed_time(e[1]) for e in evs[:steps]]
    dec = float(np.median(dec_all))
    dbytes = decode_bytes(lay.lens, hq, hkv, d, 2)
    cpu = None
    if cpu_s > 0:
        done, toks, dt = cpu_baseline(lay.tables, lay.lens, wl.host_bits(q),
                                      wl.host_bits(kc), wl.host_bits(vc), hq,
                                      1.0 / math.sqrt(d), cpu_s)
        cpu = {"value": round(toks * 2 * hkv * d * 2 / dt / 1e12, 6),
               "unit": "TB/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "tokens_per_s": round(done / dt, 2),
               "sample": f"{done} of {b} sequences ({toks} context tokens), "
                         f"fp64 numpy oracle, {dt:.1f} s"}
    chk = None
    if check:
        chk = cpu_check_decode(lay.tables, lay.lens, *host, None, None,
                               f64(out), 1.0 / math.sqrt(d), "bf16",
                               sample_sequences(lay.lens, 8, 2))
    return {
        "workload": cfg.title,
        "steps": steps,
        "cpu_baseline": cpu,
        "check": chk,
        "decode_us": round(dec * 1e3, 2),
        "decode_ms_stats": stats_ms(dec_all),
        "algorithmic_bytes": dbytes,
        "decode_tbs": round(dbytes / (dec * 1e-3) / 1e12, 4),
        "frac_of_hbm_peak": round(dbytes / (dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(b / (dec * 1e-3), 1),
        "kernel": "pa_decode (decode_partition_kernel, items ranked by the "
                  "workgroups, + decode_merge_kernel)",
    }


def verify_bytes(lens, lq, hq, hkv, d, elem, bs=16):
    """Algorithmic HBM bytes of one verify launch: every sequence's K/V once
    (Lk tokens x Hkv x D, K and V), its Lq query rows in and out, its block
    ids and cu_seqlens."""
    kv = int(sum(int(n) for n in lens)) * 2 * hkv * d * elem
    qo = len(lens) * lq * hq * d * elem * 2
    ids = 4 * int(sum(-(-int(n) // bs) for n in lens)) + 8 * (len(lens) + 1)
    return kv + qo + ids


def run_verify(steps, warmup, dev, flush, check=True, lqs=(2, 4, 8)):
    """The verify pass of speculative decoding on the 8B-shaped decode
    workload ("Warmup Guide -- Inference Serving Internals", Chapter 7; "10
    Serving Engines", section 10.6): each of the 256 sequences (contexts
    uniform in [512, 8192], the last Lq tokens being the proposed ones)
    attends Lq causal query rows, 32 query / 8 KV heads, D = 128, bf16 --
    one pa_prefill_varlen launch, which takes its small-row path (G * Lq <=
    64 packed rows per KV head).  Timed per Lq with HIP events on the
    launch's stream, the cache flushed before every call."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_slot_amd import metadata as pm
    from paged_kv_cache_slot_amd import ops

    cfg = wl.get_config(WORKLOAD)
    lay = wl.config_decode_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    b = len(lay.lens)
    kc, vc = wl.fill_pool(lay.num_blocks, bs, hkv, d, "bf16", cfg.seed, dev)
    hk = [wl.host_bits(kc), wl.host_bits(vc)] if check else None
    scale = 1.0 / math.sqrt(d)
    legs = {}
    for lq in lqs:
        q = wl.make_values((b * lq, hq, d), "bf16", cfg.seed + 20 + lq, dev)
        hq_bits = wl.host_bits(q) if check else None
        meta = pm.prefill_inputs(lay.tables, lay.lens - lq, np.full(b, lq), bs)
        cu_q = torch.as_tensor(meta["cu_seqlens_q"], device=dev)
        cu_k = torch.as_tensor(meta["cu_seqlens_k"], device=dev)
        bt = torch.as_tensor(meta["block_tables"], device=dev)
        out = torch.empty_like(q)
        need = ops.prefill_workspace_bytes(b, hq, hkv, d, meta["max_seqlen_q"],
                                           meta["max_seqlen_k"])
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

        def call(ev=None):
            if ev is not None:
                ev[0].record()
            ops.prefill_varlen(q, kc, vc, cu_q, cu_k, meta["max_seqlen_q"],
                               meta["max_seqlen_k"], bt, scale=scale,
                               causal=True, out=out, workspace=ws)
            if ev is not None:
                ev[1].record()

        for _ in range(warmup):
            call()
        settle(call)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(steps)]
        for i in range(steps):
            flush()
            call(evs[i])
        torch.cuda.synchronize()
        t_all = [e[0].elapsed_time(e[1]) for e in evs]
        t = float(np.median(t_all))
        vbytes = verify_bytes(lay.lens, lq, hq, hkv, d, 2)
        chk = None
        if check:
            chk = cpu_check_verify(lay.tables, lay.lens, lq, hq_bits, hk[0],
                                   hk[1], f64(out), scale,
                                   sample_sequences(lay.lens, 6, 30 + lq))
        legs[f"lq{lq}"] = {
            "us": round(t * 1e3, 2),
            "ms_stats": stats_ms(t_all),
            "algorithmic_bytes": vbytes,
            "tbs": round(vbytes / (t * 1e-3) / 1e12, 4),
            "frac_of_hbm_peak": round(vbytes / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "query_rows_per_s": round(b * lq / (t * 1e-3), 1),
            "check": chk,
        }
        del q, out, ws
    return {
        "workload": "verify pass on the 8B-shaped decode workload: 256 seqs, "
                    "ctx U[512,8192] incl. Lq proposed tokens, Lq causal rows "
                    "each, 32q/8kv, D=128, bf16",
        "steps": steps,
        "kernel": "pa_prefill_varlen small-row path (verify_kernel; one "
                  "partition per sequence, workgroups rank the items)",
        "legs": legs,
    }


def run_indirection(steps, warmup, dev, flush):
    """Cost of the block-table indirection ("Warmup Guide -- Inference
    Serving Internals", Chapter 3 calls it cheap): the 8B-shaped decode
    workload's tokens are placed twice -- once with each sequence's blocks
    at consecutive physical ids, once through the workload's shuffled block
    tables -- by pa_store_kv of the same rows, and pa_decode is timed on
    both, interleaved, with the cache flushed before every call.  The same
    tokens in the same logical order give bit-identical outputs."""
    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_slot_amd import metadata as pm
    from paged_kv_cache_slot_amd import ops

    cfg = wl.get_config(WORKLOAD)
    lay = wl.config_decode_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    b = len(lay.lens)
    counts = [-(-int(n) // bs) for n in lay.lens]
    starts = np.cumsum([0] + counts[:-1])
    consecutive = [np.arange(s0, s0 + c) for s0, c in zip(starts, counts)]
    total = int(sum(int(n) for n in lay.lens))
    k_all = wl.make_values((total, hkv, d), "bf16", cfg.seed + 10, dev)
    v_all = wl.make_values((total, hkv, d), "bf16", cfg.seed + 11, dev)
    q = wl.make_values((b, hq, d), "bf16", cfg.seed + 12, dev)
    zeros = np.zeros(b, dtype=np.int64)
    placements = []
    for name, tables, nb in (("consecutive", consecutive, int(sum(counts))),
                             ("permuted", lay.tables, lay.num_blocks)):
        kc = torch.empty((nb, bs, hkv, d), dtype=torch.bfloat16, device=dev)
        vc = torch.empty_like(kc)
        rows = pm.prefill_inputs(tables, zeros, lay.lens, bs)["slot_mapping"]
        ops.store_kv(k_all, v_all, kc, vc, torch.as_tensor(rows, device=dev))
        meta = pm.decode_inputs(tables, lay.lens, bs)
        bt = torch.as_tensor(meta["block_tables"], device=dev)
        cl = torch.as_tensor(meta["context_lens"], device=dev)
        ws = torch.empty(max(ops.decode_workspace_bytes(
            b, hq, hkv, d, meta["max_context_len"]), 1), dtype=torch.uint8,
            device=dev)
        out = torch.empty_like(q)
        placements.append((name, kc, vc, bt, cl, meta["max_context_len"], ws,
                           out))
    del k_all, v_all
    torch.cuda.synchronize()

    def call(pl, ev=None):
        _, kc, vc, bt, cl, mcl, ws, out = pl
        if ev is not None:
            ev[0].record()
        ops.decode(q, kc, vc, bt, cl, mcl, out=out, workspace=ws)
        if ev is not None:
            ev[1].record()

    for _ in range(warmup):
        for pl in placements:
            call(pl)
    settle(lambda: [call(pl) for pl in placements])
    torch.cuda.synchronize()
    times = {pl[0]: [] for pl in placements}
    for _ in range(steps):
        for pl in placements:
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            flush()
            call(pl, ev)
            torch.cuda.synchronize()
            times[pl[0]].append(ev[0].elapsed_time(ev[1]))
    cons = float(np.median(times["consecutive"]))
    perm = float(np.median(times["permuted"]))
    same = bool(torch.equal(placements[0][7].view(torch.int16),
                            placements[1][7].view(torch.int16)))
    return {
        "workload": cfg.title + "; the same tokens at consecutive block ids "
                    "and through shuffled block tables",
        "steps": steps,
        "consecutive_us": round(cons * 1e3, 2),
        "permuted_us": round(perm * 1e3, 2),
        "indirection_cost": round(perm / cons - 1.0, 4),
        "consecutive_ms_stats": stats_ms(times["consecutive"]),
        "permuted_ms_stats": stats_ms(times["permuted"]),
        "outputs_bit_identical": same,
    }


TOL = {"f32": 1e-5, "bf16": 2e-2}


def sample_sequences(lens, k, seed):
    """Longest, shortest and k - 2 random sequences (sorted)."""
    import numpy as np
    lens = np.asarray(lens)
    pick = {int(np.argmax(lens)), int(np.argmin(lens))}
    for b in np.random.default_rng(seed).permutation(len(lens)).tolist():
        if len(pick) >= k:
            break
        pick.add(int(b))
    return sorted(pick)


def cpu_check_decode(tables, lens, h_q, h_kc, h_vc, h_kn, h_vn, got, scale,
                     dtype, seqs):
    """Correctness of a timed decode step: the oracle's own metadata, store
    and attention on host copies of the inputs taken before any kernel ran
    (h_kn / h_vn None: nothing stored), against the GPU output `got`
    (float64 [B, Hq, D]) on the sequences `seqs`."""
    import numpy as np
    import oracle.attention as oa
    import oracle.metadata as om
    meta = om.decode_metadata([{"block_table": [int(x) for x in t],
                                "length": int(n)}
                               for t, n in zip(tables, lens)], 16)
    if h_kn is not None:
        h_kc, h_vc = oa.store_kv(h_kc, h_vc, h_kn, h_vn,
                                 meta["slot_mapping"])
    want = oa.decode_attention(h_q, h_kc, h_vc, meta["block_tables"],
                               meta["context_lens"], scale, dtype, seqs=seqs)
    err = float(np.max(np.abs(got[seqs] - want[seqs])))
    return {"max_abs_err": err, "tolerance": TOL[dtype],
            "sequences_checked": len(seqs), "ok": bool(err <= TOL[dtype])}


def cpu_check_verify(tables, lens, lq, h_q, h_kc, h_vc, got, scale, seqs):
    """Correctness of a timed verify launch: the oracle's varlen prefill
    (its own cu_seqlens) on the sequences `seqs`, every row."""
    import numpy as np
    import oracle.attention as oa
    b = len(lens)
    cu_q = np.concatenate([[0], np.cumsum(np.full(b, lq))])
    cu_k = np.concatenate([[0], np.cumsum(np.asarray(lens))])
    width = max(len(t) for t in tables)
    tab = [[int(x) for x in t] + [-1] * (width - len(t)) for t in tables]
    want = oa.prefill_attention(h_q, h_kc, h_vc, cu_q, cu_k, tab, scale, True,
                                "bf16", seqs=seqs)
    sel = [r for s in seqs for r in range(cu_q[s], cu_q[s + 1])]
    err = float(np.max(np.abs(got[sel] - want[sel])))
    ok = bool(err <= TOL["bf16"] and np.all(np.isfinite(got)))
    return {"max_abs_err": err, "tolerance": TOL["bf16"],
            "rows_checked": len(sel), "ok": ok}


def cpu_check_fp8_decode(tables, lens, h_q, h_kc, h_vc, h_kn, h_vn, got,
                         scale, k_scale, v_scale, seqs):
    """As cpu_check_decode over an 8-bit (E4M3) cache: the oracle's
    quantising store and E4M3 decode."""
    import numpy as np
    import oracle.fp8 as of8
    import oracle.metadata as om
    meta = om.decode_metadata([{"block_table": [int(x) for x in t],
                                "length": int(n)}
                               for t, n in zip(tables, lens)], 16)
    inv_k = float(np.float32(1.0) / np.float32(k_scale))
    inv_v = float(np.float32(1.0) / np.float32(v_scale))
    ek, ev = of8.store_kv(h_kc, h_vc, h_kn, h_vn, meta["slot_mapping"],
                          inv_k, inv_v, "bf16")
    want = of8.decode_attention(h_q, ek, ev, meta["block_tables"],
                                meta["context_lens"], scale, k_scale, v_scale,
                                "bf16", seqs=seqs)
    err = float(np.max(np.abs(got[seqs] - want[seqs])))
    return {"max_abs_err": err, "tolerance": TOL["bf16"],
            "sequences_checked": len(seqs), "ok": bool(err <= TOL["bf16"])}


def cpu_check_mixed(pre, dec, h_kc, h_vc, h_kn, h_vn, h_qp, h_qd, gotp, gotd,
                    scale, rows, seqs):
    """Correctness of the mixed step: the oracle's store of every new row,
    then its chunked prefill on the given rows of each chunk and its decode
    on the given decode sequences."""
    import numpy as np
    import oracle.attention as oa
    import oracle.metadata as om
    mp = om.prefill_metadata([{"block_table": [int(x) for x in t],
                               "num_cached": int(h), "num_scheduled": int(c)}
                              for t, h, c in zip(pre.tables, pre.history,
                                                 pre.chunk)], 16)
    md = om.decode_metadata([{"block_table": [int(x) for x in t],
                              "length": int(n)}
                             for t, n in zip(dec.tables, dec.lens)], 16)
    ek, ev = oa.store_kv(h_kc, h_vc, h_kn, h_vn,
                         list(mp["slot_mapping"]) + list(md["slot_mapping"]))
    width = max(len(t) for t in pre.tables)
    tables = [[int(x) for x in t] + [-1] * (width - len(t))
              for t in pre.tables]
    wantp = oa.prefill_attention(h_qp, ek, ev, mp["cu_seqlens_q"],
                                 mp["cu_seqlens_k"], tables, scale, True,
                                 "bf16", rows=rows)
    cu = mp["cu_seqlens_q"]
    sel = [cu[b] + i for b in rows for i in rows[b]]
    errp = float(np.max(np.abs(gotp[sel] - wantp[sel])))
    wantd = oa.decode_attention(h_qd, ek, ev, md["block_tables"],
                                md["context_lens"], scale, "bf16", seqs=seqs)
    errd = float(np.max(np.abs(gotd[seqs] - wantd[seqs])))
    tol = TOL["bf16"]
    return {"prefill_max_abs_err": errp, "prefill_rows_checked": len(sel),
            "decode_max_abs_err": errd, "decode_rows_checked": len(seqs),
            "tolerance": tol, "ok": bool(errp <= tol and errd <= tol)}


def cpu_baseline(case_tables, lens, h_q, h_kc, h_vc, hq, scale, budget_s):
    """Time the oracle on whole sequences until ~budget_s seconds pass."""
    import numpy as np
    import oracle.attention as oa
    import oracle.metadata as om
    order = np.random.default_rng(0).permutation(len(lens)).tolist()
    done, seqs_bytes, t0 = 0, 0, time.perf_counter()
    for b in order:
        meta = om.decode_metadata([{"block_table": [int(x) for x in
                                                    case_tables[b]],
                                    "length": int(lens[b])}], 16)
        oa.decode_attention(h_q[b:b + 1], h_kc, h_vc, meta["block_tables"],
                            meta["context_lens"], scale, "bf16")
        done += 1
        seqs_bytes += int(lens[b])
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return done, seqs_bytes, dt


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): "
              "the kernels have no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workloads as wl
    from paged_kv_cache_slot_amd import metadata as pm
    from paged_kv_cache_slot_amd import ops

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    cfg = wl.get_config(WORKLOAD)
    lay = wl.config_decode_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    b = len(lay.lens)
    elem = 2
    print(f"[bench] workload {cfg.title}; pool {lay.num_blocks} blocks",
          file=sys.stderr, flush=True)

    kc, vc = wl.fill_pool(lay.num_blocks, bs, hkv, d, "bf16", cfg.seed, dev)
    q = wl.make_values((b, hq, d), "bf16", cfg.seed + 1, dev)
    k_new = wl.make_values((b, hkv, d), "bf16", cfg.seed + 2, dev)
    v_new = wl.make_values((b, hkv, d), "bf16", cfg.seed + 3, dev)
    meta = pm.decode_inputs(lay.tables, lay.lens, bs)
    slot = torch.as_tensor(meta["slot_mapping"], device=dev)
    bt = torch.as_tensor(meta["block_tables"], device=dev)
    cl = torch.as_tensor(meta["context_lens"], device=dev)
    maxlen = meta["max_context_len"]
    scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q)
    ws_bytes = ops.decode_workspace_bytes(b, hq, hkv, d, maxlen)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    # Host copies of the inputs, taken before any kernel runs: the oracle
    # check and the CPU baseline read these.
    keep_host = not (args.no_check and args.no_cpu_baseline)
    host = [wl.host_bits(x) for x in (q, kc, vc, k_new, v_new)] \
        if keep_host else None

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ops.store_kv(k_new, v_new, kc, vc, slot)
        if ev is not None:
            ev[1].record()
        ops.decode(q, kc, vc, bt, cl, maxlen, scale=scale, out=out,
                   workspace=ws)
        if ev is not None:
            ev[2].record()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flush = Flusher(args.flush_mb, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
              for _ in range(args.steps)]
    # Timed region: exactly `steps` steps between two synchronisations; each
    # step's own events exclude the cache flush written before it.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        flush()
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_all = [e[0].elapsed_time(e[2]) for e in events]
    dec_all = [e[1].elapsed_time(e[2]) for e in events]
    step_stats = stats_ms(step_all)
    dec_stats = stats_ms(dec_all)
    step_ms = step_stats["median"]
    dec_ms_avg = dec_stats["median"]

    dbytes = decode_bytes(lay.lens, hq, hkv, d, elem)
    row = 2 * hkv * d * elem
    sbytes = 2 * b * row + 4 * b
    step_bytes = dbytes + sbytes
    value_tbs = step_bytes / (step_ms * 1e-3) / 1e12
    dec_gbs = dbytes / (dec_ms_avg * 1e-3) / 1e9

    traffic = committed_traffic("decode_8b_step_hbm_counters.md",
                                DECODE_SOURCES)

    check = None
    if not args.no_check:
        check = cpu_check_decode(lay.tables, lay.lens, *host, f64(out), scale,
                                 "bf16", sample_sequences(lay.lens, 8, 3))

    # The other workloads get their own pools: free the 8B-shaped one first
    # (the mixed pool is ~3.5 GB).
    del kc, vc, ws
    torch.cuda.empty_cache()
    chk = not args.no_check
    mixed = None
    if args.mixed_steps > 0:
        mixed = run_mixed(args.mixed_steps, max(2, args.warmup // 2), dev,
                          flush, 0.0 if args.no_cpu_baseline
                          else args.cpu_seconds / 3, chk)
        torch.cuda.empty_cache()
    prefix = None
    if args.prefix_steps > 0:
        prefix = run_prefix(args.prefix_steps, max(2, args.warmup // 2), dev,
                            flush, 0.0 if args.no_cpu_baseline
                            else args.cpu_seconds / 3, chk)
        torch.cuda.empty_cache()
    tiny = None
    if args.tiny_steps > 0:
        tiny = run_tiny(args.tiny_steps, max(2, args.warmup // 2), dev, flush,
                        chk)
    small = None
    if args.small_steps > 0:
        small = run_small(args.small_steps, max(2, args.warmup // 2), dev,
                          flush, 0.0 if args.no_cpu_baseline
                          else args.cpu_seconds / 3, chk)
        torch.cuda.empty_cache()
    fp8 = None
    if args.fp8_steps > 0:
        fp8 = run_fp8(args.fp8_steps, max(2, args.warmup // 2), dev, flush,
                      chk)
        torch.cuda.empty_cache()
    verify = None
    if args.verify_steps > 0:
        verify = run_verify(args.verify_steps, max(2, args.warmup // 2), dev,
                            flush, chk)
        torch.cuda.empty_cache()
    indirection = None
    if args.indirection_steps > 0:
        indirection = run_indirection(args.indirection_steps,
                                      max(2, args.warmup // 2), dev, flush)
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        # bounded oracle sample over host copies of the same pool
        done, toks, dt = cpu_baseline(lay.tables, lay.lens, host[0], host[1],
                                      host[2], hq, scale, args.cpu_seconds)
        cpu_bytes = toks * row
        cores = len(os.sched_getaffinity(0))
        cpu = {"value": cpu_bytes / dt / 1e12, "unit": "TB/s",
               "cores": cores, "kind": "oracle",
               "tokens_per_s": done / dt,
               "sample": f"{done} of {b} sequences ({toks} context tokens), "
                         f"fp64 numpy oracle, {dt:.1f} s"}

    line = {
        "metric": "paged decode attention achieved HBM TB/s (% of peak) + "
                  "decode tokens/s",
        "value": round(value_tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.title, "num_seqs": b,
                   "context_lens": "uniform [512, 8192], seed 3",
                   "heads_q_kv": [hq, hkv], "head_dim": d, "block_size": bs,
                   "pool_blocks": lay.num_blocks},
        "tokens_per_s": round(b / (step_ms * 1e-3), 1),
        "frac_of_hbm_peak": round(value_tbs * 1e3 / HBM_PEAK_GBS, 4),
        "decode_ms": round(dec_ms_avg, 4),
        "step_ms_stats": step_stats,
        "decode_ms_stats": dec_stats,
        "flush_mb_between_steps": args.flush_mb,
        "roofline": {"kernel": "pa_decode (large bf16 batch: verify_plan_kernel "
                               "+ verify_kernel, one query row per sequence, "
                               "two KV heads per work item)",
                     "bound": "hbm", "achieved": round(dec_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes": dbytes},
        "cpu_baseline": cpu,
        "check": check,
        "mixed_step": mixed,
        "prefix_step": prefix,
        "tiny_step": tiny,
        "small_step": small,
        "fp8_step": fp8,
        "verify_step": verify,
        "indirection_step": indirection,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
