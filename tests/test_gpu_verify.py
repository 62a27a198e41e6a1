"""The small-row path of pa_prefill_varlen against the oracle.

A speculative-decoding verify pass runs the target model once over the k
proposed positions of every sequence ("Warmup Guide -- Inference Serving
Internals", Chapter 7, the scheme; "10 Serving Engines", sections 10.6.1 and
10.6.2): Lq = k + 1 causal rows per sequence over a long paged context.
With bfloat16 and at most 64 packed rows per KV head (G * max Lq) the
library takes a split-context MFMA path for these launches; every test here
is sized to take it (its workspace size says which partitioning it chose).

All slots outside any sequence's context are NaN, so a read past Lk or a
mask applied by multiplication shows up as a non-finite output."""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oa
import workloads as wl
from paged_kv_cache_slot_amd import metadata as pm
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import (TOL, PrefillCase, bits_equal, dev_i32, f64,
                               sample_seqs, say)

pytestmark = pytest.mark.gpu


def _check(case, seqs=None):
    case.run_store()
    out = case.run_prefill()
    torch.cuda.synchronize()
    ek, ev = case.oracle_store()
    assert bits_equal(wl.host_bits(case.kc), ek), "store mismatch"
    want = case.oracle_prefill(ek, ev, seqs=seqs)
    got = f64(out)
    cu = case.meta["cu_seqlens_q"]
    bs = range(len(cu) - 1) if seqs is None else seqs
    sel = np.asarray([r for b in bs for r in range(cu[b], cu[b + 1])],
                     dtype=np.int64)
    assert np.all(np.isfinite(got[sel]))
    err = float(np.max(np.abs(got[sel] - want[sel]))) if len(sel) else 0.0
    assert err <= TOL[case.dtype], f"max abs err {err}"
    return got, want


def _layout(hist, lq, seed, num_blocks=None):
    return wl.prefill_layout(np.asarray(hist), np.asarray(lq), 16, seed=seed,
                             num_blocks=num_blocks)


@pytest.mark.parametrize("lq", [2, 4, 8])
def test_verify_8b_step_full_size(lq):
    """The 8B-shaped verify step: 256 sequences with contexts U[512, 8192]
    (the last Lq tokens are the proposed ones), 32 query / 8 KV heads,
    D = 128; one launch over the whole batch, 14 sequences (longest,
    shortest, random) checked row by row."""
    cfg = wl.get_config("decode8b")
    lay = wl.config_decode_layout(cfg)
    hq, hkv, d = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    b = len(lay.lens)
    say(f"verify 8B step full size, Lq={lq}")
    dev = "cuda"
    kc, vc = wl.fill_pool(lay.num_blocks, 16, hkv, d, "bf16", cfg.seed, dev)
    wl.poison_unused(kc, vc, wl.valid_slot_mask(lay.num_blocks, 16, lay.tables,
                                                lay.lens))
    q = wl.make_values((b * lq, hq, d), "bf16", cfg.seed + 7, dev)
    hist = lay.lens - lq
    meta = pm.prefill_inputs(lay.tables, hist, np.full(b, lq), 16)
    scale = 1.0 / math.sqrt(d)
    h_kc, h_vc, h_q = wl.host_bits(kc), wl.host_bits(vc), wl.host_bits(q)
    out = ops.prefill_varlen(q, kc, vc, dev_i32(meta["cu_seqlens_q"]),
                             dev_i32(meta["cu_seqlens_k"]), meta["max_seqlen_q"],
                             meta["max_seqlen_k"], dev_i32(meta["block_tables"]),
                             scale=scale, causal=True)
    torch.cuda.synchronize()
    seqs = sample_seqs(lay.lens, 14, seed=lq + 70)
    width = max(len(t) for t in lay.tables)
    tables = [[int(x) for x in t] + [-1] * (width - len(t)) for t in lay.tables]
    cu_q = np.concatenate([[0], np.cumsum(np.full(b, lq))])
    cu_k = np.concatenate([[0], np.cumsum(lay.lens)])
    want = oa.prefill_attention(h_q, h_kc, h_vc, cu_q, cu_k, tables, scale, True,
                                "bf16", seqs=seqs)
    got = f64(out)
    sel = np.asarray([r for s in seqs for r in range(cu_q[s], cu_q[s + 1])])
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got[sel] - want[sel])))
    say(f"verify Lq={lq}: sequences {seqs} max abs err {err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("lq", [3, 8])
def test_verify_split_context(lq):
    """Three sequences over 5K-20K keys: too few (sequence, KV head) pairs
    to fill the chip, so the keys are split into partitions whose partials a
    merge kernel combines -- rows whose causal limit falls in different
    partitions included."""
    say("verify split context", lq)
    hist = [20000 - lq, 5003, 12345]
    lay = _layout(hist, [lq] * 3, seed=91)
    case = PrefillCase(lay, 32, 8, 128, "bf16", seed=92)
    m = case.meta
    need = ops.prefill_workspace_bytes(3, 32, 8, 128, m["max_seqlen_q"],
                                       m["max_seqlen_k"])
    assert need > 4096, "partials in the workspace"
    _check(case)


@pytest.mark.parametrize("d,hq,hkv,lq,n", [
    (128, 64, 8, 8, 24),     # G = 8: 64 rows, four row tiles
    (128, 64, 8, 8, 160),    # the same with one partition per sequence
    (128, 8, 8, 50, 24),     # G = 1: 50 rows of one head, padded to 64
    (128, 16, 16, 16, 24),   # G = 1: exactly one row tile
    (128, 32, 8, 1, 24),     # one row per sequence (a decode row)
    (64, 16, 8, 5, 24),      # D = 64, G = 2: 10 rows
    (64, 16, 8, 5, 160),     # the same with one partition per sequence
    (64, 32, 4, 8, 24),      # D = 64, G = 8: 64 rows
    (64, 8, 8, 20, 160),     # D = 64, G = 1: 20 rows, two row tiles
])
def test_verify_shapes(d, hq, hkv, lq, n):
    """Every row-tile count and both head sizes, with ragged rows: Lq from 1
    to the maximum per sequence, histories from 0 (Lk = Lq) to 3,000 keys,
    blocks ending mid-block.  24 sequences split their keys into partitions
    (merged); 160 sequences x 8 KV heads fill the chip with one partition
    each (sampled sequences checked)."""
    say("verify shapes", d, hq, hkv, lq, n)
    rng = np.random.default_rng(d * 1000 + hq + lq + n)
    chunk = rng.integers(1, lq + 1, n)
    chunk[0] = lq
    hist = rng.integers(0, 3000, n)
    hist[1] = 0
    hist[2] = 16 - chunk[2] % 16 + 32
    lay = _layout(hist, chunk, seed=93 + lq)
    seqs = None if n <= 24 else sample_seqs(hist + chunk, 16, seed=lq)
    _check(PrefillCase(lay, hq, hkv, d, "bf16", seed=94 + lq), seqs=seqs)


def test_verify_empty_rows_and_short_contexts():
    """Sequences with no query rows in the batch, contexts shorter than a
    block, and a one-token context."""
    say("verify empty rows")
    hist = [0, 7, 0, 300, 2, 40]
    chunk = [1, 4, 0, 6, 0, 3]
    lay = _layout(hist, chunk, seed=95)
    _check(PrefillCase(lay, 32, 8, 128, "bf16", seed=96))


def test_verify_non_causal():
    """Without the causal mask every row sees all Lk keys."""
    say("verify non-causal")
    lay = _layout([100, 2000, 5], [4, 8, 2], seed=97)
    _check(PrefillCase(lay, 32, 8, 128, "bf16", seed=98, causal=False))


def test_verify_large_values_in_partials():
    """V scaled by 2^20: outputs past the binary16 range, so the merged
    partials must take the scaled (flagged) form; the error is judged
    relative to the largest output."""
    say("verify large values")
    lay = _layout([9000, 3000, 700], [4, 4, 4], seed=99)
    case = PrefillCase(lay, 32, 8, 128, "bf16", seed=100)
    case.run_store()
    factor = float(2 ** 20)
    case.vc.mul_(factor)
    case.h_vc = wl.host_bits(case.vc)
    case.v_new.mul_(factor)
    case.h_vn = wl.host_bits(case.v_new)
    out = case.run_prefill()
    torch.cuda.synchronize()
    ek, ev = case.oracle_store()
    want = case.oracle_prefill(ek, ev)
    got = f64(out)
    top = float(np.max(np.abs(want)))
    assert top > 65504.0
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    assert err <= top * 2.0 ** -7, (err, top)


def _blocks(lk, part_tokens):
    return [-(-min(k, part_tokens) // 16) for k in lk]


def test_verify_plan_kernel_order():
    """More work items than one workgroup has threads (300 sequences): a
    plan kernel writes the longest-first schedule into the workspace (filled
    with garbage beforehand); it lists every sequence once, by
    non-increasing key blocks, and the result matches the oracle on sampled
    sequences."""
    say("verify plan kernel")
    rng = np.random.default_rng(101)
    n = 300
    hist = rng.integers(0, 2500, n)
    lay = _layout(hist, [4] * n, seed=102)
    case = PrefillCase(lay, 32, 8, 128, "bf16", seed=103)
    m = case.meta
    need = ops.prefill_workspace_bytes(n, 32, 8, 128, m["max_seqlen_q"],
                                       m["max_seqlen_k"])
    assert need >= 4 * n
    ws = torch.full((need // 4,), -7, dtype=torch.int32, device="cuda")
    case.run_store()
    out = case.run_prefill(workspace=ws)
    torch.cuda.synchronize()
    ek, ev = case.oracle_store()
    seqs = sample_seqs(hist + 4, 12, seed=104)
    want = case.oracle_prefill(ek, ev, seqs=seqs)
    got = f64(out)
    cu = m["cu_seqlens_q"]
    sel = np.asarray([r for b in seqs for r in range(cu[b], cu[b + 1])])
    assert np.all(np.isfinite(got))
    assert np.max(np.abs(got[sel] - want[sel])) <= TOL["bf16"]
    order = ws.cpu().numpy()[:n]
    assert sorted(order.tolist()) == list(range(n))
    w = np.asarray(_blocks(hist + 4, 1 << 30))
    assert np.all(np.diff(np.minimum(w[order], 1023)) <= 0)


def test_verify_workspace_garbage_and_repeat():
    """The plan kernel rewrites the schedule and zeroes the ticket counter
    on every call: a workspace full of garbage beforehand, or left by the
    previous call, gives the same bits, and the output (NaN beforehand)
    matches the oracle on sampled sequences."""
    say("verify workspace reuse")
    rng = np.random.default_rng(105)
    hist = rng.integers(0, 9000, 200)
    lay = _layout(hist, [5] * 200, seed=106)
    case = PrefillCase(lay, 16, 8, 128, "bf16", seed=107)
    m = case.meta
    need = ops.prefill_workspace_bytes(200, 16, 8, 128, m["max_seqlen_q"],
                                       m["max_seqlen_k"])
    ws = torch.full((need // 4,), -7, dtype=torch.int32, device="cuda")
    case.run_store()
    out = torch.full_like(case.q, float("nan"))
    case.run_prefill(out=out, workspace=ws)
    torch.cuda.synchronize()
    ek, ev = case.oracle_store()
    seqs = sample_seqs(hist, 10, seed=108)
    want = case.oracle_prefill(ek, ev, seqs=seqs)
    got = f64(out)
    assert np.all(np.isfinite(got))
    cu = m["cu_seqlens_q"]
    sel = np.asarray([r for b in seqs for r in range(cu[b], cu[b + 1])])
    assert np.max(np.abs(got[sel] - want[sel])) <= TOL["bf16"]
    again = case.run_prefill(workspace=ws)
    ws.fill_(0x7fffffff)
    third = case.run_prefill(workspace=ws)
    torch.cuda.synchronize()
    assert bits_equal(wl.host_bits(out), wl.host_bits(again))
    assert bits_equal(wl.host_bits(out), wl.host_bits(third))
