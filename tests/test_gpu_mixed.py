"""The mixed chunked-prefill + decode step at full size, run exactly as the
benchmark runs it, against the oracle.

One pa_store_kv writes every new row of the step (8 x 512 chunk rows and 192
decode rows) into one shared pool; then pa_prefill_varlen attends the chunks
and pa_decode the 192 decode rows ("10 Serving Engines", section 10.3:
chunked prefill puts prompt chunks and decode rows in one step;
"3.6 ModelRunner, CUDA Graph, and benchmarks", section 2: prepare_prefill
and prepare_decode).  The decode rows are also run through pa_prefill_varlen
as one-row causal chunks: a one-row chunk at the end of its context is a
decode.  Every slot no sequence keeps is NaN."""

import math

import numpy as np
import pytest
import torch

import oracle.attention as oa
import oracle.metadata as om
import workloads as wl
from paged_kv_cache_slot_amd import metadata as pm
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import TOL, bits_equal, dev_i32, f64, sample_seqs, say

pytestmark = pytest.mark.gpu


def test_mixed_step_full_size():
    cfg = wl.get_config("mixed")
    pre, dec = wl.mixed_layout(cfg)
    hq, hkv, d, bs = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, 16
    say("mixed step full size: store 4288 rows, prefill, decode 192 rows")
    dev = "cuda"
    kc, vc = wl.fill_pool(pre.num_blocks, bs, hkv, d, "bf16", cfg.seed, dev)
    tables = list(pre.tables) + list(dec.tables)
    lens = np.concatenate([pre.history + pre.chunk, dec.lens])
    wl.poison_unused(kc, vc, wl.valid_slot_mask(pre.num_blocks, bs, tables,
                                                lens))
    tq = int(pre.chunk.sum())
    nd = len(dec.lens)
    qp = wl.make_values((tq, hq, d), "bf16", cfg.seed + 1, dev)
    qd = wl.make_values((nd, hq, d), "bf16", cfg.seed + 2, dev)
    k_new = wl.make_values((tq + nd, hkv, d), "bf16", cfg.seed + 3, dev)
    v_new = wl.make_values((tq + nd, hkv, d), "bf16", cfg.seed + 4, dev)
    h_kc, h_vc = wl.host_bits(kc), wl.host_bits(vc)
    h_qp, h_qd = wl.host_bits(qp), wl.host_bits(qd)
    h_kn, h_vn = wl.host_bits(k_new), wl.host_bits(v_new)

    # HIP path: the package's metadata, one store, prefill, decode
    mp = pm.prefill_inputs(pre.tables, pre.history, pre.chunk, bs)
    md = pm.decode_inputs(dec.tables, dec.lens, bs)
    slots = dev_i32(np.concatenate([mp["slot_mapping"], md["slot_mapping"]]))
    scale = 1.0 / math.sqrt(d)
    ops.store_kv(k_new, v_new, kc, vc, slots)
    outp = ops.prefill_varlen(qp, kc, vc, dev_i32(mp["cu_seqlens_q"]),
                              dev_i32(mp["cu_seqlens_k"]), mp["max_seqlen_q"],
                              mp["max_seqlen_k"], dev_i32(mp["block_tables"]),
                              scale=scale, causal=True)
    outd = ops.decode(qd, kc, vc, dev_i32(md["block_tables"]),
                      dev_i32(md["context_lens"]), md["max_context_len"],
                      scale=scale)
    # the same decode rows as one-row causal chunks over their contexts
    m1 = pm.prefill_inputs(dec.tables, dec.lens - 1,
                           np.ones(nd, dtype=np.int64), bs)
    outd1 = ops.prefill_varlen(qd, kc, vc, dev_i32(m1["cu_seqlens_q"]),
                               dev_i32(m1["cu_seqlens_k"]), m1["max_seqlen_q"],
                               m1["max_seqlen_k"], dev_i32(m1["block_tables"]),
                               scale=scale, causal=True)
    torch.cuda.synchronize()

    # oracle: its own metadata, store, gather and softmax
    o_pre = om.prefill_metadata(
        [{"block_table": [int(x) for x in t], "num_cached": int(h),
          "num_scheduled": int(c)}
         for t, h, c in zip(pre.tables, pre.history, pre.chunk)], bs)
    o_dec = om.decode_metadata(
        [{"block_table": [int(x) for x in t], "length": int(n)}
         for t, n in zip(dec.tables, dec.lens)], bs)
    ek, ev = oa.store_kv(h_kc, h_vc, h_kn, h_vn,
                         list(o_pre["slot_mapping"]) +
                         list(o_dec["slot_mapping"]))
    assert bits_equal(wl.host_bits(kc), ek), "K cache differs after the store"
    assert bits_equal(wl.host_bits(vc), ev), "V cache differs after the store"

    seqs = sample_seqs(dec.lens, 14, seed=55)
    want = oa.decode_attention(h_qd, ek, ev, o_dec["block_tables"],
                               o_dec["context_lens"], scale, "bf16",
                               seqs=seqs)
    for name, out in (("pa_decode", outd), ("pa_prefill_varlen Lq=1", outd1)):
        got = f64(out)
        assert np.all(np.isfinite(got)), name
        err = float(np.max(np.abs(got[seqs] - want[seqs])))
        say(f"{name}: decode rows {seqs} max abs err {err:.3e}")
        assert err <= TOL["bf16"], (name, err)

    # a few rows of every chunk of the same step
    width = max(len(t) for t in pre.tables)
    ptab = [[int(x) for x in t] + [-1] * (width - len(t)) for t in pre.tables]
    rows = {b: [0, 255, 511] for b in range(len(pre.chunk))}
    wantp = oa.prefill_attention(h_qp, ek, ev, o_pre["cu_seqlens_q"],
                                 o_pre["cu_seqlens_k"], ptab, scale, True,
                                 "bf16", rows=rows)
    cu = o_pre["cu_seqlens_q"]
    sel = np.asarray([cu[b] + i for b in rows for i in rows[b]])
    gotp = f64(outp)
    assert np.all(np.isfinite(gotp[sel]))
    err = float(np.max(np.abs(gotp[sel] - wantp[sel])))
    assert err <= TOL["bf16"], err
