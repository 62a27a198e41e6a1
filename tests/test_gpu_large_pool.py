"""Cache pools past 4 GiB: every block a case uses sits above the 4 GiB mark
of its cache, so each kernel forms byte offsets beyond 2^32 (block id times
block bytes, slot times row bytes).  A small case's pool is copied into the
top of a large pool; the HIP path runs on the large pool with its block ids
and slots shifted by the offset, the oracle on the small pool's host copy
with the original ids.  Only the used top of the large pool is read back."""

import numpy as np
import pytest
import torch

import oracle.attention as oa
import workloads as wl
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import (TOL, DecodeCase, PrefillCase, bits_equal,
                               dev_i32, f64, say)

pytestmark = pytest.mark.gpu

# bf16 with 8 KV heads of 128: 32 KiB per block, so 140,000 blocks put the
# first used block 4.59 GB (> 2^32 bytes) into each cache.
OFF = 140_000


def _shift(a, off):
    a = np.asarray(a, dtype=np.int64)
    return np.where(a >= 0, a + off, a)


def _big_pool(small, off):
    """A pool of off + len(small) blocks whose top holds ``small``; the
    blocks below are never referenced and stay uninitialised."""
    big = torch.empty((off + small.shape[0],) + tuple(small.shape[1:]),
                      dtype=small.dtype, device=small.device)
    big[off:].copy_(small)
    assert off * small[0].numel() * small.element_size() > (1 << 32)
    return big


def test_decode_above_4gib():
    rng = np.random.default_rng(9300)
    lens = rng.integers(1, 3000, 12, endpoint=True).tolist()
    lens[0] = 3000
    say("decode, pool past 4 GiB", lens)
    case = DecodeCase(wl.decode_layout(lens, 16, seed=9301), 32, 8, 128,
                      "bf16", seed=9302)
    kc, vc = _big_pool(case.kc, OFF), _big_pool(case.vc, OFF)
    case.kc = case.vc = None
    slots = dev_i32(_shift(case.meta["slot_mapping"], OFF * case.bs))
    bt = dev_i32(_shift(case.meta["block_tables"], OFF))
    ops.store_kv(case.k_new, case.v_new, kc, vc, slots)
    out = ops.decode(case.q, kc, vc, bt, case.context_lens,
                     case.max_context_len, scale=case.scale)
    torch.cuda.synchronize()
    ek, ev = case.oracle_store()
    assert bits_equal(wl.host_bits(kc[OFF:]), ek), "store mismatch (K)"
    assert bits_equal(wl.host_bits(vc[OFF:]), ev), "store mismatch (V)"
    want = case.oracle_decode(ek, ev)
    got = f64(out)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL["bf16"], f"max abs err {err}"


def test_prefill_above_4gib():
    say("chunked prefill, pool past 4 GiB")
    lay = wl.prefill_layout([700, 0, 1500, 33], [130, 257, 64, 1], 16,
                            seed=9311)
    case = PrefillCase(lay, 32, 8, 128, "bf16", seed=9312)
    kc, vc = _big_pool(case.kc, OFF), _big_pool(case.vc, OFF)
    case.kc = case.vc = None
    m = case.meta
    slots = dev_i32(_shift(m["slot_mapping"], OFF * case.bs))
    bt = dev_i32(_shift(m["block_tables"], OFF))
    ops.store_kv(case.k_new, case.v_new, kc, vc, slots)
    out = ops.prefill_varlen(case.q, kc, vc, case.cu_q, case.cu_k,
                             m["max_seqlen_q"], m["max_seqlen_k"], bt,
                             scale=case.scale, causal=True)
    torch.cuda.synchronize()
    ek, ev = case.oracle_store()
    assert bits_equal(wl.host_bits(kc[OFF:]), ek), "store mismatch (K)"
    assert bits_equal(wl.host_bits(vc[OFF:]), ev), "store mismatch (V)"
    want = case.oracle_prefill(ek, ev)
    got = f64(out)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL["bf16"], f"max abs err {err}"


def test_copy_blocks_above_4gib():
    say("copy_blocks, pool past 4 GiB")
    nb = 64
    kc_s, vc_s = wl.fill_pool(nb, 16, 8, 128, "bf16", 9321, "cuda")
    h_k, h_v = wl.host_bits(kc_s).copy(), wl.host_bits(vc_s).copy()
    kc, vc = _big_pool(kc_s, OFF), _big_pool(vc_s, OFF)
    del kc_s, vc_s
    pairs = np.array([[0, 63], [5, 6], [40, 1], [7, 7], [nb + 3, 2]],
                     dtype=np.int64)
    # the last pair names a block past the small pool: shifted, it is past
    # the large pool too, so both sides skip it
    ops.copy_blocks(kc, vc, dev_i32(pairs + OFF))
    torch.cuda.synchronize()
    ek, ev = oa.copy_blocks(h_k, h_v, pairs)
    assert bits_equal(wl.host_bits(kc[OFF:]), ek)
    assert bits_equal(wl.host_bits(vc[OFF:]), ev)


def test_fp8_decode_above_4gib():
    """8-bit cache: 16 KiB per block, so the offset doubles to stay past
    2^32 bytes."""
    import math

    import oracle.fp8 as of8
    from paged_kv_cache_slot_amd import metadata as pm
    from tests.test_gpu_fp8 import _poison
    off8 = 2 * OFF
    lens = [3000, 1, 17, 513, 2048, 999]
    say("fp8 decode, pool past 4 GiB", lens)
    lay = wl.decode_layout(lens, 16, seed=9331)
    kc_s, vc_s = wl.fill_pool_codes(lay.num_blocks, 16, 8, 128, 9332, "cuda")
    _poison(kc_s, vc_s, lay.tables, lay.lens, lay.num_blocks, 16)
    h_k, h_v = wl.host_bits(kc_s).copy(), wl.host_bits(vc_s).copy()
    kc, vc = _big_pool(kc_s, off8), _big_pool(vc_s, off8)
    del kc_s, vc_s
    q = wl.make_values((len(lens), 32, 128), "bf16", 9333, "cuda")
    meta = pm.decode_inputs(lay.tables, lay.lens, 16)
    scale = 1.0 / math.sqrt(128)
    out = ops.decode_fp8(q, kc, vc, dev_i32(_shift(meta["block_tables"], off8)),
                         dev_i32(meta["context_lens"]), meta["max_context_len"],
                         1 / 16, 1 / 8, scale=scale)
    torch.cuda.synchronize()
    want = of8.decode_attention(wl.host_bits(q), h_k, h_v,
                                meta["block_tables"], meta["context_lens"],
                                scale, 1 / 16, 1 / 8, "bf16")
    got = f64(out)
    assert np.all(np.isfinite(got))
    err = float(np.max(np.abs(got - want)))
    assert err <= TOL["bf16"], f"max abs err {err}"
