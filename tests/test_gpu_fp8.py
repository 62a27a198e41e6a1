"""8-bit (E4M3) KV cache on the GPU against the oracle: the quantising store
byte for byte, and decode over E4M3 caches within the bf16 tolerance.

Cache codes are drawn by the workload generator (never produced by the GPU
store for the oracle's use); slots outside every context hold the NaN code,
so a read past a context shows up as a non-finite output."""

import math

import numpy as np
import pytest
import torch

import oracle.fp8 as of8
import workloads as wl
from paged_kv_cache_slot_amd import metadata as pm
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import TOL, dev_i32, f64, sample_seqs, say

pytestmark = pytest.mark.gpu


def _inv(x):
    """1 / scale as the library computes it: one float32 division."""
    return float(np.float32(1.0) / np.float32(x))


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("k_scale,v_scale,gain", [
    (1.0, 1.0, 1.0), (0.0625, 0.37, 30.0), (3.0, 1 / 256, 200.0),
])
def test_store_fp8_bit_exact(src, k_scale, v_scale, gain):
    """Random rows (some far past +-448 after scaling: saturation), slots in
    random order with padding (-1) and out-of-pool slots: the caches equal
    the oracle's quantising store byte for byte."""
    say("store fp8", src, k_scale, v_scale, gain)
    nb, bs, hkv, d, t = 40, 16, 4, 128, 300
    kc, vc = wl.fill_pool_codes(nb, bs, hkv, d, 81, "cuda")
    k = wl.make_values((t, hkv, d), src, 82)
    v = wl.make_values((t, hkv, d), src, 83)
    k = (k.float() * gain).to(k.dtype)
    v = (v.float() * gain * 0.5).to(v.dtype)
    rng = np.random.default_rng(84)
    slots = rng.permutation(nb * bs)[:t].astype(np.int64)
    slots[::17] = -1
    slots[5] = nb * bs + 3
    h_kc, h_vc = wl.host_bits(kc), wl.host_bits(vc)
    h_k, h_v = wl.host_bits(k), wl.host_bits(v)
    ops.store_kv_fp8(k.cuda(), v.cuda(), kc, vc, dev_i32(slots), k_scale,
                     v_scale)
    torch.cuda.synchronize()
    valid = [s if s < nb * bs else -1 for s in slots.tolist()]
    ek, ev = of8.store_kv(h_kc, h_vc, h_k, h_v, valid, _inv(k_scale),
                          _inv(v_scale), src)
    assert np.array_equal(wl.host_bits(kc), ek)
    assert np.array_equal(wl.host_bits(vc), ev)


def _poison(kc, vc, tables, lens, nb, bs):
    mask = wl.valid_slot_mask(nb, bs, tables, lens)
    bad = torch.as_tensor(~mask, device=kc.device)
    kc[bad] = 0x7F
    vc[bad] = 0x7F


def _decode_case(lens, hq, hkv, k_scale, v_scale, seed, seqs=None, lay=None,
                 abs_check=True):
    """Decode over an E4M3 pool against the oracle.  With abs_check the
    outputs must be within the absolute bf16 tolerance; returns (got, want)
    for the sequences compared."""
    bs, d = 16, 128
    if lay is None:
        lay = wl.decode_layout(lens, bs, seed=seed)
    kc, vc = wl.fill_pool_codes(lay.num_blocks, bs, hkv, d, seed + 1, "cuda")
    _poison(kc, vc, lay.tables, lay.lens, lay.num_blocks, bs)
    q = wl.make_values((len(lay.lens), hq, d), "bf16", seed + 2, "cuda")
    meta = pm.decode_inputs(lay.tables, lay.lens, bs)
    scale = 1.0 / math.sqrt(d)
    out = ops.decode_fp8(q, kc, vc, dev_i32(meta["block_tables"]),
                         dev_i32(meta["context_lens"]), meta["max_context_len"],
                         k_scale, v_scale, scale=scale)
    torch.cuda.synchronize()
    want = of8.decode_attention(wl.host_bits(q), wl.host_bits(kc),
                                wl.host_bits(vc), meta["block_tables"],
                                meta["context_lens"], scale, k_scale, v_scale,
                                "bf16", seqs=seqs)
    got = f64(out)
    rows = list(range(len(lay.lens))) if seqs is None else seqs
    assert np.all(np.isfinite(got[rows]))
    if abs_check:
        err = float(np.max(np.abs(got[rows] - want[rows])))
        assert err <= TOL["bf16"], f"max abs err {err}"
    return got[rows], want[rows]


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8), (16, 2)])
def test_decode_fp8_edges(hq, hkv):
    """Lengths at block and chunk edges, GQA ratios 1, 2, 4 and 8."""
    say("decode fp8 edges", hq, hkv)
    _decode_case([1, 15, 16, 17, 511, 512, 513, 1024, 1500], hq, hkv,
                 1 / 16, 1 / 8, seed=91)


def test_decode_fp8_scales_and_partitions():
    """Scales that are not powers of two, and contexts long enough for
    several partitions (partials and the merge)."""
    say("decode fp8 long")
    _decode_case([3000, 8192, 4097, 77, 6000, 12000], 32, 8, 0.0371, 0.153,
                 seed=93)


def test_decode_fp8_one_key_exact():
    """A one-token context returns code * v_scale exactly (bf16-rounded;
    with a power-of-two scale the value is exact in bf16)."""
    say("decode fp8 one key")
    got, want = _decode_case([1, 1, 1], 8, 2, 0.25, 0.5, seed=95)
    assert np.array_equal(got, want)


def test_decode_fp8_full_size_sampled():
    """The 8B-shaped decode step's shapes (256 sequences, contexts
    U[512, 8192], 32q/8kv) over an E4M3 pool; sampled rows."""
    cfg = wl.get_config("decode8b")
    say("decode fp8 full-size sampled")
    lay = wl.config_decode_layout(cfg)
    _decode_case(None, cfg.num_heads, cfg.num_kv_heads, 1 / 16, 1 / 16,
                 seed=cfg.seed, seqs=sample_seqs(lay.lens, 8, cfg.seed),
                 lay=lay)


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 8), (8, 8), (24, 3)])
def test_decode_fp8_large_batch(hq, hkv):
    """Batches with >= 1024 (sequence, KV head pair) work items run on the
    small-row attention kernel, which widens the codes to bfloat16 on their
    way to LDS: two KV heads per item where Hkv is even, one where it is
    odd (Hkv = 3, GQA 8).  Contexts from 1 to 3,000 tokens with block
    edges, a NaN-poisoned pool; one-token contexts return code * v_scale
    exactly (power-of-two scales)."""
    say("decode fp8 large batch", hq, hkv)
    per_seq = hkv // 2 if hkv % 2 == 0 else hkv
    n = -(-1024 // per_seq) + 3
    rng = np.random.default_rng(hq * 10 + hkv)
    lens = rng.integers(1, 3000, n, endpoint=True)
    lens[:9] = [1, 15, 16, 17, 511, 512, 513, 1024, 3000]
    lens[-1] = 1
    lay = wl.decode_layout(lens.tolist(), 16, seed=hq + hkv)
    seqs = sorted(set(range(9)) | {n - 1} |
                  set(sample_seqs(lens, 15, seed=hkv)))
    got, want = _decode_case(None, hq, hkv, 1 / 16, 1 / 8, seed=hq + 7,
                             seqs=seqs, lay=lay)
    one = [i for i, b in enumerate(seqs) if lens[b] == 1]
    assert one and np.array_equal(got[one], want[one])


@pytest.mark.parametrize("b,hkv,longest,part", [(192, 8, 8192, 4096),
                                                (100, 3, 12000, 3008)])
def test_decode_fp8_partitioned_small_row(b, hkv, longest, part):
    """8-bit caches on the small-row kernel with partitions of >= 2,048
    tokens (partials and a merge; v_scale reaches the output through both):
    contexts at partition and block edges, 1 token and the longest."""
    say("decode fp8 partitioned small-row", b, hkv)
    hq = 8 * hkv if hkv == 3 else 32
    rng = np.random.default_rng(b * 3 + hkv)
    lens = rng.integers(1, longest, b, endpoint=True)
    edges = [longest, 1, part - 1, part, part + 1, 2 * part + 5, 16, 17]
    lens[:len(edges)] = edges
    lay = wl.decode_layout(lens.tolist(), 16, seed=b + 11)
    seqs = sorted(set(range(len(edges))) | set(sample_seqs(lens, 8, seed=b)))
    _decode_case(None, hq, hkv, 0.0371, 0.153, seed=b + 13, seqs=seqs,
                 lay=lay)


def test_store_then_decode_fp8():
    """One decode step end to end: quantise each sequence's new row into its
    slot, then decode; both the caches and the outputs match the oracle's
    own store and decode."""
    say("store + decode fp8")
    bs, d, hq, hkv = 16, 128, 16, 4
    lay = wl.decode_layout([5, 16, 33, 700, 1200], bs, seed=97)
    kc, vc = wl.fill_pool_codes(lay.num_blocks, bs, hkv, d, 98, "cuda")
    q = wl.make_values((5, hq, d), "bf16", 99, "cuda")
    kn = wl.make_values((5, hkv, d), "bf16", 100, "cuda")
    vn = wl.make_values((5, hkv, d), "bf16", 101, "cuda")
    meta = pm.decode_inputs(lay.tables, lay.lens, bs)
    h = [wl.host_bits(x) for x in (kc, vc, q, kn, vn)]
    ks, vs = 1 / 32, 1 / 64
    ops.store_kv_fp8(kn, vn, kc, vc, dev_i32(meta["slot_mapping"]), ks, vs)
    out = ops.decode_fp8(q, kc, vc, dev_i32(meta["block_tables"]),
                         dev_i32(meta["context_lens"]), meta["max_context_len"],
                         ks, vs)
    torch.cuda.synchronize()
    ek, ev = of8.store_kv(h[0], h[1], h[3], h[4], meta["slot_mapping"],
                          _inv(ks), _inv(vs), "bf16")
    assert np.array_equal(wl.host_bits(kc), ek)
    assert np.array_equal(wl.host_bits(vc), ev)
    want = of8.decode_attention(h[2], ek, ev, meta["block_tables"],
                                meta["context_lens"], 1 / math.sqrt(d), ks, vs,
                                "bf16")
    err = float(np.max(np.abs(f64(out) - want)))
    assert err <= TOL["bf16"], err
