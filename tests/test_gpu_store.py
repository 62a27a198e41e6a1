"""pa_store_kv on the GPU against the oracle's scatter: bit-exact."""

import numpy as np
import pytest
import torch

import oracle.attention as oa
import workloads as wl
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import bits_equal, dev_i32, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,hkv,d,nb,t", [
    ("f32", 2, 64, 64, 4),
    ("bf16", 8, 128, 300, 256),
    ("bf16", 1, 64, 50, 333),
    ("f32", 8, 128, 40, 97),
    ("bf16", 8, 128, 2000, 4288),
])
def test_store_bit_exact(dtype, hkv, d, nb, t):
    say("store", dtype, hkv, d, nb, t)
    bs = 16
    rng = np.random.default_rng(nb + t)
    kc, vc = wl.fill_pool(nb, bs, hkv, d, dtype, seed=t, device="cuda")
    k = wl.make_values((t, hkv, d), dtype, seed=t + 1, device="cuda")
    v = wl.make_values((t, hkv, d), dtype, seed=t + 2, device="cuda")
    slots = rng.permutation(nb * bs)[:t].astype(np.int64)
    slots[rng.random(t) < 0.1] = -1          # batch padding rows
    h = [wl.host_bits(x) for x in (kc, vc, k, v)]
    ops.store_kv(k, v, kc, vc, dev_i32(slots))
    torch.cuda.synchronize()
    ek, ev = oa.store_kv(h[0], h[1], h[2], h[3], slots)
    assert bits_equal(wl.host_bits(kc), ek)
    assert bits_equal(wl.host_bits(vc), ev)


def test_store_all_padding_and_empty():
    say("store padding-only / empty")
    kc, vc = wl.fill_pool(8, 16, 2, 64, "bf16", seed=9, device="cuda")
    before = wl.host_bits(kc).copy()
    k = wl.make_values((5, 2, 64), "bf16", seed=1, device="cuda")
    ops.store_kv(k, k, kc, vc, dev_i32([-1] * 5))
    empty = k[:0]
    ops.store_kv(empty, empty, kc, vc, dev_i32([]))
    torch.cuda.synchronize()
    assert bits_equal(wl.host_bits(kc), before)


def test_store_slot_past_pool_is_skipped():
    """A slot at or beyond num_slots violates the precondition; the kernel
    skips it rather than writing outside the cache."""
    say("store out-of-range slot")
    kc, vc = wl.fill_pool(4, 16, 2, 64, "f32", seed=2, device="cuda")
    guard = torch.full((4096,), 7.0, device="cuda")
    before = wl.host_bits(kc).copy()
    k = wl.make_values((2, 2, 64), "f32", seed=3, device="cuda")
    ops.store_kv(k, k, kc, vc, dev_i32([64, 1 << 30]))
    torch.cuda.synchronize()
    assert bits_equal(wl.host_bits(kc), before)
    assert torch.all(guard == 7.0)
