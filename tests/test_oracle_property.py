"""Property sweep: the numpy oracle equals the pure-Python brute force on
random tiny shapes (block sizes 1-16, contexts 1-70, GQA ratios 1-4, head
dims 8 and 64, both element types)."""

import math

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle.attention as oa
from tests import brute_force as bf
from tests.oracle_pins import _bf16_bits


@settings(max_examples=25, deadline=None)
@given(bs=st.sampled_from([1, 2, 4, 16]),
       ratio=st.sampled_from([1, 2, 4]),
       hkv=st.sampled_from([1, 2]),
       d=st.sampled_from([8, 64]),
       lens=st.lists(st.integers(0, 70), min_size=1, max_size=3),
       dtype=st.sampled_from(["f32", "bf16"]),
       seed=st.integers(0, 2 ** 31 - 1))
def test_decode_matches_brute(bs, ratio, hkv, d, lens, dtype, seed):
    rng = np.random.default_rng(seed)
    hq = hkv * ratio
    need = sum(-(-n // bs) for n in lens)
    nb = need + 2
    k = rng.standard_normal((nb, bs, hkv, d)).astype(np.float32)
    v = rng.standard_normal((nb, bs, hkv, d)).astype(np.float32)
    q = rng.standard_normal((len(lens), hq, d)).astype(np.float32)
    if dtype == "bf16":
        k, v, q = _bf16_bits(k), _bf16_bits(v), _bf16_bits(q)
    perm = [int(x) for x in rng.permutation(nb)]
    width = max(1, max(-(-n // bs) for n in lens))
    tables, pos = [], 0
    for n in lens:
        c = -(-n // bs)
        tables.append(perm[pos:pos + c] + [-1] * (width - c))
        pos += c
    scale = 1.0 / math.sqrt(d)
    got = oa.decode_attention(q, k, v, tables, lens, scale, dtype)
    want = bf.brute_decode(oa.to_f64(q, dtype).tolist(),
                           oa.to_f64(k, dtype).tolist(),
                           oa.to_f64(v, dtype).tolist(), tables, lens, scale)
    assert np.max(np.abs(got - np.array(want))) < 1e-12
