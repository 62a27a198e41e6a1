"""Seeded random sweep of shapes and lengths through store + decode and
store + chunked prefill on the GPU, each against the oracle.  Every case
draws its own dtype, head_dim, GQA ratio, batch size and lengths (decode:
empty contexts included; prefill: chunks with and without history, causal
or not), so combinations the hand-picked cases do not name are exercised
too.  Sizes stay small enough for the oracle to finish in seconds."""

import numpy as np
import pytest

import workloads as wl
from tests.gpu_harness import DecodeCase, PrefillCase, say
from tests.test_gpu_decode import _check as check_decode
from tests.test_gpu_prefill import _check as check_prefill

pytestmark = pytest.mark.gpu


def _shape(rng):
    dtype = str(rng.choice(["f32", "bf16"]))
    d = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    return dtype, d, g * hkv, hkv


@pytest.mark.parametrize("seed", range(20))
def test_random_decode(seed):
    rng = np.random.default_rng(7100 + seed)
    dtype, d, hq, hkv = _shape(rng)
    b = int(rng.integers(1, 33))
    lens = rng.integers(0, 2500, b, endpoint=True)
    lens[rng.random(b) < 0.1] = 0          # batch padding rows
    say("random decode", seed, dtype, d, hq, hkv, b)
    lay = wl.decode_layout(lens.tolist(), 16, seed=7200 + seed)
    check_decode(DecodeCase(lay, hq, hkv, d, dtype, seed=7300 + seed))


@pytest.mark.parametrize("seed", range(20))
def test_random_prefill(seed):
    rng = np.random.default_rng(7400 + seed)
    dtype, d, hq, hkv = _shape(rng)
    b = int(rng.integers(1, 9))
    hist = rng.integers(0, 900, b, endpoint=True)
    hist[rng.random(b) < 0.3] = 0          # chunks with no history
    chunk = rng.integers(1, 300, b, endpoint=True)
    causal = bool(rng.random() < 0.75)
    say("random prefill", seed, dtype, d, hq, hkv, b, causal)
    lay = wl.prefill_layout(hist.tolist(), chunk.tolist(), 16, seed=7500 + seed)
    check_prefill(PrefillCase(lay, hq, hkv, d, dtype, seed=7600 + seed,
                              causal=causal))


@pytest.mark.parametrize("seed", range(10))
def test_random_fp8_decode(seed):
    """8-bit (E4M3) cache: random GQA ratio, lengths and per-cache scales.
    k_scale spans two orders of magnitude (it only sharpens the softmax);
    v_scale keeps every dequantised V within +-2, where the absolute bf16
    tolerance is meaningful.  A second call with a v_scale 200 x larger
    checks the same outputs relative to their size: bf16 output rounding
    plus the fp32 sums, within 2^-7 of the largest output."""
    from tests.test_gpu_fp8 import _decode_case
    rng = np.random.default_rng(7700 + seed)
    g = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    b = int(rng.integers(1, 25))
    lens = rng.integers(1, 2500, b, endpoint=True).tolist()
    ks = float(rng.uniform(0.01, 2.0))
    vs = float(rng.uniform(0.1, 1.0)) * 2.0 / 448.0
    say("random fp8 decode", seed, g * hkv, hkv, b, ks, vs)
    _decode_case(lens, g * hkv, hkv, ks, vs, seed=7800 + seed)
    got, want = _decode_case(lens, g * hkv, hkv, ks, vs * 200.0,
                             seed=7800 + seed, abs_check=False)
    err = float(np.max(np.abs(got - want)))
    assert err <= 2.0 ** -7 * max(1.0, float(np.max(np.abs(want)))), err


@pytest.mark.parametrize("seed", range(10))
def test_random_shared_prefix(seed):
    """Shared-prefix decode: random runs of sequences sharing 1..24 leading
    blocks, independent sequences between them, random dtype and shape."""
    from tests.test_gpu_shared_prefix import _grouped_layout, _run
    rng = np.random.default_rng(7900 + seed)
    dtype, d, hq, hkv = _shape(rng)
    spec, groups, pos = [], [], 0
    for _ in range(int(rng.integers(1, 5))):
        if rng.random() < 0.5:             # independent sequences
            n = int(rng.integers(1, 4))
            spec.append((0, rng.integers(1, 800, n, endpoint=True).tolist()))
            pos += n
        k = int(rng.integers(1, 25))       # a group sharing k blocks
        n = int(rng.integers(2, 6))
        spec.append((k, rng.integers(16 * k, 16 * k + 600, n,
                                     endpoint=True).tolist()))
        groups.append((pos, n))
        pos += n
    say("random shared prefix", seed, dtype, d, hq, hkv, spec)
    case = DecodeCase(_grouped_layout(spec, 8000 + seed), hq, hkv, d, dtype,
                      seed=8100 + seed)
    _run(case, expect_groups=groups)
