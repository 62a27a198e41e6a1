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


@pytest.mark.parametrize("seed", range(10))
def test_random_decode(seed):
    rng = np.random.default_rng(7100 + seed)
    dtype, d, hq, hkv = _shape(rng)
    b = int(rng.integers(1, 33))
    lens = rng.integers(0, 2500, b, endpoint=True)
    lens[rng.random(b) < 0.1] = 0          # batch padding rows
    say("random decode", seed, dtype, d, hq, hkv, b)
    lay = wl.decode_layout(lens.tolist(), 16, seed=7200 + seed)
    check_decode(DecodeCase(lay, hq, hkv, d, dtype, seed=7300 + seed))


@pytest.mark.parametrize("seed", range(10))
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
