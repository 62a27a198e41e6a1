"""pa_decode_noalloc (decode with the library's static per-GPU scratch instead
of a caller's workspace) against pa_decode on the same inputs.

Both entry points run the same kernels with the same plan, so the outputs
must agree bit for bit; sampled sequences are also checked against the
oracle.  Two calls in a row, the second with a smaller input (fewer
sequences, heads and partitions, another element type), show that what the
first call left in the shared scratch does not leak into the second."""

import numpy as np
import pytest
import torch

import workloads as wl
from paged_kv_cache_slot_amd import ops
from tests.gpu_harness import (TOL, DecodeCase, bits_equal, f64, sample_seqs,
                               say)

pytestmark = pytest.mark.gpu


def _run_both(case):
    out_ref = torch.full_like(case.q, float("nan"))
    out_na = torch.full_like(case.q, float("nan"))
    case.run_decode(out=out_ref)
    ops.decode_noalloc(case.q, case.kc, case.vc, case.block_tables,
                       case.context_lens, case.max_context_len,
                       scale=case.scale, out=out_na)
    torch.cuda.synchronize()
    return out_ref, out_na


def test_noalloc_matches_decode_two_calls():
    # first call: 128 sequences, 32q/8kv, D=128, bf16, contexts U[512, 8192]
    # -> 1,024-token partitions, longest-first order, ~17 MB of scratch
    rng = np.random.default_rng(71)
    lens1 = rng.integers(512, 8193, 128)
    lens1[0], lens1[1] = 8192, 512
    need1 = ops.decode_workspace_bytes(128, 32, 8, 128, int(lens1.max()))
    assert 8 << 20 < need1 <= ops.DECODE_SCRATCH_BYTES
    say("noalloc call 1: 128 seqs 32q/8kv D128 bf16, ws", need1)
    c1 = DecodeCase(wl.decode_layout(lens1, 16, seed=72), 32, 8, 128, "bf16",
                    seed=73)
    c1.run_store()
    ref1, na1 = _run_both(c1)
    assert bits_equal(wl.host_bits(ref1), wl.host_bits(na1))

    # second call, smaller: 16 sequences, 8q/2kv, D=64, fp32, contexts
    # U[1, 3000] with an empty one -> fewer partitions and slots than the
    # first call wrote
    lens2 = rng.integers(1, 3001, 16)
    lens2[3] = 0
    need2 = ops.decode_workspace_bytes(16, 8, 2, 64, int(lens2.max()))
    assert 0 < need2 < need1
    say("noalloc call 2: 16 seqs 8q/2kv D64 f32, ws", need2)
    c2 = DecodeCase(wl.decode_layout(lens2, 16, seed=74), 8, 2, 64, "f32",
                    seed=75)
    c2.run_store()
    ref2, na2 = _run_both(c2)
    assert bits_equal(wl.host_bits(ref2), wl.host_bits(na2))

    # both against the oracle on sampled sequences
    for case, got in ((c1, na1), (c2, na2)):
        ek, ev = case.oracle_store()
        seqs = sample_seqs(case.lens, 6, seed=76)
        want = case.oracle_decode(ek, ev, seqs=seqs)
        g = f64(got)
        assert np.all(np.isfinite(g[seqs]))
        err = float(np.max(np.abs(g[seqs] - want[seqs])))
        assert err <= TOL[case.dtype], (case.dtype, err)


def test_noalloc_single_partition_and_limit():
    """Contexts that fit one partition need no scratch; sizes past the
    static scratch (fp32: 64 sequences x 64 query heads over 2^20-token
    contexts, ~272 MB of partials) are refused with PA_ERR_SCRATCH_LIMIT
    before launch."""
    say("noalloc single partition")
    c = DecodeCase(wl.decode_layout([7, 16, 33, 100], 16, seed=77), 8, 2, 64,
                   "f32", seed=78)
    c.run_store()
    ref, na = _run_both(c)
    assert bits_equal(wl.host_bits(ref), wl.host_bits(na))
    from paged_kv_cache_slot_amd import _lib
    with pytest.raises(_lib.PaError, match="SCRATCH_LIMIT"):
        q = torch.zeros((64, 64, 128), dtype=torch.float32, device="cuda")
        kc = torch.zeros((1, 16, 8, 128), dtype=torch.float32, device="cuda")
        bt = torch.zeros((64, 1), dtype=torch.int32, device="cuda")
        cl = torch.zeros(64, dtype=torch.int32, device="cuda")
        ops.decode_noalloc(q, kc, kc, bt, cl, 1 << 20)
