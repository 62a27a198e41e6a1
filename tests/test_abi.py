"""The C ABI library loads and exports every symbol include/pa.h declares;
host-side argument validation returns the documented status codes.

No test here reaches a kernel launch: every call either fails validation or
is a documented no-op, so nothing touches a GPU (fake, aligned device
addresses are never dereferenced on the host)."""

import os
import re

import pytest

from paged_kv_cache_slot_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include",
                      "pa.h")
FAKE = 1 << 20            # aligned non-NULL address, never dereferenced
MISALIGNED = FAKE + 4


@pytest.fixture(scope="module")
def no_device():
    """Every case here must fail validation before any launch.  As a second
    line of defence, refuse to run where a GPU is visible: a case that
    slipped past validation would launch on fake addresses."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        count = ctypes.c_int(0)
        visible = hip.hipGetDeviceCount(ctypes.byref(count)) == 0 and \
            count.value > 0
    except OSError:
        visible = False
    if visible:
        pytest.skip("validation tests use fake device addresses; CPU only")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    lib = _lib.load()
    names = declared_symbols()
    assert {"pa_store_kv", "pa_decode", "pa_prefill_varlen"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.SIGNATURES), "binding out of sync"


def test_version_and_strings():
    lib = _lib.load()
    assert lib.pa_abi_version() == 1
    for code, name in _lib.STATUS.items():
        assert lib.pa_status_string(code).decode().startswith(name)
    assert b"unknown" in lib.pa_status_string(99)


def _decode(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=64, bs=16, bt=FAKE, w=8,
             cl=FAKE, maxlen=100, b=4, hq=8, hkv=2, d=64, scale=0.125,
             ws=None, wsb=0, dtype=_lib.PA_F32, stream=None)
    a.update(kw)
    return lib.pa_decode(a["out"], a["q"], a["k"], a["v"], a["nb"], a["bs"],
                         a["bt"], a["w"], a["cl"], a["maxlen"], a["b"],
                         a["hq"], a["hkv"], a["d"], a["scale"], a["ws"],
                         a["wsb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), 3), (dict(d=0), 2), (dict(bs=32), 3), (dict(hq=6, hkv=4), 2),
    (dict(hq=6, hkv=2), 3), (dict(hq=32, hkv=2), 3), (dict(dtype=7), 3),
    (dict(b=-1), 2), (dict(maxlen=-5), 2), (dict(out=None), 1),
    (dict(q=None), 1), (dict(cl=None), 1), (dict(bt=None), 1),
    (dict(q=MISALIGNED), 3), (dict(k=MISALIGNED), 3),
    (dict(scale=0.0), 2), (dict(scale=-0.1), 2), (dict(scale=float("inf")), 2),
    (dict(scale=float("nan")), 2),
    (dict(maxlen=4096), 4),                       # needs a workspace
    (dict(maxlen=4096, ws=FAKE, wsb=16), 4),       # workspace too small
    (dict(b=0), 0),                                # empty batch: no-op
])
def test_decode_validation(kw, code, no_device):
    assert _decode(_lib.load(), **kw) == code


def _decode_noalloc(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=64, bs=16, bt=FAKE, w=8,
             cl=FAKE, maxlen=100, b=4, hq=8, hkv=2, d=64, scale=0.125,
             dtype=_lib.PA_F32, stream=None)
    a.update(kw)
    return lib.pa_decode_noalloc(
        a["out"], a["q"], a["k"], a["v"], a["nb"], a["bs"], a["bt"], a["w"],
        a["cl"], a["maxlen"], a["b"], a["hq"], a["hkv"], a["d"], a["scale"],
        a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(b=-1), 2), (dict(hkv=3), 2), (dict(d=96), 3), (dict(bs=32), 3),
    (dict(hq=32, hkv=2), 3), (dict(dtype=9), 3), (dict(maxlen=-1), 2),
    (dict(scale=0.0), 2), (dict(scale=float("inf")), 2),
    (dict(out=None), 1), (dict(cl=None), 1), (dict(bt=None), 1),
    (dict(q=MISALIGNED), 3),
    (dict(b=0), 0),                                # empty batch: no-op
    # 64 sequences x 64 query heads over 2^20-token contexts, fp32: ~272 MB
    # of partials, past the 32 MiB static scratch -> rejected, nothing
    # launched
    (dict(b=64, hq=64, hkv=8, d=128, maxlen=1 << 20, dtype=_lib.PA_F32), 6),
])
def test_decode_noalloc_validation(kw, code, no_device):
    assert _decode_noalloc(_lib.load(), **kw) == code


def test_decode_noalloc_limit_matches_workspace_query():
    """The static scratch is 32 MiB.  The workspace query covers either
    element type (the larger need): sizes whose query fits are accepted
    for both; past it, fp32 is rejected while bfloat16, whose split-context
    partials are binary16 rows of the small-row kernel, may still fit."""
    lib = _lib.load()
    big = lib.pa_decode_workspace_bytes(64, 64, 8, 128, 1 << 20)
    assert big > 32 << 20
    assert _decode_noalloc(lib, b=64, hq=64, hkv=8, d=128, maxlen=1 << 20,
                           dtype=_lib.PA_F32) == 6
    fits = lib.pa_decode_workspace_bytes(256, 32, 8, 128, 8192)
    assert 0 < fits <= 32 << 20


def test_decode_workspace_query():
    lib = _lib.load()
    assert lib.pa_decode_workspace_bytes(4, 8, 2, 64, 100) == 0
    # 8192-token contexts over 2,048 (sequence, KV head) groups split into
    # several partitions: at least two partials of (max, sum, D floats) per
    # (sequence, query head), 256-byte aligned sections.
    one = lib.pa_decode_workspace_bytes(256, 32, 8, 128, 8192)
    assert one >= 256 * 32 * 2 * (128 + 2) * 4
    assert one % 256 == 0
    assert lib.pa_decode_workspace_bytes(0, 8, 2, 64, 100) == 0
    assert lib.pa_decode_workspace_bytes(256, 32, 0, 128, 8192) == 0
    assert lib.pa_decode_workspace_bytes(256, 32, -8, 128, 8192) == 0


def _store(lib, **kw):
    a = dict(k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, sm=FAKE, t=4, hkv=2, d=64,
             s=1024, dtype=_lib.PA_F32, stream=None)
    a.update(kw)
    return lib.pa_store_kv(a["k"], a["v"], a["kc"], a["vc"], a["sm"], a["t"],
                           a["hkv"], a["d"], a["s"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(t=-1), 2), (dict(hkv=0), 2), (dict(s=-1), 2), (dict(dtype=5), 3),
    (dict(k=None), 1), (dict(sm=None), 1), (dict(vc=MISALIGNED), 3),
    (dict(hkv=1, d=2), 3),                         # 8-byte rows
    (dict(t=0), 0), (dict(t=0, k=None), 0),        # nothing to store
])
def test_store_validation(kw, code, no_device):
    assert _store(_lib.load(), **kw) == code


def _prefill(lib, **kw):
    a = dict(out=FAKE, q=FAKE, tq=16, k=FAKE, v=FAKE, nb=64, bs=16, cuq=FAKE,
             cuk=FAKE, mq=8, mk=40, bt=FAKE, w=4, b=2, hq=8, hkv=2, d=128,
             scale=0.1, causal=1, ws=None, wsb=0, dtype=_lib.PA_BF16,
             stream=None)
    a.update(kw)
    return lib.pa_prefill_varlen(
        a["out"], a["q"], a["tq"], a["k"], a["v"], a["nb"], a["bs"], a["cuq"],
        a["cuk"], a["mq"], a["mk"], a["bt"], a["w"], a["b"], a["hq"],
        a["hkv"], a["d"], a["scale"], a["causal"], a["ws"], a["wsb"],
        a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=80), 3), (dict(bs=8), 3), (dict(hq=12, hkv=4), 3),
    (dict(tq=-1), 2), (dict(mq=-2), 2), (dict(out=None), 1),
    (dict(scale=0.0), 2), (dict(scale=-1.0), 2), (dict(scale=float("nan")), 2),
    (dict(cuq=None), 1), (dict(bt=None), 1), (dict(q=MISALIGNED), 3),
    (dict(b=0), 0), (dict(tq=0), 0), (dict(mq=0), 0),
])
def test_prefill_validation(kw, code, no_device):
    assert _prefill(_lib.load(), **kw) == code


def _copy(lib, **kw):
    a = dict(kc=FAKE, vc=FAKE, pairs=FAKE, n=3, bb=32768, nb=100, stream=None)
    a.update(kw)
    return lib.pa_copy_blocks(a["kc"], a["vc"], a["pairs"], a["n"], a["bb"],
                              a["nb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), 0),                               # nothing to copy: no-op
    (dict(bb=0), 0),                              # empty blocks: no-op
    (dict(n=-1), 2),
    (dict(bb=-16), 2),
    (dict(nb=-1), 2),
    (dict(kc=None), 1),
    (dict(vc=None), 1),
    (dict(pairs=None), 1),
    (dict(bb=32760), 3),                          # not a multiple of 16
    (dict(kc=MISALIGNED), 3),
    (dict(bb=(1 << 30) + 16 * 1024), 3),          # block above 1 GiB
])
def test_copy_blocks_validation(kw, code, no_device):
    assert _copy(_lib.load(), **kw) == code


def _shared(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=64, bs=16, bt=FAKE, w=8,
             cl=FAKE, pl=FAKE, maxsuf=60, maxpre=64, groups=FAKE, ng=1,
             maxg=4, b=4, hq=8, hkv=2, d=64, scale=0.125, ws=None, wsb=0,
             dtype=_lib.PA_F32, stream=None)
    a.update(kw)
    return lib.pa_decode_shared_prefix(
        a["out"], a["q"], a["k"], a["v"], a["nb"], a["bs"], a["bt"], a["w"],
        a["cl"], a["pl"], a["maxsuf"], a["maxpre"], a["groups"], a["ng"],
        a["maxg"], a["b"], a["hq"], a["hkv"], a["d"], a["scale"], a["ws"],
        a["wsb"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), 3), (dict(bs=8), 3), (dict(hq=6, hkv=2), 3),
    (dict(dtype=4), 3), (dict(b=-1), 2), (dict(maxsuf=-1), 2),
    (dict(maxpre=-16), 2), (dict(ng=-1), 2), (dict(maxg=-2), 2),
    (dict(maxsuf=0x7fffffff, maxpre=16), 2), (dict(scale=0.0), 2),
    (dict(out=None), 1), (dict(q=None), 1), (dict(cl=None), 1),
    (dict(pl=None), 1), (dict(bt=None), 1), (dict(groups=None), 1),
    (dict(v=MISALIGNED), 3),
    (dict(), 4),                                   # workspace is required
    (dict(ws=FAKE, wsb=64), 4),                    # and must be large enough
    (dict(b=0), 0),                                # empty batch: no-op
])
def test_shared_prefix_validation(kw, code, no_device):
    assert _shared(_lib.load(), **kw) == code


def test_shared_prefix_workspace_query():
    lib = _lib.load()
    q = lib.pa_decode_shared_prefix_workspace_bytes
    # 128 sequences sharing 2,048 tokens, suffixes up to 512: one suffix
    # partition plus the prefix chunks, (max, sum, D floats) each
    n = q(128, 32, 8, 128, 512, 2048, 1, 128)
    assert n >= 128 * 32 * 2 * (128 + 2) * 4 and n % 256 == 0
    # no prefix: still one partial slot per (sequence, head) for the merge
    assert q(4, 8, 2, 64, 100, 0, 0, 0) >= 4 * 8 * (64 + 2) * 4
    assert q(0, 8, 2, 64, 100, 0, 0, 0) == 0
    assert q(4, 8, 2, 64, -1, 0, 0, 0) == 0


def _store8(lib, **kw):
    a = dict(k=FAKE, v=FAKE, kc=FAKE, vc=FAKE, sm=FAKE, t=4, hkv=2, d=64,
             s=1024, dtype=_lib.PA_BF16, ks=0.5, vs=0.25, stream=None)
    a.update(kw)
    return lib.pa_store_kv_fp8(a["k"], a["v"], a["kc"], a["vc"], a["sm"],
                               a["t"], a["hkv"], a["d"], a["s"], a["dtype"],
                               a["ks"], a["vs"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(t=-1), 2), (dict(hkv=0), 2), (dict(s=-1), 2), (dict(ks=0.0), 2),
    (dict(vs=-1.0), 2), (dict(ks=float("inf")), 2), (dict(vs=float("nan")), 2),
    (dict(dtype=2), 3), (dict(k=None), 1), (dict(sm=None), 1),
    (dict(vc=MISALIGNED), 3), (dict(hkv=1, d=4), 3), (dict(t=0), 0),
])
def test_store_fp8_validation(kw, code, no_device):
    assert _store8(_lib.load(), **kw) == code


def _decode8(lib, **kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, nb=64, bs=16, bt=FAKE, w=8,
             cl=FAKE, maxlen=100, b=4, hq=8, hkv=2, d=128, scale=0.125,
             ks=0.5, vs=0.25, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.pa_decode_fp8(a["out"], a["q"], a["k"], a["v"], a["nb"],
                             a["bs"], a["bt"], a["w"], a["cl"], a["maxlen"],
                             a["b"], a["hq"], a["hkv"], a["d"], a["scale"],
                             a["ks"], a["vs"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=64), 3), (dict(d=96), 3), (dict(bs=32), 3), (dict(hq=6, hkv=2), 3),
    (dict(b=-1), 2), (dict(maxlen=-1), 2), (dict(scale=0.0), 2),
    (dict(ks=0.0), 2), (dict(vs=float("inf")), 2), (dict(out=None), 1),
    (dict(cl=None), 1), (dict(bt=None), 1), (dict(k=MISALIGNED), 3),
    (dict(maxlen=4096), 4), (dict(b=0), 0),
])
def test_decode_fp8_validation(kw, code, no_device):
    assert _decode8(_lib.load(), **kw) == code


def test_missing_library_raises(monkeypatch):
    """No fallback: with the library absent, loading it raises."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libpa.so")
    with pytest.raises(RuntimeError, match="no fallback"):
        _lib.load()


def test_ops_reject_host_tensors():
    """Every operation refuses CPU tensors instead of computing on the host."""
    import torch

    from paged_kv_cache_slot_amd import ops
    f = torch.zeros((2, 16, 2, 64), dtype=torch.float32)
    q = torch.zeros((1, 4, 64), dtype=torch.float32)
    i = torch.zeros((1, 1), dtype=torch.int32)
    n = torch.ones(1, dtype=torch.int32)
    calls = [
        lambda: ops.store_kv(q[:, :2], q[:, :2], f, f, n),
        lambda: ops.copy_blocks(f, f, torch.zeros((1, 2), dtype=torch.int32)),
        lambda: ops.decode(q, f, f, i, n, 1),
        lambda: ops.prefill_varlen(q, f, f, torch.tensor([0, 1], dtype=torch.int32),
                                   torch.tensor([0, 1], dtype=torch.int32), 1, 1, i),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="GPU tensors only"):
            call()


def test_ops_reject_mismatched_out():
    """A caller-supplied output buffer must match q in shape, dtype and
    device (the kernels write q.numel() elements of q's dtype into it), and a
    workspace must sit on q's device.  Checked before anything else, so no
    GPU is needed to see the errors."""
    import torch

    from paged_kv_cache_slot_amd import ops
    f = torch.zeros((2, 16, 2, 64), dtype=torch.float32)
    q = torch.zeros((3, 4, 64), dtype=torch.float32)
    qb = torch.zeros((3, 4, 128), dtype=torch.bfloat16)
    i = torch.zeros((3, 1), dtype=torch.int32)
    n = torch.ones(3, dtype=torch.int32)
    cu = torch.tensor([0, 1, 2, 3], dtype=torch.int32)
    u8 = torch.zeros((2, 16, 2, 128), dtype=torch.uint8)
    g = torch.zeros((1, 2), dtype=torch.int32)
    meta = torch.empty(16, dtype=torch.uint8, device="meta")

    def ops_with(qq, out=None, workspace=None):
        return [
            lambda: ops.decode(qq, f, f, i, n, 1, out=out,
                               workspace=workspace),
            lambda: ops.prefill_varlen(qq, f, f, cu, cu, 1, 1, i, out=out,
                                       workspace=workspace),
            lambda: ops.decode_shared_prefix(qq, f, f, i, n, n, g, 1, 0, 1,
                                             out=out, workspace=workspace),
        ]

    bad = [
        (ValueError, "shape", dict(out=torch.zeros((2, 4, 64)))),
        (ValueError, "shape", dict(out=torch.zeros((3, 4, 64)).view(-1))),
        (TypeError, "dtype", dict(out=torch.zeros((3, 4, 64),
                                                  dtype=torch.bfloat16))),
        (ValueError, "is on", dict(out=torch.empty((3, 4, 64),
                                                   device="meta"))),
        (ValueError, "workspace is on", dict(workspace=meta)),
    ]
    for exc, msg, kw in bad:
        for call in ops_with(q, **kw):
            with pytest.raises(exc, match=msg):
                call()
    # the 8-bit decode takes bf16 q / out
    with pytest.raises(TypeError, match="dtype"):
        ops.decode_fp8(qb, u8, u8, i, n, 1, 1.0, 1.0,
                       out=torch.zeros((3, 4, 128)))
    with pytest.raises(ValueError, match="shape"):
        ops.decode_fp8(qb, u8, u8, i, n, 1, 1.0, 1.0,
                       out=torch.zeros((3, 4, 64), dtype=torch.bfloat16))
