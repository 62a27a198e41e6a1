"""ctypes loader for libpa.so: argument types of every C ABI entry point.

The library is built in-tree (``python -m paged_kv_cache_slot_amd.build``).
There is no fallback: if the library is missing, every operation raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32 = 0
PA_BF16 = 1

STATUS = {
    0: "PA_OK",
    1: "PA_ERR_NULL",
    2: "PA_ERR_SHAPE",
    3: "PA_ERR_UNSUPPORTED",
    4: "PA_ERR_WORKSPACE",
    5: "PA_ERR_LAUNCH",
    6: "PA_ERR_SCRATCH_LIMIT",
}

_c_void_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_size = ctypes.c_size_t
_f32 = ctypes.c_float

SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_abi_version": (_i32, []),
    "pa_store_kv": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
        _i64, _i32, _i32, _i64, ctypes.c_int, _c_void_p]),
    "pa_copy_blocks": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p]),
    "pa_decode_workspace_bytes": (_size, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
        _c_void_p, _i32, _c_void_p, _i32, _i32, _i32, _i32, _i32, _f32,
        _c_void_p, _size, ctypes.c_int, _c_void_p]),
    "pa_decode_noalloc": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
        _c_void_p, _i32, _c_void_p, _i32, _i32, _i32, _i32, _i32, _f32,
        ctypes.c_int, _c_void_p]),
    "pa_prefill_workspace_bytes": (_size, [_i32, _i32, _i32, _i32, _i32,
                                           _i32]),
    "pa_prefill_varlen": (ctypes.c_int, [
        _c_void_p, _c_void_p, _i64, _c_void_p, _c_void_p, _i64, _i32,
        _c_void_p, _c_void_p, _i32, _i32, _c_void_p, _i32, _i32, _i32,
        _i32, _i32, _f32, _i32, _c_void_p, _size, ctypes.c_int,
        _c_void_p]),
    "pa_decode_shared_prefix_workspace_bytes": (_size, [
        _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_shared_prefix": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
        _c_void_p, _i32, _c_void_p, _c_void_p, _i32, _i32, _c_void_p, _i32,
        _i32, _i32, _i32, _i32, _i32, _f32, _c_void_p, _size, ctypes.c_int,
        _c_void_p]),
    "pa_store_kv_fp8": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
        _i64, _i32, _i32, _i64, ctypes.c_int, _f32, _f32, _c_void_p]),
    "pa_decode_fp8": (ctypes.c_int, [
        _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i32,
        _c_void_p, _i32, _c_void_p, _i32, _i32, _i32, _i32, _i32, _f32,
        _f32, _f32, _c_void_p, _size, _c_void_p]),
}

_lib = None


class PaError(RuntimeError):
    def __init__(self, name, status):
        self.status = status
        super().__init__(f"{name} failed: {status_string(status)}")


def load():
    """Load libpa.so once and declare its signatures.  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run "
            "`python -m paged_kv_cache_slot_amd.build` (or "
            "__graft_entry__.build()).  There is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status):
    try:
        return load().pa_status_string(status).decode()
    except Exception:  # noqa: BLE001 - message only
        return STATUS.get(status, f"status {status}")


def check(name, status):
    if status != 0:
        raise PaError(name, status)
