"""Build libpa.so (the gfx950 HIP kernels + the C ABI) in this directory.

Every source is compiled for gfx950 only, with packed-FP32 instruction
generation disabled, then linked into one shared library that the Python
binding loads with ctypes.  Run ``python -m paged_kv_cache_slot_amd.build``.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpa.so"
ARCH = "gfx950"

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build libpa")
    return path


def sources():
    names = sorted(os.listdir(CSRC))
    return [os.path.join(CSRC, n) for n in names
            if n.endswith(".hip") or n.endswith(".cpp")]


def _check_symbols(path):
    """Every kernel host stub must be defined in the library: a device-only
    construct the host compilation pass cannot take silently drops a
    kernel's host side, which only shows as an undefined symbol."""
    res = subprocess.run(["nm", "-D", "--undefined-only", path],
                         capture_output=True, text=True)
    if res.returncode != 0:
        return  # nm unavailable: nothing to check with
    missing = [l.split()[-1] for l in res.stdout.splitlines()
               if "_ZN2pa" in l]
    if missing:
        raise RuntimeError(f"{path} leaves library symbols undefined: "
                           + ", ".join(missing[:4]))


def build(verbose=False, jobs=None):
    """Compile every source and link ``libpa.so``; returns its path."""
    hipcc = _hipcc()
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc] + HIP_FLAGS + ["-I", INCLUDE, "-I", CSRC] + lang + \
            ["-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode != 0:
            raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    out = os.path.join(HERE, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stderr}")
    _check_symbols(tmp)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
