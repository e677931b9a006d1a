"""Build libwq.so (the HIP kernels and the C ABI of include/wq.h) for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libwq.so")
SOURCES = ["wq_api.hip", "wq_misc.hip", "wq_skinny.hip", "wq_tiled.hip", "wq_encode.hip"]
ARCH = os.environ.get("WQ_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # packed fp32 instructions stay off: plain fp32 code only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-ffp-contract=off",
]


def _headers_mtime() -> float:
    inc = os.path.join(os.path.dirname(HERE), "include")
    paths = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hpp")]
    paths += [os.path.join(inc, f) for f in os.listdir(inc) if f.endswith(".h")]
    return max(os.path.getmtime(p) for p in paths)


def _compile(src: str, obj_dir: str, force: bool = True) -> str:
    obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
    if not force and os.path.exists(obj):
        newest = max(os.path.getmtime(os.path.join(CSRC, src)), _headers_mtime())
        if os.path.getmtime(obj) >= newest:
            return obj
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, force: bool = True) -> str:
    """Compile every source (force) or only those older than their source or a header."""
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, force), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True, force="--incremental" not in sys.argv)
