"""Build libhstu.so (the C-ABI library) for gfx950 with hipcc.

Run as ``python -m hstu_pointwise_attention_causal_amd.build`` or call
``build()``. Objects go to ``_build/`` at the repository root; the library is
written next to this file, where the Python binding loads it from. Every call
recompiles every source.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libhstu.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 VALU forms are disabled on every device pass (plain float code
# must not be turned into v_pk_{add,mul,fma}_f32).
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *DEVICE_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        err = "\n".join(line for line in (r.stderr or "").splitlines()
                        if "not a recognized feature" not in line)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libhstu.so; returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = _sources()
    workers = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # every kernel launched from host code must have its host stub in the library
    nm = subprocess.run(["nm", "-C", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.strip() for ln in nm.stdout.splitlines() if "hstu::" in ln]
    if missing:
        raise RuntimeError("undefined library symbols after link:\n" + "\n".join(missing))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
