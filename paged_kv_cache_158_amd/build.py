"""Build libpa.so (HIP kernels for gfx950 + the C ABI + the host block manager).

Run as a script (`python paged_kv_cache_158_amd/build.py`) or call `build()`.
Every source is compiled with hipcc for gfx950 only, in parallel, into
`_build/` next to this file, then linked into `libpa.so` in the package
directory, where the Python binding loads it.  The build never runs
anything on a GPU.

`build(timeline=True)` (`build.py --timeline`) builds the same sources with
PA_TIMELINE into `libpa_timeline.so` instead: kernels that also record
per-wave timestamps for `timeline.py`.  The product library has none of it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libpa.so")
OBJDIR = os.path.join(HERE, "_build")
OUT_TIMELINE = os.path.join(HERE, "libpa_timeline.so")
OBJDIR_TIMELINE = os.path.join(HERE, "_build_timeline")

SOURCES = ["pa_api.cpp", "block_manager.cpp", "cache_ops.hip", "decode.hip", "varlen.hip"]

ARCH = "gfx950"
# Packed fp32 VALU ops are kept off: hipcc would otherwise fuse scalar float
# code into v_pk_* instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libpa)")


def _compile(src: str, jobs_env: dict, objdir: str, defines: list) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, *defines, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True, env=jobs_env)
    noise = "is not a recognized feature for this target"
    err = "\n".join(ln for ln in (r.stderr or "").splitlines() if noise not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def sources_digest() -> str:
    """sha256 over every source and header the library is built from."""
    import hashlib
    h = hashlib.sha256()
    for d in (CSRC, INCLUDE):
        for fn in sorted(os.listdir(d)):
            if fn.endswith((".hip", ".cpp", ".h")):
                h.update(fn.encode())
                with open(os.path.join(d, fn), "rb") as f:
                    h.update(f.read())
    return h.hexdigest()


def build(verbose: bool = True, timeline: bool = False) -> str:
    """Compile every source and link libpa.so (libpa_timeline.so with
    timeline=True); returns its path."""
    out, objdir = (OUT_TIMELINE, OBJDIR_TIMELINE) if timeline else (OUT, OBJDIR)
    defines = ["-DPA_TIMELINE"] if timeline else []
    os.makedirs(objdir, exist_ok=True)
    env = dict(os.environ)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, env, objdir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking {os.path.basename(out)} failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, out)
    if timeline:  # timeline.py checks that the library matches the sources
        with open(out + ".sources", "w") as f:
            f.write(sources_digest() + "\n")
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build(timeline="--timeline" in sys.argv[1:])
