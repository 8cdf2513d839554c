"""Locate libpa.so for the tests; build it only when nothing is built."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "paged_kv_cache_158_amd", "libpa.so")


def ensure_built() -> str:
    if not os.path.exists(LIB):
        subprocess.run([sys.executable, os.path.join(ROOT, "paged_kv_cache_158_amd", "build.py")],
                       check=True)
    return LIB
