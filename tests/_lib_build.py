"""Test helper: make sure liblachunk.so exists (build it if nothing is built)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "chunkwise_gated_delta_la_amd", "liblachunk.so")


def ensure_built():
    if not os.path.exists(LIB):
        subprocess.run([sys.executable,
                        os.path.join(ROOT, "chunkwise_gated_delta_la_amd", "csrc", "build.py")],
                       check=True)
    return LIB
