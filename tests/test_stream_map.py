"""The chain kernel's stream decode, checked on the CPU: tests/native/
stream_map_check.cpp compiles the decode (stream_info in la_kernels.hpp) for
the host and enumerates every stream of the sequence-parallel passes over
many shapes, checking each stays inside the tensors it indexes and that the
passes cover what the scan and the output need.  Nothing runs on a GPU."""
import os
import shutil
import subprocess

import pytest

from _lib_build import ROOT

CSRC = os.path.join(ROOT, "chunkwise_gated_delta_la_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "native", "stream_map_check.cpp")


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


def test_stream_decode_stays_in_bounds(tmp_path):
    cc = _hipcc()
    if cc is None:
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "stream_map_check")
    subprocess.run([cc, "-x", "hip", "--cuda-host-only", "-O1", "-std=c++17", "-I", CSRC,
                    SRC, "-o", exe], check=True, capture_output=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok ")
