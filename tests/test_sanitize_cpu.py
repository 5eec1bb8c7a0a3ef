"""The C ABI's host code, and the kernels' index maps on the host, under
AddressSanitizer and UndefinedBehaviorSanitizer.

The library sources are compiled again with the host pass instrumented
(`-Xarch_host -fsanitize=address`, `-Xarch_host -fsanitize=undefined`, no
recovery; the device code is built as usual but never runs) and linked into
tests/native/abi_sanitize.cpp, which calls every entry point with NULL
pointers, bad and extreme sizes, overlapping fake pointers and bad
workspaces, and sweeps the workspace-size queries over sizes whose byte
counts pass 2^31 and 2^63.  Every such call must return its error code before
the first HIP call, so no GPU is involved.  A heap or stack error, a signed
overflow, a misaligned access or a wrong code fails the test.

tests/native/index_check.cpp takes the chunk kernels' index maps
(csrc/la_index.hpp: the tile swizzle, the DMA source offsets, the
transposed-read offsets, the state-row order, the T fragment and block
indices) and simulates on byte images of the LDS tiles every transfer and
read the kernels make with them, checking each lane's elements against the
operand layout and every offset against its array.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "chunkwise_gated_delta_la_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
SOURCES = ["la_api.hip", "la_decode.hip", "la_chunk.hip", "la_chunk_pipe.hip", "la_bwd.hip"]


def _hipcc():
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
COMMON = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(" ".join(cmd) + "\n" + r.stdout[-2000:] + r.stderr[-4000:])


def _build():
    cc = _hipcc()
    os.makedirs(OUT, exist_ok=True)
    dev = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    cmds = [[cc] + dev + SAN + COMMON + ["-c", os.path.join(CSRC, s),
                                         "-o", os.path.join(OUT, s + ".o")] for s in SOURCES]
    cmds.append([cc, "-x", "hip", "--offload-host-only"] + SAN + COMMON +
                ["-c", os.path.join(ROOT, "tests", "native", "abi_sanitize.cpp"),
                 "-o", os.path.join(OUT, "abi_sanitize.o")])
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        list(ex.map(_run, cmds))
    exe = os.path.join(OUT, "abi_sanitize")
    _run([cc, "--offload-arch=gfx950"] + SAN[:4] + ["-o", exe, os.path.join(OUT, "abi_sanitize.o")]
         + [os.path.join(OUT, s + ".o") for s in SOURCES])
    return exe


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_abi_validation_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert " 0 failures" in r.stdout, out[-6000:]


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_index_maps_on_the_host():
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "index_check")
    _run([_hipcc(), "-x", "hip", "--offload-host-only"] + SAN + COMMON +
         [os.path.join(ROOT, "tests", "native", "index_check.cpp"), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-6000:]
    assert r.returncode == 0 and " 0 failures" in r.stdout, out[-6000:]
