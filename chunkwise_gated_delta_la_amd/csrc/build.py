"""Build liblachunk.so (gfx950) in-tree with hipcc.

    python chunkwise_gated_delta_la_amd/csrc/build.py [--jobs N] [--verbose]

Each .hip translation unit is compiled to an object under _build/ at the
repository root (in parallel), then linked into
chunkwise_gated_delta_la_amd/liblachunk.so.  Always rebuilds.
"""
import argparse
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
OBJ_DIR = os.path.join(ROOT, "_build", "lachunk")
LIB = os.path.join(PKG, "liblachunk.so")
SOURCES = ["la_api.hip", "la_decode.hip", "la_chunk.hip", "la_chunk_pipe.hip", "la_bwd.hip"]
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed FP32 instructions are disabled for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the chain kernel's accumulators feed
    # VALU work (splits, scaling) every chunk, and AGPR-resident results
    # would need a v_accvgpr_read per value
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"), "-I", HERE,
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = r.stdout + r.stderr
    # hipcc's host pass does not know the device-only target feature; the
    # warning it prints for that is expected and filtered here.
    lines = [ln for ln in out.splitlines()
             if "packed-fp32-ops' is not a recognized feature" not in ln]
    return r.returncode, "\n".join(lines)


def build(jobs=None, verbose=False):
    os.makedirs(OBJ_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc] + CFLAGS + ["-c", os.path.join(HERE, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 16)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    failed = False
    for (rc, msg), src in zip(results, SOURCES):
        if msg.strip():
            print(f"[{src}]\n{msg}", file=sys.stderr)
        failed |= rc != 0
    if failed:
        raise RuntimeError("liblachunk: compilation failed")
    tmp = LIB + ".tmp"
    # -z defs: a symbol left undefined fails the link instead of the load
    rc, msg = _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp]
                   + objs, verbose)
    if rc != 0:
        raise RuntimeError("liblachunk: link failed\n" + msg)
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=None)
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.verbose))


if __name__ == "__main__":
    main()
