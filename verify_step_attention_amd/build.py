"""Builds libvsa.so (the HIP library behind include/vsa.h) for gfx950 with hipcc.

    python -m verify_step_attention_amd.build        # or __graft_entry__.build()
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libvsa.so")
SOURCES = ["api.hip", "attention.hip", "sample_accept.hip", "sample_fused.hip", "qmm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed-fp32 instructions are kept out of the device code on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]

# Per-source flags. The attention kernels keep their MFMA accumulators in ordinary vector
# registers: with the default accumulation-register form, every rescale of O (a vector
# multiply) copied the accumulators out and back, about 150 moves per 32-key sub-tile.
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False, extra_flags=()):
    """Compiles every source to an object (in parallel), then links libvsa.so."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    tmp = LIB + ".tmp"
    with tempfile.TemporaryDirectory(prefix="vsa_build_") as td:
        objs = [os.path.join(td, os.path.basename(s) + ".o") for s in srcs]
        jobs = [[HIPCC, *FLAGS, *SOURCE_FLAGS.get(os.path.basename(s), []), *extra_flags, "-c",
                 s, "-o", o] for s, o in zip(srcs, objs)]
        workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
        with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(lambda c: _run(c, verbose), jobs))
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra_flags=sys.argv[1:])
