"""Build libpsffn.so in-tree with hipcc for gfx950.

    python activation_sparse_ffn_psffn_amd/build.py   (or __graft_entry__.build())

Every HIP source is compiled with packed-fp32 instructions disabled (the compiler still emits
plain and vector fp32 code), position independent, then linked into one shared library next to
this file.  Sources are compiled in parallel; the link is atomic (temp file + rename).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpsffn.so")
SOURCES = ["api.hip", "predict.hip", "ffn.hip", "fused.hip", "batch.hip", "misc.hip", "stream.hip"]
ARCH = "gfx950"
# Per-source extra flags.  The MFMA kernels keep their accumulators in ordinary VGPRs: by default the
# compiler parks loaded weights in AGPRs and copies them back (about 20% of the 4-bit down kernel's
# instructions); measured on MI355X, OPT-175B-shaped 4-bit layer at 8 tokens 106.4 -> 103.5 us.
EXTRA_FLAGS = {"batch.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpsffn")


def flags() -> list:
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str, out_dir: str) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, "\n".join(msgs)))
    if any(("warning" in m or "error" in m) for m in msgs):
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def build(verbose: bool = False) -> str:
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, out_dir), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
