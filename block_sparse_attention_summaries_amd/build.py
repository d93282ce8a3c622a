"""Build libsparse_attn.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_attn.so")
SOURCES = ["api.hip", "summaries.hip", "select.hip", "select_mfma.hip", "select_bwd.hip", "retain.hip", "forest.hip", "attn.hip", "decode_step.hip", "attn_mfma.hip", "attn_bwd_mfma.hip", "probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 (v_pk_*_f32) instructions in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one object each) and link
    libsparse_attn.so.  Always recompiles."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        jobs.append((obj, [HIPCC, *compile_flags, "-c", os.path.join(CSRC, src), "-o", obj]))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, cmd, verbose) for _, cmd in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, *FLAGS, *[obj for obj, _ in jobs], "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
