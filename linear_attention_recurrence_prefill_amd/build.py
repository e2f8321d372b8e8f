"""Build the gfx950 HIP library (libgdn_mi355x.so) in-tree with hipcc.

Run ``python -m linear_attention_recurrence_prefill_amd.build`` (or call :func:`build`).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgdn_mi355x.so")
SOURCES = ["gdn_api.cpp", "gdn_fwd.hip", "gdn_fwd_fast.hip", "gdn_fwd_ws.hip",
           "gdn_fwd_split.hip", "gdn_bwd.hip", "gdn_bwd_chain.hip",
           "gdn_bwd_grad.hip", "gdn_decode.hip", "gdn_calib.hip", "gdn_check.hip",
           "gdn_noalloc.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions are not to be generated: they are turned off for the device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
             "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-munsafe-fp-atomics"]


# Per-source additions.  The pipelined forward kernel is latency-bound on one wave per SIMD; the
# ILP-first scheduler interleaves its independent MFMA chains and loads better than the default.
EXTRA_FLAGS = {"gdn_fwd_ws.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source (each to an object, in parallel) and link the shared library."""
    hipcc = _hipcc()
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in SOURCES:
        path = os.path.join(CSRC, src)
        if not os.path.exists(path):
            continue
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [hipcc, *HIP_FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-I",
               os.path.join(ROOT, "include"), "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT),
                      src))
        objs.append(obj)
        while len([p for p, _ in procs if p.poll() is None]) >= jobs:
            procs[0][0].wait()
    failed = []
    for p, src in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        lines = [ln for ln in text.splitlines() if "packed-fp32-ops" not in ln]
        if lines and (verbose or p.returncode):
            print("\n".join(lines), file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
