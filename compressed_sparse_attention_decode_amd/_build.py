"""Build libcsa2.so (HIP, gfx950) in the package directory with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libcsa2.so")
SOURCES = ["api.hip", "encode.hip", "scan.hip", "select.hip", "reindex.hip", "attend.hip"]
# The indexer contractions keep their MFMA accumulators in VGPRs (the epilogue
# reads every result with VALU ops; AGPR results would each need a
# v_accvgpr_read first) and assume finite scores (non-finite inputs are
# undefined by the ABI), so max(x, 0) needs no NaN canonicalisation.
EXTRA = {"scan.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"],
         "attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "reindex.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-fno-honor-nans"]}

# No fast-math: the FP4 encoder needs the correctly rounded fp32 division.
# Packed fp32 instructions are disabled for every device compile.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the CSA2 library needs ROCm's hipcc to build")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    return r.returncode, out


def build(verbose: bool = False) -> str:
    cc = hipcc()
    obj_dir = os.path.join(PKG, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    jobs = []
    for s in SOURCES:
        o = os.path.join(obj_dir, s.replace(".hip", ".o"))
        jobs.append((s, [cc, *FLAGS, *EXTRA.get(s, []), "-c", os.path.join(CSRC, s), "-o", o], o))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: (j[0], *_run(j[1])), jobs))
    failed = [(s, out) for s, rc, out in results if rc != 0]
    for s, rc, out in results:
        if verbose and out.strip():
            print(f"[{s}]\n{out}", file=sys.stderr)
    if failed:
        msg = "\n".join(f"== {s}\n{out}" for s, out in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    rc, out = _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[j[2] for j in jobs]])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
