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
SOURCES = ["api.hip", "encode.hip", "scan.hip", "select.hip", "reindex.hip", "attend.hip", "calib.hip"]
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
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Rpass-analysis=kernel-resource-usage"]


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


def _resource_usage(out: str):
    """(kernel, VGPRs, scratch bytes per lane) from the compiler's
    kernel-resource-usage remarks."""
    res, name, vgpr = [], None, None
    for line in out.splitlines():
        if "remark: Function Name:" in line:
            name = line.split("Function Name:")[1].split("[")[0].strip()
        elif "remark:     VGPRs:" in line:
            vgpr = int(line.split("VGPRs:")[1].split("[")[0])
        elif "remark:     ScratchSize [bytes/lane]:" in line and name:
            res.append((name, vgpr, int(line.split(":")[-1].split("[")[0])))
    return res


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
    spills = []
    for s, rc, out in results:
        usage = _resource_usage(out)
        spills += [f"{s}: {k} uses {b} B/lane of scratch ({v} VGPRs)" for k, v, b in usage if b > 0]
        if verbose:
            for k, v, b in usage:
                print(f"[{s}] {k}: {v} VGPRs, scratch {b}", file=sys.stderr)
            rest = "\n".join(l for l in out.splitlines() if "remark" not in l and "kernel-resource-usage" not in l
                             and not l.strip().startswith(("|", "^")) and l.strip() and not l.strip()[0].isdigit())
            if rest.strip():
                print(f"[{s}]\n{rest}", file=sys.stderr)
    # a register spill to scratch memory costs more than any kernel here can
    # afford: fail the build rather than ship one
    if spills:
        failed.append(("register spills", "\n".join(spills)))
    if failed:
        msg = "\n".join(f"== {s}\n{out}" for s, out in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    rc, out = _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[j[2] for j in jobs]])
    if rc != 0:
        raise RuntimeError(f"link failed:\n{out}")
    os.replace(tmp, LIB)
    return LIB


def build_host_asan() -> str:
    """libcsa2 with AddressSanitizer on its host code only (argument checks,
    workspace sizing, launch planning), for the host-side tests.  The device
    code is compiled as usual (it never runs there).  Written to
    _build/asan/libcsa2_asan.so."""
    cc = hipcc()
    out_dir = os.path.join(PKG, "_build", "asan")
    os.makedirs(out_dir, exist_ok=True)
    host = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    jobs = [(s, [cc, *host, "-c", os.path.join(CSRC, s), "-o", os.path.join(out_dir, s.replace(".hip", ".o"))])
            for s in SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        results = list(ex.map(lambda j: (j[0], *_run(j[1])), jobs))
    failed = [(s, out) for s, rc, out in results if rc != 0]
    if failed:
        raise RuntimeError("hipcc (host ASan) failed:\n" + "\n".join(f"== {s}\n{out}" for s, out in failed))
    lib = os.path.join(out_dir, "libcsa2_asan.so")
    rc, out = _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-o", lib,
                    *[os.path.join(out_dir, s.replace(".hip", ".o")) for s in SOURCES]])
    if rc != 0:
        raise RuntimeError(f"link (host ASan) failed:\n{out}")
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
