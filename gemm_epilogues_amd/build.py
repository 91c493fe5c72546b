"""Build the fused-chain library: hipcc for gfx950 -> gemm_epilogues_amd/libfc.so.

Every translation unit under csrc/ is compiled in parallel to an object file,
then linked into one shared library exporting the C ABI of include/fc.h, and
the measurement probes into libfcenv.so (include/fc_envelope.h).  The
compiler's per-kernel resource report (VGPRs, AGPRs, SGPRs, LDS, scratch,
occupancy) is parsed into kernel_resources.json next to the library.

Usage: python gemm_epilogues_amd/build.py [--jobs N]
"""
from __future__ import annotations

import argparse
import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfc.so")
ENV_LIB = os.path.join(HERE, "libfcenv.so")
RES = os.path.join(HERE, "kernel_resources.json")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          # packed fp32 instructions stay off
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]
SOURCES = ["chain.hip", "chain_fat.hip", "softmax.hip", "gemm.hip", "attention.hip", "rmsnorm.hip", "api.cpp"]
# measurement probes (stream and MFMA ceilings), a library of their own
ENV_SOURCES = ["envelope.hip"]


def _parse_resources(text: str) -> dict:
    out, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s*(-?\d+)", line)
        if m and cur is not None:
            key = m.group(1).strip()
            cur[key] = int(m.group(2))
    return out


def build(jobs: int = 0, verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    procs = []
    for src in SOURCES + ENV_SOURCES:
        path = os.path.join(CSRC, src)
        obj = os.path.join(OBJ, src + ".o")
        cmd = [HIPCC] + COMMON + ["-c", path, "-o", obj]
        if src.endswith(".hip"):
            cmd += ["-Rpass-analysis=kernel-resource-usage"]
        else:
            cmd = [HIPCC, "-O2", "-std=c++17", "-fPIC", "-c", path, "-o", obj]
        procs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.PIPE, text=True)))
    resources, failed = {}, []
    for src, obj, p in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            failed.append((src, err))
        else:
            resources.update(_parse_resources(err))
            if verbose:
                sys.stderr.write(err)
    if failed:
        for src, err in failed:
            sys.stderr.write(f"--- {src} failed ---\n{err}\n")
        raise RuntimeError("hipcc failed: " + ", ".join(s for s, _ in failed))
    for lib, srcs in ((LIB, SOURCES), (ENV_LIB, ENV_SOURCES)):
        tmp = lib + ".tmp"
        link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + \
            [os.path.join(OBJ, s + ".o") for s in srcs]
        subprocess.run(link, check=True)
        os.replace(tmp, lib)
    with open(RES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.verbose))
