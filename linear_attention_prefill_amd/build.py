"""Ahead-of-time build of libkda.so for gfx950 (hipcc, no JIT at first call).

    python -m linear_attention_prefill_amd.build [--resource-usage]

Compiles every HIP source under csrc/ plus the C ABI into
``linear_attention_prefill_amd/libkda.so``.  Object files go to ``_build/``.
"""
from __future__ import annotations

import argparse
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkda.so")
# The same kernels with phase clocks recorded (kda_phase_clocks); built only
# on request, never loaded by the library's own calls.
CLOCKS_LIB = os.path.join(PKG, "libkda_clocks.so")
ARCH = "gfx950"

HIP_SOURCES = ["kda_prefill.hip", "kda_decode.hip", "kda_conv.hip", "kda_check.hip", "kda_stream.hip",
               "kda_mfma_probe.hip"]
CXX_SOURCES = ["kda_api.cpp"]

# Packed fp32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The state scan's matrix-core accumulators (the state and the output
# tiles) are also scaled and converted on the VALU every step: with them in
# accumulation registers the compiler moved them to and from vector registers
# around every such use (2 to 5 accumulator moves per product).  Keeping the
# products' C/D operands in vector registers removes those moves (16 packed
# sequences: scan 108 -> 103 us).
# The issue probe uses the same form, so that its rates are the ones the
# prefill kernels' products see.
PER_SOURCE_FLAGS = {"kda_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                    "kda_mfma_probe.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
          "-I" + os.path.join(ROOT, "include"), "-I" + CSRC]


HASH_FILE = LIB + ".srchash"


def source_hash() -> str:
    """sha256 over the library's sources (csrc/ and include/), in name order."""
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))
             if f.endswith((".hip", ".h", ".cpp"))]
    files += [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))]
    for path in files:
        h.update(os.path.relpath(path, ROOT).encode())
        with open(path, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def build(resource_usage: bool = False, verbose: bool = False, phase_clocks: bool = False) -> str:
    """Build libkda.so, or with phase_clocks libkda_clocks.so (-DKDA_PHASE_CLOCKS)."""
    hipcc = _hipcc()
    bdir = BUILD + ("_clocks" if phase_clocks else "")
    lib = CLOCKS_LIB if phase_clocks else LIB
    extra = ["-DKDA_PHASE_CLOCKS"] if phase_clocks else []
    os.makedirs(bdir, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        cmd = [hipcc, "-x", "hip", "--offload-arch=" + ARCH, *COMMON, *DEVICE_FLAGS, *extra,
               *PER_SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if resource_usage:
            cmd.append("-Rpass-analysis=kernel-resource-usage")
        jobs.append((src, obj, cmd))
    for src in CXX_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        cmd = [hipcc, "-x", "c++", *COMMON, "-D__HIP_PLATFORM_AMD__",
               "-I" + os.path.join(_rocm(), "include"), "-c",
               os.path.join(CSRC, src), "-o", obj]
        jobs.append((src, obj, cmd))
    procs = [(src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
             for src, obj, cmd in jobs]
    failed = []
    for src, obj, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        lines = [ln for ln in out.splitlines() if "not a recognized feature" not in ln]
        if resource_usage or verbose or p.returncode != 0:
            sys.stdout.write("\n".join(lines) + ("\n" if lines else ""))
        if p.returncode != 0:
            failed.append(src)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(failed))
    tmp = lib + ".tmp%d" % os.getpid()
    link = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp,
            *[obj for _, obj, _ in jobs]]
    subprocess.check_call(link)
    os.replace(tmp, lib)
    with open(lib + ".srchash", "w") as fh:   # which sources this library was built from
        fh.write(source_hash() + "\n")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--phase-clocks", action="store_true",
                    help="build libkda_clocks.so, whose kernels record phase clocks (kda_phase_clocks)")
    args = ap.parse_args()
    print(build(resource_usage=args.resource_usage, phase_clocks=args.phase_clocks))
