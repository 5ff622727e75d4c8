"""Builds the in-tree HIP library ``libcascade_attn.so`` for gfx950.

Usage: ``python -m shared_prefix_attention_amd.build`` (or ``__graft_entry__.build()``).
Compiles every time it is called; the result lands next to this file so that
it travels with the source tree.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcascade_attn.so")

HIP_SOURCES = ["run.hip"]
HOST_SOURCES = ["plan.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed-fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: no AGPR <-> VGPR copies around the softmax rescale
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def check_resource_usage(remarks: str) -> list:
    """Parses hipcc's kernel-resource-usage remarks and returns one record per
    kernel. The LDS reads of the attention kernels are inline asm whose
    results the code waits for by hand (an explicit lgkmcnt wait that names
    the destination registers); that is only sound while the compiler keeps
    every such register in place. So a kernel that uses scratch memory
    (VGPR spills, a stack) fails the build. SGPR spills are allowed and
    reported: they go to lanes of a VGPR the compiler reserves for them
    (v_writelane / v_readlane, no memory), and lds_wait_check verifies on the
    final assembly that no instruction touches an LDS read's destination
    before its wait."""
    kernels = []
    cur = None
    for line in remarks.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            kernels.append(cur)
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|SGPRs Spill|VGPRs Spill|VGPRs|AGPRs|"
                      r"Occupancy \[waves/SIMD\]|LDS Size \[bytes/block\]|Dynamic Stack): (\S+)", line)
        if m and cur is not None:
            cur[m.group(1)] = m.group(2)
    bad = [k for k in kernels if k.get("ScratchSize [bytes/lane]", "0") != "0" or k.get("VGPRs Spill", "0") != "0"
           or k.get("Dynamic Stack", "False") != "False"]
    if not kernels:
        raise RuntimeError("no kernel-resource-usage remarks found in the HIP compile output")
    if bad:
        raise RuntimeError("kernels use scratch memory or spill VGPRs (the inline-asm LDS reads rely on "
                           "neither): " + "; ".join(f"{k['name']}: {k}" for k in bad))
    # The attention work-groups are 4 waves; the single cascade launch holds
    # two per CU (an MFMA-bound prefix item beside a bandwidth-bound suffix
    # item), so every attention kernel whose LDS leaves room for two must fit
    # two in registers as well (2 waves per SIMD).
    low = [k for k in kernels if ("attn_tile_kernel" in k["name"] or "cascade_phases_kernel" in k["name"])
           and int(k.get("LDS Size [bytes/block]", "0")) <= 80 * 1024
           and int(k.get("Occupancy [waves/SIMD]", "0")) < 2]
    if low:
        raise RuntimeError("attention kernels below two work-groups per CU: " +
                           "; ".join(f"{k['name']}: {k}" for k in low))
    return kernels


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC,
              "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    usage = []
    for src in HIP_SOURCES:
        obj = os.path.join(objdir, src + ".o")
        # the compiler's own gfx950 assembly of the same source (compiled
        # alongside the object): every inline-asm LDS read is waited for
        # before any use of its registers
        asm_path = os.path.join(objdir, src + ".s")
        asm_cmd = [hipcc, *HIPCC_FLAGS, "--cuda-device-only", "-S", "-I", INCLUDE, "-I", CSRC,
                   os.path.join(CSRC, src), "-o", asm_path]
        print("+", " ".join(asm_cmd), flush=True)
        asm_proc = subprocess.Popen(asm_cmd)
        cmd = [hipcc, *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        print("+", " ".join(cmd), flush=True)
        try:
            r = subprocess.run(cmd, capture_output=True, text=True)
        finally:
            asm_rc = asm_proc.wait()
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise subprocess.CalledProcessError(r.returncode, cmd)
        if asm_rc != 0:
            raise subprocess.CalledProcessError(asm_rc, asm_cmd)
        usage += check_resource_usage(r.stderr)
        objs.append(obj)
        from shared_prefix_attention_amd import lds_wait_check
        nfun, nreads, problems = lds_wait_check.check(open(asm_path).read())
        if problems:
            raise RuntimeError(f"{len(problems)} uses of inline-asm LDS read results before their wait:\n" +
                               "\n".join(problems[:20]))
        if verbose:
            print(f"  {nfun} kernels, {nreads} inline-asm LDS reads: every result waited for before use",
                  flush=True)
    with open(os.path.join(objdir, "kernel_resource_usage.txt"), "w") as f:
        for k in usage:
            f.write(" ".join(f"{key}={val}" for key, val in k.items()) + "\n")
    if verbose:
        print(f"  {len(usage)} kernels: no scratch, no VGPR spills; max VGPRs "
              f"{max(int(k.get('VGPRs', 0)) for k in usage)}; SGPR spills to VGPR lanes: max "
              f"{max(int(k.get('SGPRs Spill', 0)) for k in usage)}", flush=True)
    tmp = LIB + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
