"""Compile the HIP library liblinattn.so in-tree for gfx950.

    python -m chunked_linear_attention_packed_amd.build

The host code (pack.cpp: packer and planners; cache.cpp: view-state cache
directory) is compiled with g++; the kernels and their host entry points
(scan.hip: the linear-attention scan; piece.hip: its d = 64 bf16 path;
attn.hip: the tree-masked softmax attention) with hipcc; all are linked into
one shared library next to this file.  Always recompiles.  Every kernel is
designed to fit its registers: a kernel that needs scratch memory (register
spills, or a private array) fails the build.
"""
import os
import re
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblinattn.so")
HOST_SOURCES = ["pack.cpp", "cache.cpp"]
HIP_SOURCES = ["scan.hip", "piece.hip", "attn.hip"]

HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: avoids AGPR->VGPR copies before the bf16 packing
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    # the first kernel arguments arrive in SGPRs at wave launch (no load)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wextra", "-Wno-unused-function",
]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblinattn.so)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return out


def _scratch_kernels(remarks):
    """(kernel, bytes per lane) of every kernel with scratch memory, from
    the compiler's kernel-resource-usage remarks."""
    found, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name and int(m.group(1)) > 0:
            found.append((name, int(m.group(1))))
    return found


def build(verbose=False):
    hipcc = _hipcc()
    with tempfile.TemporaryDirectory(prefix="linattn_build_") as tmp:
        host_o = []
        for name in HOST_SOURCES:
            obj = os.path.join(tmp, name.replace(".cpp", ".o"))
            _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-c",
                  os.path.join(CSRC, name), "-o", obj], verbose)
            host_o.append(obj)
        dev_o = []
        for name in HIP_SOURCES:
            obj = os.path.join(tmp, name.replace(".hip", ".o"))
            out = _run([hipcc] + HIP_FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-I",
                                              INCLUDE, "-c", os.path.join(CSRC, name), "-o", obj],
                       False)
            spills = _scratch_kernels(out)
            if spills:
                raise RuntimeError(f"{name}: kernels using scratch memory: {spills}")
            dev_o.append(obj)
        tmp_lib = LIB + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC"] + host_o + dev_o +
             ["-o", tmp_lib], verbose)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
