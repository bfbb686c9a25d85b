"""Build libattamba.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m ssm_compressed_chunked_amd.build

Objects go to ssm_compressed_chunked_amd/_build/, the library to
ssm_compressed_chunked_amd/libattamba.so. Every call compiles from scratch.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattamba.so")
# the issue-rate microbenchmark behind the instruction-issue rooflines (not part of libattamba)
PROBE_SRC = "issue_probe.hip"
PROBE_LIB = os.path.join(PKG, "libattamba_probe.so")
SOURCES = ["boundaries.hip", "kvssm_scan.hip", "chunk_attn.hip", "attn_mfma.hip", "decode.hip", "proj_gemm.hip",
           "kvssm_scan_bwd.hip", "chunk_attn_bwd.hip", "attn_mfma_bwd.hip", "abi.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed FP32 instructions are switched off for device code (the host pass of hipcc warns that
# it does not know the feature; that warning is harmless).
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


# Matrix-core accumulators in VGPRs (not AGPRs) so the softmax rescale of the output
# accumulator needs no AGPR<->VGPR copies.
EXTRA = {"attn_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"], "proj_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "attn_mfma_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    if os.path.isdir(BUILD):
        shutil.rmtree(BUILD)
    os.makedirs(BUILD)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(pair):
        src, obj = pair
        return _run([HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj])

    probe_obj = os.path.join(BUILD, PROBE_SRC.replace(".hip", ".o"))
    jobs = list(zip(SOURCES, objs)) + [(PROBE_SRC, probe_obj)]
    with ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        logs = list(ex.map(compile_one, jobs))
    for lib, lib_objs in ((LIB, objs), (PROBE_LIB, [probe_obj])):
        tmp = lib + ".tmp"
        logs.append(_run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *lib_objs]))
        os.replace(tmp, lib)
    if verbose:
        for l in logs:
            if l.strip():
                print(l)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
