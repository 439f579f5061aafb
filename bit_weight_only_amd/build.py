"""Build liblbq.so in-tree: hipcc for the HIP sources (gfx950), g++ for the
host packer, one shared library next to this file.

    python -m bit_weight_only_amd.build        # or bit_weight_only_amd.build.build()
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblbq.so")

HIP_SOURCES = ["api.hip", "rotate.hip", "gemv.hip", "gemv_mfma.hip", "gemm.hip", "gemm_rtn.hip", "gemm_mx.hip", "pvq.hip", "pvq_mx.hip", "moe.hip", "moe_mx.hip", "unpack.hip", "measure.hip", "readout.hip"]
HOST_SOURCES = ["pack.cpp", "gptq.cpp"]

ARCH = os.environ.get("LBQ_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # never emit packed-fp32 VALU ops (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the GEMM rescales them every group, and the
    # AGPR form would add a copy in and out per value
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result",
]
HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-ffp-contract=off", "-pthread",
              "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "is not a recognized feature for this target" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


# host-side sanitizers (address, undefined behaviour) for the checking build:
# applied to the host pass only, the GPU code is built as usual
SAN_HOST = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]
LIB_SANITIZED = os.path.join(PKG, "_build_san", "liblbq_san.so")


def build(verbose: bool = False, jobs: int | None = None, sanitize: bool = False) -> str:
    """Compile every source and link liblbq.so; returns the library path.

    sanitize=True builds _build_san/liblbq_san.so instead: every host-side
    part (the packers, the argument checks and launch code of the C ABI) under
    AddressSanitizer and UndefinedBehaviorSanitizer, all of it with the ROCm
    clang so one sanitizer runtime serves the process (load it with LD_PRELOAD
    of clang's libclang_rt.asan-x86_64.so and point LBQ_LIBRARY at the file).
    """
    bdir = os.path.join(PKG, "_build_san") if sanitize else BUILD
    os.makedirs(bdir, exist_ok=True)
    jobs = jobs or min(8, os.cpu_count() or 4)
    cmds = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        san = [f for flag in SAN_HOST for f in ("-Xarch_host", flag)] if sanitize else []
        cmds.append([HIPCC, *HIP_FLAGS, *san, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(bdir, src + ".o")
        if sanitize:
            clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang++")
            cmds.append([clang, *HOST_FLAGS, *SAN_HOST, "-c", os.path.join(CSRC, src), "-o", obj])
        else:
            cmds.append(["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with cf.ThreadPoolExecutor(jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    lib = LIB_SANITIZED if sanitize else LIB
    tmp = lib + ".tmp"
    link_san = ["-shared-libsan", *[f for flag in SAN_HOST[:1] for f in ("-Xarch_host", flag)]] if sanitize else []
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_san, "-o", tmp, *objs, "-pthread"])
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
