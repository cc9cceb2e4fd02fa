"""Build the HIP library ``libattnfuse.so`` for gfx950, in-tree.

Each ``csrc/*.hip`` file is compiled to an object with ``hipcc`` (in parallel),
then all objects are linked into ``attention_attnfuse_fwd_amd/libattnfuse.so``.
Usage: ``python -m attention_attnfuse_fwd_amd.build`` or ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(os.path.dirname(PKG_DIR), "_build")
LIB_NAME = "libattnfuse.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Keep the compiler from forming packed-fp32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    # dma16() lists m0 as clobbered; clang warns that m0 is reserved.
    "-Wno-inline-asm",
]


# Per-source extra flags.  In the two- and four-wave forward instances (one
# wave per SIMD) and the backward's block-sparse dQ kernels the register
# allocator otherwise parks the MFMA accumulators in AGPRs and copies every
# score out of them (about a hundred extra moves per key tile in the
# forward); forcing the VGPR form of the MFMAs keeps them in VGPRs without
# new spills.  The eight-wave forward instances and the other backward
# kernels use no AGPRs either way.
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA_FLAGS = {
    **{f"fwd_bf16_d{d}_nw{nw}.hip": _VGPR_FORM for d in (64, 128) for nw in (2, 4)},
    **{f"bwd_d{d}.hip": _VGPR_FORM for d in (64, 128)},
}


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libattnfuse.so")


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Kernels that order their direct-to-LDS loads by counting vmcnt: VGPR
# spills would add scratch loads and stores to that count, so any VGPR spill
# or scratch use in them fails the build.  (SGPR spills live in VGPR lanes
# and issue no memory instruction.)
NO_SCRATCH_KERNELS = ("fwd_bf16_kernel",)


def kernel_resources(remarks: str) -> dict:
    """Parse clang's kernel-resource-usage remarks: {kernel: {field: int}}."""
    out, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*?): (\d+)", line)
        if m and name:
            out[name][m.group(1).strip()] = int(m.group(2))
    return out


def _compile(hipcc: str, src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []),
           "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    for kname, r in kernel_resources(res.stderr).items():
        if any(k in kname for k in NO_SCRATCH_KERNELS):
            spill = r.get("VGPRs Spill", 0)
            scratch = r.get("ScratchSize [bytes/lane]", 0)
            if spill or scratch:
                raise RuntimeError(f"{kname} in {os.path.basename(src)} spills ({spill} registers, "
                                   f"{scratch} B scratch per lane); its DMA wait counts assume none")
    return obj


def build(jobs: int | None = None, verbose: bool = True) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), srcs))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} from {len(srcs)} sources", file=sys.stderr)
    return LIB_PATH


if __name__ == "__main__":
    build()
