"""Build libtilegemm.so in-tree with hipcc for gfx950.

    python -m tiled_dense_gemm_tile_amd.build

Each translation unit under csrc/ is compiled on its own (in parallel) and
linked into one shared library next to this file.

Every kernel's register use is read from the compiler's resource-usage
remarks, written to _build/resource_usage.txt, and the build fails if any
kernel uses scratch memory or spills registers: the accumulators of the
MFMA kernels are tied to inline-asm MFMAs whose register accesses the
compiler cannot see, so a spilled accumulator would be read or written at
the wrong time and give silently wrong results.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libtilegemm.so")
OBJDIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         # no packed-fp32 instruction selection (v_pk_*_f32 are never emitted)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


class ResourceError(RuntimeError):
    """A kernel uses scratch memory or spills registers."""


def resource_usage(remarks: str):
    """Per-kernel usage from -Rpass-analysis=kernel-resource-usage output:
    a list of dicts (name, VGPRs, AGPRs, ScratchSize, VGPRs Spill, ...)."""
    kernels, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            kernels.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[bytes/lane\])?: (\d+) \[", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return kernels


def offenders(kernels):
    # (SGPR spills go to VGPR lanes, not memory: they do not count)
    return [k for k in kernels if k.get("ScratchSize", 0) or k.get("VGPRs Spill", 0)]


def compile_unit(src, obj, extra=()):
    """hipcc -c with the library's flags; returns the kernels' resource usage
    and raises ResourceError if any of them spills or uses scratch."""
    cmd = [HIPCC] + FLAGS + ["-Rpass-analysis=kernel-resource-usage"] + list(extra) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    kernels = resource_usage(r.stderr)
    bad = offenders(kernels)
    if bad:
        raise ResourceError("%s: kernels spilling or using scratch:\n%s" % (
            os.path.basename(src), "\n".join("  %s scratch %d B/lane, %d VGPRs spilled" % (
                k["name"], k.get("ScratchSize", 0), k.get("VGPRs Spill", 0)) for k in bad)))
    return kernels


def _compile(src):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    return obj, compile_unit(src, obj)


def build(verbose: bool = True) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError("hipcc not found at %s" % HIPCC)
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        done = list(ex.map(_compile, srcs))
    objs = [o for o, _ in done]
    kernels = [k for _, ks in done for k in ks]
    with open(os.path.join(OBJDIR, "resource_usage.txt"), "w") as f:
        for k in sorted(kernels, key=lambda k: k["name"]):
            f.write("%-4d VGPR %-4d AGPR %-6d LDS scratch %d  %s\n" % (
                k.get("VGPRs", 0), k.get("AGPRs", 0), k.get("LDS Size", 0), k.get("ScratchSize", 0), k["name"]))
    tmp = OUT + ".tmp%d" % os.getpid()
    # -z defs: an instance that silently lost its kernels fails the link here
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, OUT)
    if verbose:
        print("built %s: %d kernels, none spilling (max %d VGPR + %d AGPR); per-kernel usage in %s" % (
            OUT, len(kernels), max(k.get("VGPRs", 0) for k in kernels), max(k.get("AGPRs", 0) for k in kernels),
            os.path.join(OBJDIR, "resource_usage.txt")), file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()
