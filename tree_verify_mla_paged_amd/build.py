"""Build libtreeverify.so in-tree for gfx950 with hipcc (no JIT, no pip install)."""
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SO = os.path.join(PKG, "libtreeverify.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in
           ("tv_split.hip", "tv_merge.hip", "tv_pack.hip", "tv_append.hip", "tv_static.hip",
            "tv_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         # packed fp32 VALU ops stay off (see the kernel notes)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # the split kernel's software-pipelined QK chain (36 MFMAs with other
         # work between them) must unroll fully; it exceeds the default limit
         "-mllvm", "-pragma-unroll-threshold=1000000",
         "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]


# Per-kernel resource remarks of a device compile: [(kernel, scratch bytes per
# lane, VGPRs spilled)].  Every kernel here keeps its state in registers and
# LDS; a spill to scratch (e.g. the 256 accumulator registers of the split
# kernel demoted to memory) would still be correct but many times slower, so
# the build refuses it.
_NAME = re.compile(r"remark: Function Name: (\S+)")
_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")
_VSPILL = re.compile(r"remark:\s+VGPRs Spill: (\d+)")


def resource_usage(remarks: str):
    out, name, scratch = [], None, 0
    for line in remarks.splitlines():
        m = _NAME.search(line)
        if m:
            name = m.group(1)
            continue
        m = _SCRATCH.search(line)
        if m and name:
            scratch = int(m.group(1))
            continue
        m = _VSPILL.search(line)
        if m and name:
            out.append((name, scratch, int(m.group(1))))
            name = None
    return out


def build(verbose: bool = False) -> str:
    objs = []
    for src in SOURCES:
        obj = os.path.join(PKG, "csrc", os.path.basename(src) + ".o")
        extra = ["-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
        cmd = [HIPCC] + FLAGS + extra + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed on " + src)
        if extra:
            usage = resource_usage(r.stderr)
            if not usage and "__global__" in open(src).read():
                raise RuntimeError("no kernel resource remarks from hipcc for " + src)
            bad = [u for u in usage if u[1] or u[2]]
            if bad:
                raise RuntimeError("kernels spilling to scratch in %s: %s" % (
                    os.path.basename(src),
                    ", ".join("%s (%d bytes/lane, %d VGPRs)" % b for b in bad)))
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", SO + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
