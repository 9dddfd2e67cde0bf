"""Build libtreeverify.so in-tree for gfx950 with hipcc (no JIT, no pip install)."""
import os
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


def build(verbose: bool = False) -> str:
    objs = []
    for src in SOURCES:
        obj = os.path.join(PKG, "csrc", os.path.basename(src) + ".o")
        cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed on " + src)
        objs.append(obj)
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", SO + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(SO + ".tmp", SO)
    return SO


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
