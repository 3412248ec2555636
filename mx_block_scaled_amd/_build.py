"""Build of libmxfp8.so (the HIP library) for gfx950 with hipcc, in-tree.

The sources are compiled with ``-Xclang -target-feature -Xclang -packed-fp32-ops`` so the
compiler never emits packed fp32 arithmetic (hipcc's host pass warns that it does not know the
feature; that warning is harmless).
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxfp8.so")
SOURCES = ["mx_api.cpp", "mx_quant.hip", "mx_prepack.hip", "mx_gemm.hip", "mx_small_m.hip",
           "mx_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps.append(os.path.join(ROOT, "include", "mxfp8.h"))
    return any(os.path.getmtime(d) > t for d in deps)


def build(verbose=False):
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + sources()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmxfp8.so")
    if verbose:
        noise = "packed-fp32-ops' is not a recognized feature"
        out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        if out.strip():
            sys.stderr.write(out + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
