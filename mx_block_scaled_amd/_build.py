"""Build of libmxfp8.so (the HIP library) for gfx950 with hipcc, in-tree.

The sources are compiled with ``-Xclang -target-feature -Xclang -packed-fp32-ops`` so the
compiler never emits packed fp32 arithmetic (hipcc's host pass warns that it does not know the
feature; that warning is harmless).  Each source is compiled to an object in parallel, then the
objects are linked.  ``build_peaks`` builds libmxpeaks.so, the microbenchmarks that give
bench.py its attainable-peak denominators; the layer library does not contain them.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmxfp8.so")
PEAKS_LIB = os.path.join(HERE, "libmxpeaks.so")
SOURCES = ["mx_api.cpp", "mx_quant.hip", "mx_prepack.hip", "mx_gemm.hip", "mx_small_m.hip",
           "mx_noalloc.hip"]
PEAKS_SOURCES = [os.path.join("bench", "mx_peaks.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]
NOISE = "packed-fp32-ops' is not a recognized feature"


def sources():
    return [os.path.join(CSRC, s) for s in SOURCES]


def stale():
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = sources() + [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".h")]
    deps.append(os.path.join(ROOT, "include", "mxfp8.h"))
    return any(os.path.getmtime(d) > t for d in deps)


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if NOISE not in l)
    return r.returncode, out


def _link(srcs, lib, verbose):
    tmpdir = tempfile.mkdtemp(prefix="mxbuild")
    try:
        objs = [os.path.join(tmpdir, "%d.o" % i) for i in range(len(srcs))]
        jobs = [[HIPCC] + CFLAGS + (["-x", "hip"] if s.endswith(".hip") else []) +
                ["-c", s, "-o", o] for s, o in zip(srcs, objs)]
        with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
            res = list(ex.map(_run, jobs))
        for (rc, out), s in zip(res, srcs):
            if rc != 0:
                sys.stderr.write(out + "\n")
                raise RuntimeError("hipcc failed compiling %s" % os.path.basename(s))
            if verbose and out.strip():
                sys.stderr.write(out + "\n")
        tmp = lib + ".tmp%d" % os.getpid()
        rc, out = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
        if rc != 0:
            sys.stderr.write(out + "\n")
            raise RuntimeError("hipcc failed linking %s" % os.path.basename(lib))
        os.replace(tmp, lib)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return lib


def build(verbose=False):
    return _link(sources(), LIB, verbose)


def build_peaks(verbose=False):
    return _link([os.path.join(CSRC, s) for s in PEAKS_SOURCES], PEAKS_LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_peaks(verbose=True))
