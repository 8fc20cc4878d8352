"""Build libss.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libss.so")
SOURCES = ["ss_fwd.hip", "ss_bwd.hip", "ss_conv.hip", "ss_ssd.hip", "ss_probe.hip", "ss_noalloc.hip", "ss_abi.cpp"]
HEADERS = ["ss_device.h", "ss_internal.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed-FP32 VALU forms are disabled for every HIP translation unit.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I" + os.path.join(ROOT, "include")]


def _inputs():
    files = [os.path.join(CSRC, f) for f in SOURCES + HEADERS]
    files.append(os.path.join(ROOT, "include", "ss.h"))
    return files


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in _inputs())


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every source to an object, then link libss.so; returns its path."""
    if not force and not stale():
        return LIB
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    # one compiler per source, at most `jobs` at a time
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1)))
    pending = list(SOURCES)
    while pending or procs:
        while pending and len(procs) < jobs:
            src = pending.pop(0)
            obj = os.path.join(objdir, src + ".o")
            cmd = [HIPCC] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        src, pr = procs.pop(0)
        out, _ = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out)
            for _, other in procs:
                other.kill()
            raise RuntimeError("hipcc failed on %s" % src)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libss.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose="-v" in sys.argv))
