"""Builds libq8s.so (the HIP library, gfx950) in place, next to this file.

    python q8_gemv_sparse_amd/build.py        # or build() from Python (the package
                                              # itself refuses to import unbuilt)

hipcc compiles every csrc/*.hip for gfx950 only.  Flags: -O3; float32
division and square root correctly rounded (the Q8_0 quantiser's scale and
its reciprocal are IEEE divisions); no floating-point contraction except the
fused multiply-adds the kernels write out; packed-fp32 instructions disabled.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libq8s.so")
ARCH = "gfx950"

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    "-fvisibility=hidden",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def build(verbose=False, jobs=8):
    """Compiles each translation unit, then links libq8s.so.  Always rebuilds."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc")]
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc] + [f for f in FLAGS if f not in ("-shared",)] + inc + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
    if lines:
        print("\n".join(lines), file=sys.stderr)
    if p.returncode != 0:
        raise RuntimeError("hipcc failed on %s" % src)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
