"""Compile the HIP library (libmoe.so) for gfx950 with hipcc, in-tree, and
the host-only validation library (libmoe_host.so: the argument checks and
workspace layouts of the C ABI, no HIP runtime) with g++."""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
HOST_LIB = os.path.join(HERE, "libmoe_host.so")
SOURCES = ["api.cpp", "validate.cpp", "decode.hip", "prefill.hip", "repack.hip", "probe.hip", "attn.hip"]
HOST_SOURCES = ["validate.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    # code object v5: loadable by the HIP runtime PyTorch ships (ROCm 7.0)
    "-mcode-object-version=5",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # packed FP32 instructions off for every device function
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc():
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found")
    return p


def build(verbose=False):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + ["-I", os.path.join(ROOT, "include")]
    # .cpp files are host-and-device C++ for hipcc as well
    cmd += ["-x", "hip"] + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + errs)
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def build_host(out=HOST_LIB, extra_flags=()):
    """The validation unit alone, with g++ (no HIP headers or runtime).
    extra_flags: e.g. sanitizer options for a host-only test build."""
    tmp = out + ".tmp"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-Wall", "-Wextra", *extra_flags,
           "-I", os.path.join(ROOT, "include")] + [os.path.join(CSRC, s) for s in HOST_SOURCES] + ["-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_host()
