"""Build liblmoe.so (the HIP library) in-tree for gfx950.

Every HIP source is compiled with hipcc for gfx950 only, with packed-fp32
instructions disabled (-Xclang -target-feature -Xclang -packed-fp32-ops),
and linked into latent_mixture_experts_amd/liblmoe.so.
"""

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblmoe.so")
BUILD = os.path.join(PKG, "_build")
SOURCES = ["api.hip", "layout.hip", "decode.hip", "prefill.hip", "ple.hip"]
ARCH = "gfx950"


def hipcc():
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")


def flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr[-8000:]))
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-8000:])
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
