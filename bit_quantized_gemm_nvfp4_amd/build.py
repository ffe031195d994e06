"""Build the gfx950 shared library ``libnvfp4.so`` from ``csrc/*.hip``.

Every source is compiled by hipcc for gfx950 only, with packed-FP32
instructions disabled (the compiler may otherwise emit v_pk_{add,mul,fma}_f32
from ordinary float code), then linked into one shared library that exports
the C ABI of ``include/nvfp4.h``.

    python -m bit_quantized_gemm_nvfp4_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libnvfp4.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the NVFP4 library)")


COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs, procs = [], []
    for s in srcs:
        o = os.path.join(BUILD_DIR, os.path.basename(s) + ".o")
        objs.append(o)
        cmd = [cc, *COMMON_FLAGS, "-c", s, "-o", o]
        if verbose:
            print(" ".join(cmd))
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for s, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        # hipcc's host pass does not know the packed-fp32 feature; that note is harmless
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((s, text))
        elif text.strip() and verbose:
            print(text)
    if failed:
        for s, t in failed:
            sys.stderr.write(f"--- {s}\n{t}\n")
        raise RuntimeError("HIP compilation failed")
    tmp = OUT + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        sys.stderr.write(r.stdout.decode(errors="replace"))
        raise RuntimeError("linking libnvfp4.so failed")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
