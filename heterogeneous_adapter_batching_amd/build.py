"""Build the gfx950 library libhab_lora.so in-tree with hipcc.

The library is the C ABI of include/lora_sgmv.h: host code (pool, plan,
validation) and the HIP kernels, linked into one shared object that the
Python binding loads with ctypes.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhab_lora.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = [os.path.join(CSRC, "lora_sgmv.cpp"), os.path.join(CSRC, "exchange.cpp"),
           os.path.join(CSRC, "kernels.hip")]

# Packed float32 ALU ops are switched off for all device code; the compiler's
# host pass warns that it does not know the feature, which is harmless.
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
         "-Wall", "-Wextra", "-Wno-unused-parameter",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def build(out: str = LIB, extra=()) -> str:
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "is not a recognized feature for this target"
    log = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{log}")
    if log.strip():
        print(log, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build())
