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
# the same library with the kernels' bounds checks compiled in (LORA_SGMV_DEBUG)
DEBUG_LIB = os.path.join(PKG, "libhab_lora_debug.so")
DEBUG_FLAGS = ["-DLORA_SGMV_DEBUG"]
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


def _start(out: str, extra):
    cmd = [HIPCC, *FLAGS, *extra, "-o", out + ".tmp", *SOURCES]
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


def _finish(proc, out: str) -> str:
    text = proc.communicate()[0]
    noise = "is not a recognized feature for this target"
    log = "\n".join(l for l in text.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{log}")
    if log.strip():
        print(log, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def build(out: str = LIB, extra=()) -> str:
    return _finish(_start(out, extra), out)


def build_all() -> list:
    """The library and its debug build, compiled side by side."""
    jobs = [(LIB, _start(LIB, ())), (DEBUG_LIB, _start(DEBUG_LIB, DEBUG_FLAGS))]
    return [_finish(proc, out) for out, proc in jobs]


# The host sources built with g++ alone (no device code: host_only.cpp
# stands in for the kernel launchers) under AddressSanitizer and
# UndefinedBehaviorSanitizer, to run the host-side tests against.
SANITIZE = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all"]


def host_sanitized(out: str) -> str:
    srcs = [os.path.join(CSRC, "lora_sgmv.cpp"), os.path.join(CSRC, "exchange.cpp"),
            os.path.join(CSRC, "host_only.cpp")]
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", *SANITIZE,
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", INCLUDE, "-I", CSRC, *srcs,
           "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed ({res.returncode}):\n{res.stdout}")
    return out


if __name__ == "__main__":
    print(build_all())
