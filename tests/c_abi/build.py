"""Compile tests/c_abi/sgmv_from_c.c: a C program that drives the library
through its C ABI alone (HIP runtime calls for memory and the stream), with
the CPU oracle linked as its reference.  Test infrastructure."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "sgmv_from_c.c")
BIN = os.path.join(HERE, "sgmv_from_c")
ROCM = "/opt/rocm"


def build(out: str = BIN) -> str:
    pkg = os.path.join(ROOT, "heterogeneous_adapter_batching_amd")
    orc = os.path.join(ROOT, "oracle")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-o", out + ".tmp", "-L", pkg, "-lhab_lora", "-L", orc, "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm", "-fopenmp",
           "-Wl,-rpath,$ORIGIN/../../heterogeneous_adapter_batching_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stdout}")
    if res.stdout.strip():
        print(res.stdout, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
