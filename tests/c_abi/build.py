"""Build tests/c_abi/abi_roundtrip: a plain C program that calls libmbt
through include/mbt.h (device buffers from the HIP runtime, no Python) and
checks the results against the CPU oracle.  Test infrastructure: it links
the oracle, which the product library never does.  Needs libmbt.so and
liboracle.so built first."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_roundtrip.c")
EXE = os.path.join(HERE, "abi_roundtrip")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out=EXE):
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
           SRC, "-o", out,
           "-L", os.path.join(ROOT, "memory_bound_transformer_amd"), "-lmbt",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           f"-L{ROCM}/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../memory_bound_transformer_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", f"-Wl,-rpath,{ROCM}/lib"]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
