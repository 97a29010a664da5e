"""Build libmbt.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m memory_bound_transformer_amd.build        (or python .../build.py)

Every source under csrc/ is compiled by hipcc for --offload-arch=gfx950 with
packed-fp32 instruction selection and floating-point contraction switched
off, then linked into
memory_bound_transformer_amd/libmbt.so next to the Python binding.  Only the
symbols declared in include/mbt.h are exported.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmbt.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["mbt_api.cpp", "qknorm_rope.hip", "rope.hip", "rmsnorm.hip", "gated_act.hip",
           "stream_copy.hip"]

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
         "-Wall", "-Wno-unused-function",
         # every fp32 operation rounds where the source writes it: no product is
         # fused with an add or with a narrowing conversion (v_fma_mix*) unless
         # the source calls fmaf, so every kernel rounds in the same places
         "-ffp-contract=off",
         # no v_pk_*_f32 from the compiler: scalar fp32 arithmetic only
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for _, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp,
           *[o for o, _ in results]]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
