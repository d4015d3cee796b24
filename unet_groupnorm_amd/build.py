"""Build step for libgn.so, the HIP GroupNorm library (gfx950 only).

Compiles the C ABI (csrc/gn_api.cpp), the launch plans (csrc/gn_plan.cpp) and the
kernels (csrc/gn_kernels.hip for NCDHW, csrc/gn_kernels_cl.hip for channels-last) with
hipcc into ``unet_groupnorm_amd/libgn.so``.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgn.so")
SOURCES = ["gn_plan.cpp", "gn_api.cpp", "gn_kernels.hip", "gn_kernels_cl.hip", "gn_kernels_shard.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # Arithmetic exactly as written: no implicit contraction into fused multiply-adds
    # (the kernels spell out every fma they want).
    "-ffp-contract=off",
    # No packed-fp32 instructions (v_pk_add/mul/fma_f32) anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra=None, out=None) -> str:
    out = out or LIB
    cmd = [HIPCC] + FLAGS + (extra or []) + ["-I", INCLUDE, "-I", CSRC, "-x", "hip"] + \
        [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
