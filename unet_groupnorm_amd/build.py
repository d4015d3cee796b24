"""Build step for libgn.so, the HIP GroupNorm library (gfx950 only), and for
libgn_probe.so, the measurement kernels that the benchmark and the tests use beside it.

libgn.so: the C ABI (csrc/gn_api.cpp), the launch plans (csrc/gn_plan.cpp) and the kernels
(csrc/gn_kernels.hip for NCDHW, csrc/gn_kernels_cl.hip for channels-last,
csrc/gn_kernels_shard.hip for spatial shards), compiled with hipcc one source at a time in
parallel, then linked into ``unet_groupnorm_amd/libgn.so``.

libgn_probe.so (csrc/probe_kernels.hip): streaming read, write and copy kernels that measure
the device's achievable HBM rates, and an atomic-accumulation reduction kept as the negative
control of the determinism tests. It is not part of the GroupNorm path and libgn.so does not
link it.
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgn.so")
PROBE_LIB = os.path.join(HERE, "libgn_probe.so")
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["gn_plan.cpp", "gn_api.cpp", "gn_kernels.hip", "gn_kernels_cl.hip", "gn_kernels_shard.hip"]
PROBE_SOURCES = ["probe_kernels.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Arithmetic exactly as written: no implicit contraction into fused multiply-adds
    # (the kernels spell out every fma they want).
    "-ffp-contract=off",
    # No packed-fp32 instructions (v_pk_add/mul/fma_f32) anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _link(sources, out, extra, verbose):
    os.makedirs(OBJDIR, exist_ok=True)
    stem = os.path.splitext(os.path.basename(out))[0]
    objs = [os.path.join(OBJDIR, f"{stem}.{os.path.splitext(s)[0]}.o") for s in sources]
    cmds = [[HIPCC] + FLAGS + (extra or []) + ["-I", INCLUDE, "-I", CSRC, "-x", "hip", "-c",
                                               os.path.join(CSRC, s), "-o", o]
            for s, o in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False, extra=None, out=None) -> str:
    """Compiles libgn.so (and libgn_probe.so beside it when building the default library)."""
    lib = _link(SOURCES, out or LIB, extra, verbose)
    if out is None:
        _link(PROBE_SOURCES, PROBE_LIB, extra, verbose)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
