"""Build step for libgn.so, the HIP GroupNorm library (gfx950 only), and for
libgn_probe.so, the measurement kernels that the benchmark and the tests use beside it.

libgn.so: the C ABI (csrc/gn_api.cpp), the launch plans (csrc/gn_plan.cpp) and the kernels
(csrc/gn_kernels.hip for NCDHW, csrc/gn_kernels_cl.hip for channels-last,
csrc/gn_kernels_shard.hip for spatial shards), compiled with hipcc one source at a time in
parallel, then linked into ``unet_groupnorm_amd/libgn.so``.

_gnbind (csrc/gn_binding.cpp, a Python extension module linked against libgn.so and torch):
the compiled marshalling of the per-step calls gn_forward and gn_backward for torch tensors.
Host code only, compiled with g++ against torch's headers.

libgn_probe.so (csrc/probe_kernels.hip): streaming read, write and copy kernels that measure
the device's achievable HBM rates, and an atomic-accumulation reduction kept as the negative
control of the determinism tests. It is not part of the GroupNorm path and libgn.so does not
link it.
"""
import os
import subprocess
import sysconfig
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
BIND_SOURCE = "gn_binding.cpp"
BIND_NAME = "_gnbind"
BIND_LIB = os.path.join(HERE, BIND_NAME + sysconfig.get_config_var("EXT_SUFFIX"))

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


def _bind_commands():
    """(compile, link) commands of the _gnbind extension module."""
    import torch
    from torch.utils.cpp_extension import include_paths, library_paths
    obj = os.path.join(OBJDIR, BIND_NAME + ".o")
    inc = [f"-I{p}" for p in include_paths()] + [f"-I{sysconfig.get_paths()['include']}", "-I/opt/rocm/include",
                                                 f"-I{INCLUDE}"]
    defs = ["-D__HIP_PLATFORM_AMD__=1", "-DUSE_ROCM=1", f"-DTORCH_EXTENSION_NAME={BIND_NAME}",
            "-DTORCH_API_INCLUDE_EXTENSION_H", f"-D_GLIBCXX_USE_CXX11_ABI={int(torch._C._GLIBCXX_USE_CXX11_ABI)}"]
    compile_cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-w"] + defs + inc + \
        ["-c", os.path.join(CSRC, BIND_SOURCE), "-o", obj]
    tlib = library_paths()[0]
    link_cmd = ["g++", "-shared", obj, "-o", BIND_LIB + ".tmp", f"-L{HERE}", "-lgn", "-Wl,-rpath,$ORIGIN",
                f"-L{tlib}", "-lc10", "-lc10_hip", "-ltorch", "-ltorch_cpu", "-ltorch_hip", "-ltorch_python",
                f"-Wl,-rpath,{tlib}"]
    return compile_cmd, link_cmd


def _link(sources, out, extra, verbose, also=()):
    os.makedirs(OBJDIR, exist_ok=True)
    stem = os.path.splitext(os.path.basename(out))[0]
    objs = [os.path.join(OBJDIR, f"{stem}.{os.path.splitext(s)[0]}.o") for s in sources]
    cmds = [[HIPCC] + FLAGS + (extra or []) + ["-I", INCLUDE, "-I", CSRC, "-x", "hip", "-c",
                                               os.path.join(CSRC, s), "-o", o]
            for s, o in zip(sources, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds) + len(also), 8)) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds + list(also)]:
            f.result()
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False, extra=None, out=None) -> str:
    """Compiles libgn.so (and, when building the default library, _gnbind against it and
    libgn_probe.so beside it)."""
    if out is not None:
        return _link(SOURCES, out, extra, verbose)
    os.makedirs(OBJDIR, exist_ok=True)
    bind_compile, bind_link = _bind_commands()
    lib = _link(SOURCES, LIB, extra, verbose, also=[bind_compile])
    _run(bind_link, verbose)
    os.replace(BIND_LIB + ".tmp", BIND_LIB)
    _link(PROBE_SOURCES, PROBE_LIB, extra, verbose)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
