"""Loads libgn.so (the HIP GroupNorm library) and declares its C ABI for ctypes.

There is no fallback: if the library has not been built, importing the package
raises, so nothing can silently run anything other than the HIP kernels.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgn.so")

# Status codes and dtype codes of include/gn.h.
GN_OK = 0
GN_F32, GN_BF16, GN_F16 = 0, 1, 2
GN_ACT_NONE, GN_ACT_RELU = 0, 1
STATUS_NAMES = {
    0: "GN_OK", 1: "GN_ERR_NULL", 2: "GN_ERR_SHAPE", 3: "GN_ERR_GROUPS", 4: "GN_ERR_DTYPE",
    5: "GN_ERR_EPS", 6: "GN_ERR_WORKSPACE", 7: "GN_ERR_ALIGN", 8: "GN_ERR_DEVICE", 9: "GN_ERR_LAUNCH",
    10: "GN_ERR_ACTIVATION", 11: "GN_ERR_LAYOUT", 12: "GN_ERR_SCRATCH",
}
# Size of the static scratch array that gn_forward_noalloc uses as its workspace.
GN_NOALLOC_SCRATCH_BYTES = 1 << 20


class GnPlanInfo(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
        ("chunks_per_row", ctypes.c_int64),
        ("jobs", ctypes.c_int64),
        ("partials_per_group", ctypes.c_int64),
        ("block", ctypes.c_int32),
        ("vectors_per_step", ctypes.c_int32),
        ("apply_chunk", ctypes.c_int64),
        ("apply_chunks_per_row", ctypes.c_int64),
        ("apply_jobs", ctypes.c_int64),
        ("apply_block", ctypes.c_int32),
        ("apply_vectors", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("resident_forward", ctypes.c_int32),
        ("resident_backward", ctypes.c_int32),
        ("resident_block_forward", ctypes.c_int32),
        ("resident_vectors_forward", ctypes.c_int32),
        ("resident_block_backward", ctypes.c_int32),
        ("resident_vectors_backward", ctypes.c_int32),
        ("fold_chunk", ctypes.c_int64),
        ("fold_chunks_per_row", ctypes.c_int64),
        ("fold_jobs", ctypes.c_int64),
        ("resident_backward_split", ctypes.c_int32),
    ]


class GnPlanInfoCL(ctypes.Structure):
    _fields_ = [
        ("chunk", ctypes.c_int64),
        ("jobs_per_sample", ctypes.c_int64),
        ("jobs", ctypes.c_int64),
        ("voxels_per_round", ctypes.c_int64),
        ("apply_chunk", ctypes.c_int64),
        ("apply_jobs_per_sample", ctypes.c_int64),
        ("apply_jobs", ctypes.c_int64),
        ("block", ctypes.c_int32),
        ("rounds_per_step", ctypes.c_int32),
        ("apply_rounds", ctypes.c_int32),
        ("groups_per_vector", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("resident_forward", ctypes.c_int32),
        ("resident_backward", ctypes.c_int32),
        ("resident_block_forward", ctypes.c_int32),
        ("resident_vectors_forward", ctypes.c_int32),
        ("resident_block_backward", ctypes.c_int32),
        ("resident_vectors_backward", ctypes.c_int32),
    ]


def _declare(lib):
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "gn_workspace_bytes": (SZ, [I64, I64, I64, I64]),
        "gn_forward": (I, [P, I, P, P, I64, I64, I64, I64, F, I, P, I, P, P, P, SZ, P]),
        "gn_forward_noalloc": (I, [P, I, P, P, I64, I64, I64, I64, F, I, P, I, P, P, P]),
        "gn_forward_stats": (I, [P, I, P, P, I64, I64, I64, I64, F, P, P, P, SZ, P]),
        "gn_forward_apply": (I, [P, I, I64, I64, I64, I64, I, P, I, P, SZ, P]),
        "gn_backward": (I, [P, I, P, I, P, P, P, P, I, I64, I64, I64, I64, P, P, P, P, SZ, P]),
        "gn_backward_reduce": (I, [P, I, P, I, P, P, P, P, I, I64, I64, I64, I64, P, P, P, SZ, P]),
        "gn_backward_apply": (I, [P, I, P, I, I64, I64, I64, I64, I, P, P, SZ, P]),
        "gn_status_string": (ctypes.c_char_p, [I]),
        "gn_plan_query": (I, [I64, I64, I64, I64, ctypes.POINTER(GnPlanInfo)]),
        "gn_abi_version": (I, []),
        "gn_workspace_bytes_cl": (SZ, [I64, I64, I64, I64]),
        "gn_forward_cl": (I, [P, I, P, P, I64, I64, I64, I64, F, I, P, I, P, P, P, SZ, P]),
        "gn_backward_cl": (I, [P, I, P, I, P, P, P, P, I, I64, I64, I64, I64, P, P, P, P, SZ, P]),
        "gn_plan_query_cl": (I, [I64, I64, I64, I64, ctypes.POINTER(GnPlanInfoCL)]),
        "gn_forward_partials": (I, [P, I, I64, I64, I64, I64, P, SZ, P]),
        "gn_forward_finish": (I, [P, I, P, P, I64, I64, I64, I64, F, I, P, I, P, P, P, SZ, P]),
        "gn_backward_partials": (I, [P, I, P, I, P, P, P, P, I, I64, I64, I64, I64, P, SZ, P]),
        "gn_backward_finish": (I, [P, I, P, I, P, P, P, P, I, I64, I64, I64, I64, P, P, P, P, SZ, P]),
        "gn_forward_shard_stats": (I, [P, I, I64, I64, I64, I64, P, P, SZ, P]),
        "gn_forward_shard_merge": (I, [P, I64, P, P, I64, I64, I64, I64, F, P, P, P, SZ, P]),
        "gn_backward_shard_sums": (I, [P, I, P, I, P, P, P, P, I, I64, I64, I64, I64, P, P, SZ, P]),
        "gn_backward_shard_merge": (I, [P, I64, P, P, P, P, I64, I64, I64, I64, I64, P, P, P, SZ, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(
            f"unet_groupnorm_amd: {path} is missing; build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    return _declare(ctypes.CDLL(path))


lib = load()
