"""Python face of the fp64 CPU GroupNorm oracle (``gn_oracle.c``).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import this module. It never touches the GPU
library and shares no code with it.

Arrays are numpy. Typed inputs are passed as ``(array, dtype_tag)`` where the tag
is ``"f32"`` (float32 array), ``"bf16"`` (uint16 array of bf16 bit patterns) or
``"f64"`` (float64 array). Torch CPU tensors are accepted and converted without
changing a bit.

The definition it implements and the passages it follows are stated in the
header of ``gn_oracle.c``.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgn_oracle.so")

_TAGS = {"f32": (0, np.float32), "bf16": (1, np.uint16), "f64": (2, np.float64), "f16": (3, np.float16)}

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from oracle import build as _b  # building the checker is not using it
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    lib.gno_group_stats.argtypes = [P, ctypes.c_int, I64, I64, I64, I64, F, P, P, P]
    CI = ctypes.c_int
    lib.gno_forward.argtypes = [P, CI, P, P, I64, I64, I64, I64, F, CI, P, P, P, P]
    lib.gno_forward_at.argtypes = [P, CI, P, P, I64, I64, I64, I64, CI, P, P, P, I64, P]
    lib.gno_backward.argtypes = [P, CI, P, CI, P, P, CI, I64, I64, I64, I64, F,
                                 P, P, P, P, P, P, P]
    lib.gno_backward_at.argtypes = [P, CI, P, CI, P, P, CI, I64, I64, I64, I64,
                                    P, P, P, P, P, I64, P]
    lib.gno_channel_abs_sums.argtypes = [P, CI, P, CI, P, P, CI, I64, I64, I64, I64, P, P, P, P]
    lib.gno_channel_abs_sums.restype = ctypes.c_int
    lib.gno_relu_value.argtypes = [ctypes.c_double]
    lib.gno_relu_value.restype = ctypes.c_double
    lib.gno_gate_value.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.gno_gate_value.restype = ctypes.c_double
    lib.gno_round_bf16.argtypes = [ctypes.c_double]
    lib.gno_round_bf16.restype = ctypes.c_uint16
    lib.gno_round_bf16_array.argtypes = [P, I64, P]
    lib.gno_round_f32_array.argtypes = [P, I64, P]
    lib.gno_round_f16.argtypes = [ctypes.c_double]
    lib.gno_round_f16.restype = ctypes.c_uint16
    lib.gno_round_f16_array.argtypes = [P, I64, P]
    lib.gno_f16_decode_array.argtypes = [P, I64, P]
    for fn in ("gno_group_stats", "gno_forward", "gno_forward_at", "gno_backward", "gno_backward_at"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _typed(a, tag=None):
    """Returns (contiguous numpy array, tag code)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16), 1
            if a.dtype == torch.float32:
                return a.numpy(), 0
            if a.dtype == torch.float64:
                return a.numpy(), 2
            if a.dtype == torch.float16:
                return a.numpy(), 3
            raise TypeError(f"oracle: unsupported torch dtype {a.dtype}")
    except ImportError:
        pass
    a = np.ascontiguousarray(a)
    if tag is None:
        tag = {np.dtype(np.float32): "f32", np.dtype(np.uint16): "bf16",
               np.dtype(np.float64): "f64", np.dtype(np.float16): "f16"}[a.dtype]
    code, dt = _TAGS[tag]
    if a.dtype != dt:
        raise TypeError(f"oracle: tag {tag} needs {dt}, got {a.dtype}")
    return a, code


def _f32vec(v, C):
    if v is None:
        return None
    try:
        import torch
        if isinstance(v, torch.Tensor):
            v = v.detach().cpu().numpy()
    except ImportError:
        pass
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert v.shape == (C,), v.shape
    return v


def _ptr(a):
    return None if a is None else a.ctypes.data


def _shape(x):
    N, C = int(x.shape[0]), int(x.shape[1])
    S = int(np.prod(x.shape[2:])) if len(x.shape) > 2 else 1
    return N, C, S


def group_stats(x, G, eps=1e-5, tag=None):
    """(mean, var, rstd), each [N, G] fp64."""
    xa, code = _typed(x, tag)
    N, C, S = _shape(xa)
    mean = np.empty((N, G)); var = np.empty((N, G)); rstd = np.empty((N, G))
    rc = _load().gno_group_stats(_ptr(xa), code, N, C, S, G, eps, _ptr(mean), _ptr(var), _ptr(rstd))
    if rc:
        raise ValueError(f"oracle: bad shape {xa.shape} G={G}")
    return mean, var, rstd


def forward(x, G, gamma=None, beta=None, eps=1e-5, tag=None, relu=False):
    """Returns dict(y [x.shape] fp64, mean/var/rstd [N, G] fp64); y = relu(GN(x)) if relu."""
    xa, code = _typed(x, tag)
    N, C, S = _shape(xa)
    y = np.empty(xa.shape, dtype=np.float64)
    mean = np.empty((N, G)); var = np.empty((N, G)); rstd = np.empty((N, G))
    g = _f32vec(gamma, C); b = _f32vec(beta, C)
    rc = _load().gno_forward(_ptr(xa), code, _ptr(g), _ptr(b), N, C, S, G, eps, int(relu),
                             _ptr(y), _ptr(mean), _ptr(var), _ptr(rstd))
    if rc:
        raise ValueError(f"oracle: bad shape {xa.shape} G={G}")
    return {"y": y, "mean": mean, "var": var, "rstd": rstd}


def forward_at(x, G, idx, mean, rstd, gamma=None, beta=None, tag=None, relu=False):
    """y (fp64) at flat indices ``idx`` given the oracle's own statistics."""
    xa, code = _typed(x, tag)
    N, C, S = _shape(xa)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.shape, dtype=np.float64)
    mean = np.ascontiguousarray(mean, dtype=np.float64)
    rstd = np.ascontiguousarray(rstd, dtype=np.float64)
    g = _f32vec(gamma, C); b = _f32vec(beta, C)
    _load().gno_forward_at(_ptr(xa), code, _ptr(g), _ptr(b), N, C, S, G, int(relu),
                           _ptr(mean), _ptr(rstd), _ptr(idx), idx.size, _ptr(out))
    return out


def backward(dy, x, G, gamma=None, eps=1e-5, want_dx=True, dy_tag=None, x_tag=None, beta=None,
             relu=False):
    """Returns dict(dx [x.shape] fp64 or None, dgamma/dbeta [C], mean/rstd/c1/c2 [N, G]).
    With relu, dy is the gradient of relu(GN(x)) (beta is then needed for the gate)."""
    xa, xc = _typed(x, x_tag)
    ga, gc = _typed(dy, dy_tag)
    assert ga.shape == xa.shape
    N, C, S = _shape(xa)
    dx = np.empty(xa.shape, dtype=np.float64) if want_dx else None
    dgamma = np.empty(C); dbeta = np.empty(C)
    mean = np.empty((N, G)); rstd = np.empty((N, G)); c1 = np.empty((N, G)); c2 = np.empty((N, G))
    g = _f32vec(gamma, C); b = _f32vec(beta, C)
    rc = _load().gno_backward(_ptr(ga), gc, _ptr(xa), xc, _ptr(g), _ptr(b), int(relu), N, C, S, G, eps,
                              _ptr(dx), _ptr(dgamma), _ptr(dbeta),
                              _ptr(mean), _ptr(rstd), _ptr(c1), _ptr(c2))
    if rc:
        raise ValueError(f"oracle: bad shape {xa.shape} G={G}")
    return {"dx": dx, "dgamma": dgamma, "dbeta": dbeta,
            "mean": mean, "rstd": rstd, "c1": c1, "c2": c2}


def backward_at(dy, x, G, idx, mean, rstd, c1, c2, gamma=None, dy_tag=None, x_tag=None, beta=None,
                relu=False):
    """dx (fp64) at flat indices ``idx`` given the oracle's own statistics and coefficients."""
    xa, xc = _typed(x, x_tag)
    ga, gc = _typed(dy, dy_tag)
    N, C, S = _shape(xa)
    idx = np.ascontiguousarray(idx, dtype=np.int64)
    out = np.empty(idx.shape, dtype=np.float64)
    arrs = [np.ascontiguousarray(a, dtype=np.float64) for a in (mean, rstd, c1, c2)]
    g = _f32vec(gamma, C); b = _f32vec(beta, C)
    _load().gno_backward_at(_ptr(ga), gc, _ptr(xa), xc, _ptr(g), _ptr(b), int(relu), N, C, S, G,
                            *[_ptr(a) for a in arrs], _ptr(idx), idx.size, _ptr(out))
    return out


def channel_abs_sums(dy, x, G, mean, rstd, dy_tag=None, x_tag=None, gamma=None, beta=None, relu=False):
    """(sum |g|, sum |g * xhat|) per channel [C], xhat from the given fp64 statistics, g = dy
    or the relu-gated dy."""
    xa, xc = _typed(x, x_tag)
    ga, gc = _typed(dy, dy_tag)
    N, C, S = _shape(xa)
    a = np.empty(C); b = np.empty(C)
    mean = np.ascontiguousarray(mean, dtype=np.float64)
    rstd = np.ascontiguousarray(rstd, dtype=np.float64)
    gm = _f32vec(gamma, C); bt = _f32vec(beta, C)
    _load().gno_channel_abs_sums(_ptr(ga), gc, _ptr(xa), xc, _ptr(gm), _ptr(bt), int(relu), N, C, S, G,
                                 _ptr(mean), _ptr(rstd), _ptr(a), _ptr(b))
    return a, b


def round_bf16(v):
    """fp64 -> bf16 bit patterns (uint16), rounded once to nearest-even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().gno_round_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


def round_f16(v):
    """fp64 -> fp16 bit patterns (uint16), rounded once to nearest-even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().gno_round_f16_array(_ptr(v), v.size, _ptr(out))
    return out


def f16_bits_to_f64(bits):
    """Exact decode of fp16 bit patterns to fp64 (the oracle's own binary16 decoder)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().gno_f16_decode_array(_ptr(bits), bits.size, _ptr(out))
    return out


def round_f32(v):
    """fp64 -> fp32, rounded once to nearest-even."""
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.float32)
    _load().gno_round_f32_array(_ptr(v), v.size, _ptr(out))
    return out


def bf16_bits_to_f64(bits):
    """Exact decode of bf16 bit patterns to fp64 (the upper half of an fp32)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
