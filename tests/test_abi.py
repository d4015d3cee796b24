"""The C ABI on a host without a GPU: every declared symbol is exported, and invalid
arguments are rejected with the documented status before anything touches the device."""
import ctypes
import os
import re

import pytest

import unet_groupnorm_amd as g
from unet_groupnorm_amd._lib import GN_BF16, GN_F32, STATUS_NAMES, lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gn_[a-z_]+)\s*\(", text, flags=re.M)))


def test_every_declared_function_is_exported():
    names = _declared_functions()
    assert len(names) == 23, names
    for name in names:
        assert hasattr(lib, name), name


def test_status_enum_matches_header():
    text = open(HEADER).read()
    for code, name in STATUS_NAMES.items():
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text), name
    assert re.search(r"GN_F32\s*=\s*0", text) and re.search(r"GN_BF16\s*=\s*1", text)
    assert re.search(r"GN_F16\s*=\s*2", text)
    assert re.search(r"GN_ACT_NONE\s*=\s*0", text) and re.search(r"GN_ACT_RELU\s*=\s*1", text)
    assert GN_F32 == 0 and GN_BF16 == 1
    for code in STATUS_NAMES:
        assert lib.gn_status_string(code)
    assert lib.gn_status_string(1234) == b"unknown status"
    assert lib.gn_abi_version() == int(re.search(r"#define GN_ABI_VERSION (\d+)", text).group(1)) == 11


# Fake but aligned, non-null addresses: validation never dereferences them, and every
# case below fails validation before the device is queried.
A = ctypes.c_void_p(0x10000)
B = ctypes.c_void_p(0x20000)


def fwd(fn="gn_forward", **kw):
    args = dict(x=A, xdt=GN_BF16, gamma=None, beta=None, N=1, C=8, S=64, G=4, eps=1e-5, act=0, y=B,
                ydt=GN_BF16, mean=A, rstd=B, ws=A, wsb=1 << 20, stream=None)
    args.update(kw)
    return getattr(lib, fn)(*args.values())


def bwd(fn="gn_backward", **kw):
    args = dict(dy=A, dydt=GN_BF16, x=B, xdt=GN_BF16, mean=A, rstd=B, gamma=None, beta=None, act=0,
                N=1, C=8, S=64, G=4, dx=A, dgamma=None, dbeta=None, ws=B, wsb=1 << 20, stream=None)
    args.update(kw)
    return getattr(lib, fn)(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(mean=None), 1), (dict(ws=None), 1),
    (dict(N=0), 2), (dict(S=0), 2), (dict(S=-1), 2), (dict(G=0), 2), (dict(C=0), 2),
    (dict(C=8, G=8, S=1), 2),
    (dict(C=6, G=4), 3),
    (dict(xdt=2), 4), (dict(xdt=GN_F32, ydt=GN_BF16), 4), (dict(ydt=7), 4),
    (dict(eps=-1e-5), 5), (dict(eps=float("nan")), 5), (dict(eps=float("inf")), 5),
    (dict(wsb=16), 6),
    (dict(x=ctypes.c_void_p(0x10002)), 7), (dict(y=ctypes.c_void_p(0x20008)), 7),
    (dict(ws=ctypes.c_void_p(0x10004)), 7), (dict(mean=ctypes.c_void_p(0x10001)), 7),
    (dict(act=2), 10), (dict(act=-1), 10),
])
@pytest.mark.parametrize("fn", ["gn_forward", "gn_forward_finish"])
def test_forward_validation(kw, status, fn):
    assert fwd(fn, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(dy=None), 1), (dict(x=None), 1), (dict(rstd=None), 1), (dict(ws=None), 1),
    (dict(C=6, G=4), 3), (dict(N=-2), 2), (dict(N=0), 2), (dict(S=0), 2), (dict(dydt=5), 4),
    (dict(xdt=3), 4),
    (dict(wsb=0), 6), (dict(dx=ctypes.c_void_p(0x10008)), 7),
    (dict(dgamma=ctypes.c_void_p(0x10002)), 7), (dict(beta=ctypes.c_void_p(0x10002)), 7),
    (dict(act=5), 10),
])
@pytest.mark.parametrize("fn", ["gn_backward", "gn_backward_finish"])
def test_backward_validation(kw, status, fn):
    assert bwd(fn, **kw) == status


def test_partials_validation():
    assert lib.gn_forward_partials(None, GN_BF16, 1, 8, 64, 4, A, 1 << 20, None) == 1
    assert lib.gn_forward_partials(A, GN_BF16, 1, 8, 64, 4, None, 1 << 20, None) == 1
    assert lib.gn_forward_partials(A, GN_BF16, 1, 8, 64, 3, A, 1 << 20, None) == 3
    assert lib.gn_forward_partials(A, GN_BF16, 0, 8, 64, 4, A, 1 << 20, None) == 2
    assert lib.gn_forward_partials(A, 9, 1, 8, 64, 4, A, 1 << 20, None) == 4
    assert lib.gn_forward_partials(A, GN_BF16, 1, 8, 64, 4, A, 8, None) == 6
    assert lib.gn_forward_partials(ctypes.c_void_p(0x10002), GN_BF16, 1, 8, 64, 4, A, 1 << 20, None) == 7
    args = [A, GN_BF16, B, GN_BF16, A, B, None, None, 0, 1, 8, 64, 4, A, 1 << 20, None]
    assert lib.gn_backward_partials(*args[:-3], None, 1 << 20, None) == 1
    assert lib.gn_backward_partials(None, *args[1:]) == 1
    assert lib.gn_backward_partials(*args[:8], 3, *args[9:]) == 10
    assert lib.gn_backward_partials(*args[:12], 3, *args[13:]) == 3
    assert lib.gn_backward_partials(*args[:-2], 16, None) == 6
    assert lib.gn_backward_partials(*args[:4], ctypes.c_void_p(0x10001), *args[5:]) == 7


def test_split_phase_validation():
    assert lib.gn_forward_stats(None, GN_BF16, None, None, 1, 8, 64, 4, 1e-5, A, B, A, 1 << 20, None) == 1
    assert lib.gn_forward_stats(A, GN_BF16, None, None, 1, 8, 64, 3, 1e-5, A, B, A, 1 << 20, None) == 3
    assert lib.gn_forward_stats(A, GN_BF16, None, None, 1, 8, 64, 4, 1e-5, A, B, A, 8, None) == 6
    assert lib.gn_forward_stats(A, GN_BF16, None, None, 1, 8, 64, 4, -1.0, A, B, A, 1 << 20, None) == 5
    assert lib.gn_forward_apply(A, GN_BF16, 1, 8, 64, 4, 0, None, GN_BF16, A, 1 << 20, None) == 1
    assert lib.gn_forward_apply(A, GN_F32, 1, 8, 64, 4, 0, B, GN_BF16, A, 1 << 20, None) == 4
    assert lib.gn_forward_apply(A, GN_BF16, 1, 8, 64, 4, 3, B, GN_BF16, A, 1 << 20, None) == 10
    assert lib.gn_backward_reduce(A, 9, B, GN_BF16, A, B, None, None, 0, 1, 8, 64, 4, None, None, A,
                                  1 << 20, None) == 4
    assert lib.gn_backward_reduce(A, GN_BF16, B, GN_BF16, A, B, None, None, 0, 1, 8, 64, 4, None, None,
                                  A, 8, None) == 6
    assert lib.gn_backward_reduce(A, GN_BF16, B, GN_BF16, A, B, None, None, 7, 1, 8, 64, 4, None, None,
                                  A, 1 << 20, None) == 10
    assert lib.gn_backward_apply(A, GN_BF16, B, GN_BF16, 1, 8, 64, 4, 0, None, A, 1 << 20, None) == 1
    assert lib.gn_backward_apply(A, GN_BF16, B, GN_BF16, 1, 8, 64, 4, 0, ctypes.c_void_p(0x30004), A,
                                 1 << 20, None) == 7
    assert lib.gn_backward_apply(A, GN_BF16, B, GN_BF16, 1, 8, 64, 4, 2, ctypes.c_void_p(0x30000), A,
                                 1 << 20, None) == 10


def _struct_fields(text, name):
    body = re.search(r"typedef struct %s \{(.*?)\} %s;" % (name, name), text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if not decl:
            continue
        ctype, names = decl.split(None, 1)
        for nm in names.split(","):
            fields.append((nm.strip(), ctype))
    return fields


@pytest.mark.parametrize("cname,pyname", [("gn_plan_info", "GnPlanInfo"), ("gn_plan_info_cl", "GnPlanInfoCL")])
def test_plan_info_struct_matches_header(cname, pyname):
    """The ctypes mirrors of the plan structs have the header's fields, in order, with the
    same widths (a drift here would make the query write past the Python structure)."""
    import pathlib

    from unet_groupnorm_amd import _lib as L
    text = (pathlib.Path(__file__).resolve().parents[1] / "include" / "gn.h").read_text()
    width = {"int64_t": 8, "int32_t": 4, "size_t": 8}
    ours = [(nm, ctypes.sizeof(t)) for nm, t in getattr(L, pyname)._fields_]
    assert ours == [(nm, width[t]) for nm, t in _struct_fields(text, cname)]



def cl_fwd(**kw):
    args = dict(x=A, xdt=GN_BF16, gamma=None, beta=None, N=1, C=32, S=64, G=8, eps=1e-5, act=0, y=B,
                ydt=GN_BF16, mean=A, rstd=B, ws=A, wsb=1 << 24, stream=None)
    args.update(kw)
    return lib.gn_forward_cl(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(C=12, G=4), 11),            # C not a multiple of 8
    (dict(C=24, G=8), 11),            # C/8 = 3 does not divide 256
    (dict(C=48, G=4), 11),            # C/G = 12: neither divides 8 nor a multiple of 8
    (dict(C=4096, G=8), 11),          # C/8 = 512 > 256
    (dict(C=32, G=5), 3),             # C % G
    (dict(N=0), 2),
    (dict(S=0), 2),
    (dict(x=None), 1),
    (dict(wsb=16), 6),
    (dict(xdt=7), 4),
    (dict(act=3), 10),
    (dict(y=ctypes.c_void_p(0x20004)), 7),
])
def test_channels_last_validation(kw, status):
    assert cl_fwd(**kw) == status


@pytest.mark.parametrize("C,G", [(8, 8), (16, 2), (32, 8), (64, 8), (128, 16), (512, 32), (2048, 1), (8, 1)])
def test_channels_last_supported_shapes_have_a_plan(C, G):
    p = g.gn_plan_query_cl(2, C, 1000, G)
    Cg = C // G
    assert p["groups_per_vector"] == max(1, 8 // Cg)
    assert p["voxels_per_round"] * (C // 8) == p["block"]
    assert lib.gn_workspace_bytes_cl(2, C, 1000, G) == p["workspace_bytes"] > 0
    assert lib.gn_backward_cl(A, GN_BF16, B, GN_BF16, A, B, None, None, 0, 2, C, 1000, G, None, None, None,
                              A, 16, None) == 6


def test_shard_entry_points_validate_before_launch():
    U = ctypes.c_void_p
    m = U(0x40000)
    # forward shard stats
    assert lib.gn_forward_shard_stats(None, GN_BF16, 1, 8, 64, 4, m, A, 1 << 20, None) == 1
    assert lib.gn_forward_shard_stats(A, GN_BF16, 1, 8, 64, 4, U(0x40008), A, 1 << 20, None) == 7
    assert lib.gn_forward_shard_stats(A, GN_BF16, 1, 8, 64, 4, m, A, 8, None) == 6
    assert lib.gn_forward_shard_stats(A, GN_BF16, 1, 2, 1 << 32, 1, m, A, 1 << 20, None) == 2   # count past 32 bits
    # forward merge
    assert lib.gn_forward_shard_merge(m, 0, None, None, 1, 8, 64, 4, 1e-5, A, B, A, 1 << 20, None) == 2
    assert lib.gn_forward_shard_merge(m, 2, None, None, 1, 8, 64, 3, 1e-5, A, B, A, 1 << 20, None) == 3
    assert lib.gn_forward_shard_merge(m, 2, None, None, 1, 8, 64, 4, -1.0, A, B, A, 1 << 20, None) == 5
    assert lib.gn_forward_shard_merge(None, 2, None, None, 1, 8, 64, 4, 1e-5, A, B, A, 1 << 20, None) == 1
    # backward sums
    assert lib.gn_backward_shard_sums(A, GN_BF16, B, GN_BF16, A, B, None, None, 0, 1, 8, 64, 4, None, A,
                                      1 << 20, None) == 1
    assert lib.gn_backward_shard_sums(A, GN_BF16, B, GN_BF16, A, B, None, None, 0, 1, 8, 64, 4, U(0x40004), A,
                                      1 << 20, None) == 7
    # backward merge
    s = U(0x50000)
    assert lib.gn_backward_shard_merge(s, 2, A, B, None, None, 1, 8, 64, 32, 4, None, None, A, 1 << 20, None) == 2
    assert lib.gn_backward_shard_merge(s, 0, A, B, None, None, 1, 8, 64, 64, 4, None, None, A, 1 << 20, None) == 2
    # a shard whose groups are single elements of larger groups is a valid shape (it gets as far as
    # the device check, which host memory fails)
    assert lib.gn_backward_shard_merge(s, 2, A, B, None, None, 2, 4, 1, 2, 4, None, None, A, 1 << 20, None) == 8
    assert lib.gn_backward_shard_merge(s, 2, A, B, None, None, 1, 8, 64, 128, 4, None, None, A, 8, None) == 6


def test_moments_record_layout():
    import pathlib
    text = (pathlib.Path(__file__).resolve().parents[1] / "include" / "gn.h").read_text()
    assert [(n, t) for n, t in _struct_fields(text, "gn_moments")] == [
        ("mean_hi", "float"), ("mean_lo", "float"), ("m2", "float"), ("count", "uint32_t")]


def fwd_noalloc(**kw):
    args = dict(x=A, xdt=GN_BF16, gamma=None, beta=None, N=1, C=8, S=64, G=4, eps=1e-5, act=0, y=B,
                ydt=GN_BF16, mean=A, rstd=B, stream=None)
    args.update(kw)
    return lib.gn_forward_noalloc(*args.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(rstd=None), 1),
    (dict(N=0), 2), (dict(S=0), 2), (dict(C=8, G=8, S=1), 2), (dict(C=6, G=4), 3),
    (dict(xdt=7), 4), (dict(xdt=GN_F32, ydt=GN_BF16), 4), (dict(eps=float("nan")), 5),
    (dict(x=ctypes.c_void_p(0x10002)), 7), (dict(act=5), 10),
    # a shape whose workspace exceeds the static scratch (65536 rows need 2 MiB of row records)
    (dict(N=64, C=1024, S=8, G=32), 12),
    # a valid shape that fits gets as far as the device check, which host addresses fail
    (dict(), 8), (dict(N=32, C=256, S=8, G=32), 8),
])
def test_noalloc_forward_validation(kw, status):
    assert fwd_noalloc(**kw) == status


def test_noalloc_scratch_size_in_header_and_binding():
    from unet_groupnorm_amd._lib import GN_NOALLOC_SCRATCH_BYTES
    text = open(HEADER).read()
    m = re.search(r"#define GN_NOALLOC_SCRATCH_BYTES \(1u << (\d+)\)", text)
    assert m and (1 << int(m.group(1))) == GN_NOALLOC_SCRATCH_BYTES
    # the largest case above that fits, and the one that does not
    assert lib.gn_workspace_bytes(32, 256, 8, 32) <= GN_NOALLOC_SCRATCH_BYTES < lib.gn_workspace_bytes(64, 1024, 8, 32)
