"""Host-side checks of the launch plan and of the kernels' index arithmetic (no GPU).

The plan comes from libgn.so (gn_plan_query). The job -> element and lane -> vector
arithmetic of gn_kernels.hip is restated here in numpy and checked for every shape:
each element of the volume belongs to exactly one job, every vector load or store a
kernel issues stays inside the volume, and every partial index stays inside the
workspace. These are the conditions under which the kernels cannot touch memory
outside their buffers.
"""
import itertools

import numpy as np
import pytest

import unet_groupnorm_amd as g
from unet_groupnorm_amd._lib import lib

VEC = 8


def _jobs(plan, S):
    K, chunk = plan["chunks_per_row"], plan["chunk"]
    for j in range(plan["jobs"]):
        row, k = divmod(j, K)
        lo = row * S + k * chunk
        hi = row * S + min((k + 1) * chunk, S)
        yield j, row, k, lo, hi


SHAPES = [
    (1, 8, 4096, 4), (1, 32, 128 ** 3, 8), (1, 32, 256 ** 3, 8), (4, 512, 512, 32),
    (1, 64, 64 ** 3, 8), (1, 128, 32 ** 3, 16), (1, 256, 16 ** 3, 32), (1, 512, 8 ** 3, 32),
    (2, 6, 105, 2), (3, 4, 1, 4), (1, 4, 7, 2), (2, 12, 4913, 3), (1, 2, 3 * 8192 + 5, 1),
    (5, 10, 333, 5), (1, 1, 2 ** 20 + 3, 1), (2, 3, 65537, 3),
]


@pytest.mark.parametrize("N,C,S,G", SHAPES)
def test_plan_is_consistent(N, C, S, G):
    p = g.gn_plan_query(N, C, S, G)
    assert p["rows"] == N * C
    assert p["jobs"] == p["rows"] * p["chunks_per_row"]
    assert p["partials_per_group"] == (C // G) * p["chunks_per_row"]
    assert p["block"] in (64, 128, 256, 512)
    assert (p["chunks_per_row"] - 1) * p["chunk"] < S <= p["chunks_per_row"] * p["chunk"]
    assert p["workspace_bytes"] >= 8 * p["jobs"] and p["workspace_bytes"] % 256 == 0
    assert g.gn_workspace_bytes(N, C, S, G) == p["workspace_bytes"]
    if p["chunks_per_row"] > 1:
        step = p["block"] * p["vectors_per_step"] * VEC
        assert p["chunk"] % step == 0
    # streaming decomposition
    assert p["apply_block"] in (64, 128, 256)
    assert p["apply_jobs"] == p["rows"] * p["apply_chunks_per_row"]
    assert (p["apply_chunks_per_row"] - 1) * p["apply_chunk"] < S <= p["apply_chunks_per_row"] * p["apply_chunk"]
    assert p["apply_chunk"] <= p["apply_block"] * p["apply_vectors"] * VEC
    # workspace: partials, then 256-byte aligned per-row coefficients (two float4 per row)
    coef_off = -(-8 * p["jobs"] // 256) * 256
    assert p["workspace_bytes"] >= coef_off + 32 * p["rows"]


@pytest.mark.parametrize("N,C,S,G", [s for s in SHAPES if s[0] * s[1] * s[2] <= 2 ** 22])
def test_jobs_cover_every_element_once_and_stay_in_bounds(N, C, S, G):
    p = g.gn_plan_query(N, C, S, G)
    total = N * C * S
    seen = np.zeros(total, dtype=np.int32)
    blk, U = p["block"], p["vectors_per_step"]
    stepv = blk * U
    for j, row, k, lo, hi in _jobs(p, S):
        assert 0 <= lo < hi <= total
        seen[lo:hi] += 1
        v0 = lo // VEC
        vf0, vf1 = (lo + VEC - 1) // VEC, hi // VEC
        nvec = (hi + VEC - 1) // VEC - v0
        touched = np.zeros(nvec, dtype=np.int32)
        # the kernels pipeline the full steps [fs, fe) with unconditional vector loads and
        # take every other step through the masked path
        nsteps = -(-nvec // stepv)
        fs = 1 if v0 < vf0 else 0
        fe = max((vf1 - v0) // stepv, fs)
        assert nsteps - fe <= 1 and fs <= 1
        for si, sv0 in enumerate(range(v0, v0 + nvec, stepv)):
            full = sv0 >= vf0 and sv0 + stepv <= vf1
            assert full == (fs <= si < fe)
            lanes = np.arange(blk)
            for u in range(U):
                vi = sv0 + u * blk + lanes
                if full:
                    # full path: every lane loads/stores a whole vector
                    assert vi.min() >= vf0 and vi.max() < vf1
                    assert (vi.max() + 1) * VEC <= total
                    touched[vi - v0] += 1
                else:
                    whole = (vi >= vf0) & (vi < vf1)
                    assert ((vi[whole] + 1) * VEC <= total).all()
                    elems = vi[~whole][:, None] * VEC + np.arange(VEC)[None, :]
                    ok = (elems >= lo) & (elems < hi)
                    assert (elems[ok] < total).all() and (elems[ok] >= 0).all()
                    inside = (vi - v0 >= 0) & (vi - v0 < nvec)
                    touched[(vi - v0)[inside]] += 1
        assert (touched == 1).all(), "each vector of a job is visited by exactly one lane-step"
        # the finalize reads partials (n*C + g*Cg)*K + [0, P) of the job's group
        n, c = divmod(row, C)
        grp = c // (C // G)
        pbase = (n * C + grp * (C // G)) * p["chunks_per_row"]
        assert 0 <= pbase and pbase + p["partials_per_group"] <= p["jobs"]
    assert (seen == 1).all()


@pytest.mark.parametrize("N,C,S,G", [s for s in SHAPES if s[0] * s[1] * s[2] <= 2 ** 22])
def test_streaming_jobs_cover_every_element_once_and_stay_in_bounds(N, C, S, G):
    p = g.gn_plan_query(N, C, S, G)
    total = N * C * S
    seen = np.zeros(total, dtype=np.int32)
    blk, U = p["apply_block"], p["apply_vectors"]
    stepv = blk * U
    K, chunk = p["apply_chunks_per_row"], p["apply_chunk"]
    for j in range(p["apply_jobs"]):
        row, k = divmod(j, K)
        lo, hi = row * S + k * chunk, row * S + min((k + 1) * chunk, S)
        assert 0 <= lo < hi <= total and row < p["rows"]
        v0, vf0, vf1 = lo // VEC, (lo + VEC - 1) // VEC, hi // VEC
        nvec = (hi + VEC - 1) // VEC - v0
        assert nvec <= 2 * stepv  # at most two steps per streaming job
        for sv0 in range(v0, v0 + nvec, stepv):
            for u in range(U):
                vi = sv0 + u * blk + np.arange(blk)
                whole = (vi >= vf0) & (vi < vf1)
                assert ((vi[whole] + 1) * VEC <= total).all()
                seen_v = vi[whole]
                for e in range(VEC):
                    np.add.at(seen, seen_v * VEC + e, 1)
                elems = vi[~whole][:, None] * VEC + np.arange(VEC)[None, :]
                ok = (elems >= lo) & (elems < hi)
                np.add.at(seen, elems[ok], 1)
    assert (seen == 1).all()


def _full_step_range(v0, vf0, vf1, nvec, stepv):
    nsteps = -(-nvec // stepv)
    fs = 1 if v0 < vf0 else 0
    fe = max((vf1 - v0) // stepv, fs)
    return fs, fe, nsteps


@pytest.mark.parametrize("V", [1, 2, 4])
@pytest.mark.parametrize("N,C,S,G", [s for s in SHAPES if s[0] * s[1] * s[2] <= 2 ** 22])
def test_folded_jobs_cover_every_element_once_and_stay_in_bounds(N, C, S, G, V):
    """apply_fin_kernel / bwd_apply_fin_kernel: 256 threads, V vectors per lane per step,
    full steps [fs, fe) from raw vector loads, at most one edge step on each side element by
    element; every group has exactly one publishing job (its first row's first job) and
    every channel one dgamma/dbeta job (sample 0, first job)."""
    p = g.gn_plan_query(N, C, S, G)
    total = N * C * S
    seen = np.zeros(total, dtype=np.int32)
    blk, stepv = 256, 256 * V
    K, chunk = p["fold_chunks_per_row"], p["fold_chunk"]
    assert p["fold_jobs"] == p["rows"] * K
    assert chunk <= max(p["chunk"], 1) and (chunk <= 8192 or chunk == p["chunk"])
    assert (K - 1) * chunk < S <= K * chunk
    Cg = C // G
    publishers = np.zeros(N * G, dtype=np.int32)
    param_jobs = np.zeros(C, dtype=np.int32)
    for j in range(p["fold_jobs"]):
        row, k = divmod(j, K)
        n, c = divmod(row, C)
        gg = c // Cg
        if k == 0 and c == gg * Cg:
            publishers[n * G + gg] += 1
        if k == 0 and n == 0:
            param_jobs[c] += 1
        pbase = (n * C + gg * Cg) * p["chunks_per_row"]
        assert 0 <= pbase and pbase + p["partials_per_group"] <= p["jobs"]
        lo, hi = row * S + k * chunk, row * S + min((k + 1) * chunk, S)
        assert 0 <= lo < hi <= total
        v0, vf0, vf1 = lo // VEC, (lo + VEC - 1) // VEC, hi // VEC
        nvec = (hi + VEC - 1) // VEC - v0
        fs, fe, nsteps = _full_step_range(v0, vf0, vf1, nvec, stepv)
        lanes = np.arange(blk)
        for s_ in range(fs, fe):  # raw loads: every vector must be whole and inside the job
            vi = (v0 + s_ * stepv + np.arange(V)[:, None] * blk + lanes[None, :]).reshape(-1)
            assert ((vi >= vf0) & (vi < vf1)).all()
            for e in range(VEC):
                np.add.at(seen, vi * VEC + e, 1)
        edge = ([0] if fs > 0 else []) + ([fe] if fe < nsteps else [])
        for s_ in edge:
            vi = (v0 + s_ * stepv + np.arange(V)[:, None] * blk + lanes[None, :]).reshape(-1)
            whole = (vi >= vf0) & (vi < vf1)
            for e in range(VEC):
                np.add.at(seen, vi[whole] * VEC + e, 1)
            elems = vi[~whole][:, None] * VEC + np.arange(VEC)[None, :]
            ok = (elems >= lo) & (elems < hi)
            np.add.at(seen, elems[ok], 1)
    assert (seen == 1).all()
    assert (publishers == 1).all() and (param_jobs == 1).all()


def test_invalid_shapes_are_rejected_before_any_launch():
    info = g.gn_plan_query  # noqa: F841
    assert lib.gn_workspace_bytes(0, 4, 8, 2) == 0
    assert lib.gn_workspace_bytes(1, 6, 8, 4) == 0        # C % G != 0
    assert lib.gn_workspace_bytes(1, 4, 1, 4) == 0        # a single value per group set
    assert lib.gn_workspace_bytes(2, 4, 1, 4) > 0         # M == 1 with N > 1 is legal
    assert lib.gn_workspace_bytes(1, 4, 1, 2) > 0
    assert lib.gn_workspace_bytes(1, 2 ** 20, 2 ** 30, 1) == 0  # too many elements


def test_plan_is_a_pure_function_of_shape():
    shapes = list(itertools.product([1, 2, 4], [8, 32, 512], [1, 343, 512, 4096, 128 ** 3], [1, 8]))
    first = {s: g.gn_plan_query(*s) for s in shapes if s[1] % s[3] == 0 and s[0] * (s[1] // s[3]) * s[2] > 1}
    for s in reversed(list(first)):
        assert g.gn_plan_query(*s) == first[s]


# ----------------------------------------------------------------------------- resident path

RES_MAX_VECS = 4096  # 1024 threads x 4 vectors: the register capacity of one workgroup

RES_SHAPES = [
    (1, 8, 4096, 4), (4, 512, 512, 32), (1, 256, 16 ** 3, 32), (1, 512, 8 ** 3, 32),
    (1, 16, 4096, 2), (1, 16, 4104, 2), (8, 8, 1024, 2), (9, 8, 1024, 2), (3, 10, 24, 2),
    (2, 64, 8, 1), (2, 16, 8, 16), (2, 8, 216, 4), (1, 32, 128 ** 3, 8), (2, 6, 105, 2),
    (4096, 2, 8, 2), (4097, 2, 8, 2), (1, 4096, 8, 1), (2, 4, 1, 4), (70000, 1, 8, 1),
]


def test_fastdiv_is_exact_where_used():
    """The resident kernels divide in-workgroup indices (< 4096) by S/8, M/8 or C/G
    (<= 4096) as (x * m) >> 32 with m = floor(2^32 / d) + 1; exact for every x < 2^16
    and d <= 4096, and for sampled divisors up to 2^16."""
    x = np.arange(1 << 16, dtype=np.uint64)
    divisors = list(range(1, 4097)) + list(np.random.default_rng(5).integers(4097, 65537, 200))
    for d in divisors:
        m = np.uint64((1 << 32) // int(d) + 1)
        assert np.array_equal((x * m) >> np.uint64(32), x // np.uint64(d)), d


def _res_expect(N, C, S, G):
    M = C // G * S
    ok = S % VEC == 0 and G <= 2 ** 30
    f = ok and M // VEC <= RES_MAX_VECS and N <= 65535   # forward grid (G, N)
    b = ok and N * (M // VEC) <= RES_MAX_VECS
    return f, b


def _check_res_shape(nv, block, vecs):
    assert vecs in (1, 2, 4) and block % 64 == 0 and 64 <= block <= 1024
    assert block * vecs >= nv, "every vector has a lane"
    if vecs > 1:
        assert nv > 1024 * (vecs // 2), "no more vectors per lane than needed"


@pytest.mark.parametrize("N,C,S,G", RES_SHAPES)
def test_resident_choice_and_shape(N, C, S, G):
    p = g.gn_plan_query(N, C, S, G)
    ef, eb = _res_expect(N, C, S, G)
    assert bool(p["resident_forward"]) == ef and bool(p["resident_backward"]) == eb
    M = C // G * S
    if ef:
        _check_res_shape(M // VEC, p["resident_block_forward"], p["resident_vectors_forward"])
    if eb:
        assert p["resident_backward_split"] == int(N > 1)
        nv = _split_max_vectors(N, C, S, G) if N > 1 else N * M // VEC
        _check_res_shape(nv, p["resident_block_backward"], p["resident_vectors_backward"])
    else:
        assert p["resident_backward_split"] == 0


def _split_ncol(N, Cg, n):
    """Channels i of a group with i mod N == n."""
    return (Cg - 1 - n) // N + 1 if Cg > n else 0


def _split_max_vectors(N, C, S, G):
    Cg, W = C // G, S // VEC
    return Cg * W + (N - 1) * _split_ncol(N, Cg, 0) * W


@pytest.mark.parametrize("N,C,S,G", [s for s in RES_SHAPES if s[0] * s[1] * s[2] <= 2 ** 22])
def test_resident_workgroups_cover_every_element_once_and_stay_in_bounds(N, C, S, G):
    """Restates the lane -> vector -> (sample, row, address) arithmetic of res_fwd_kernel
    and res_bwd_kernel and checks it against the volume and the LDS arrays."""
    p = g.gn_plan_query(N, C, S, G)
    Cg, M = C // G, C // G * S
    total = N * C * S
    if p["resident_forward"]:
        B, V = p["resident_block_forward"], p["resident_vectors_forward"]
        vg, W = M // VEC, S // VEC
        seen = np.zeros(total // VEC, dtype=np.int32)
        w = (np.arange(V)[:, None] * B + np.arange(B)[None, :]).reshape(-1)
        w = w[w < vg]
        for ng in range(N * G):
            n, gg = divmod(ng, G)
            vb = (n * C + gg * Cg) * W
            assert 0 <= (w // W).max() < Cg
            np.add.at(seen, vb + w, 1)
        assert (seen == 1).all()
    if p["resident_backward"] and p["resident_backward_split"]:
        _check_split_backward(N, C, S, G, p)
    elif p["resident_backward"]:
        B, V = p["resident_block_backward"], p["resident_vectors_backward"]
        vg, W = M // VEC, S // VEC
        nvt, nrows = N * vg, N * Cg
        assert nvt <= RES_MAX_VECS and nrows <= RES_MAX_VECS and N <= RES_MAX_VECS
        seen = np.zeros(total // VEC, dtype=np.int32)
        w = (np.arange(V)[:, None] * B + np.arange(B)[None, :]).reshape(-1)
        w = w[w < nvt]
        n, r = w // vg, w % vg
        # per-vector sums sit at s_v[w]; row rho = n*Cg + r//W covers s_v[rho*W, (rho+1)*W)
        assert ((n * Cg + r // W) * W + r % W == w).all()
        for gg in range(G):
            gv = (n * C + gg * Cg) * W + r
            np.add.at(seen, gv, 1)
        assert (seen == 1).all()


def _check_split_backward(N, C, S, G, p):
    """res_bwd_split_kernel restated: workgroup (g, n) holds its own rows (n, g*Cg + rho),
    vector rho*W + k, then column rows crow = idx(n')*ncol + j for each other sample n' (idx:
    its rank among the others) and channel i = n + j*N, vector (Cg + crow)*W + k. Own
    vectors cover the volume once; every (sample, channel) row of a group is summed for
    dgamma exactly once, by the workgroup whose n is the channel's index mod N, in sample
    order; every index stays inside the volume and the LDS arrays."""
    Cg, W = C // G, S // VEC
    B, V = p["resident_block_backward"], p["resident_vectors_backward"]
    total = N * C * S // VEC
    own = np.zeros(total, dtype=np.int32)
    for gg in range(G):
        dg_rows = {}
        for n in range(N):
            ncol = _split_ncol(N, Cg, n)
            nrows = Cg + (N - 1) * ncol
            nvt = nrows * W
            assert nvt <= B * V and nvt <= RES_MAX_VECS and nrows <= RES_MAX_VECS
            w = (np.arange(V)[:, None] * B + np.arange(B)[None, :]).reshape(-1)
            w = w[w < nvt]
            R, k = w // W, w % W
            nr = np.where(R < Cg, n, 0)
            c = np.where(R < Cg, gg * Cg + R, 0)
            col = R >= Cg
            if col.any():
                crow = R[col] - Cg
                ni, j = crow // ncol, crow % ncol
                nr[col] = np.where(ni < n, ni, ni + 1)
                c[col] = gg * Cg + n + j * N
                assert ((n + j * N) < Cg).all() and (nr[col] != n).all()
            gv = (nr * C + c) * W + k
            assert gv.min() >= 0 and gv.max() < total
            np.add.at(own, gv[~col], 1)
            # rows each dgamma sum reads, in sample order
            for jj in range(ncol):
                i = n + jj * N
                rows = [i if np_ == n else Cg + (np_ if np_ < n else np_ - 1) * ncol + jj for np_ in range(N)]
                assert max(rows) < nrows
                # the row index maps back to (np_, channel i)
                for np_, Rr in enumerate(rows):
                    if Rr < Cg:
                        assert np_ == n and Rr == i
                    else:
                        cr = Rr - Cg
                        ni2, j2 = cr // ncol, cr % ncol
                        assert (ni2 if ni2 < n else ni2 + 1) == np_ and n + j2 * N == i
                assert i not in dg_rows
                dg_rows[i] = n
        assert sorted(dg_rows) == list(range(Cg)) and all(dg_rows[i] == i % N for i in dg_rows)
    assert (own == 1).all()


# ----------------------------------------------------------------------------- channels-last

CL_SHAPES = [
    (1, 32, 4096, 8), (2, 32, 1000, 8), (1, 64, 64 ** 3, 8), (3, 8, 77, 8), (1, 8, 77, 1),
    (2, 16, 333, 2), (1, 512, 512, 32), (2, 2048, 40, 1), (1, 1024, 300, 64), (4, 128, 8, 16),
    (1, 256, 4097, 32), (5, 64, 1, 64),
]


@pytest.mark.parametrize("N,C,S,G", CL_SHAPES)
def test_channels_last_lanes_cover_every_vector_once(N, C, S, G):
    """Restates the job -> voxel and lane -> (voxel, channel vector) arithmetic of the
    channels-last kernels: every (voxel, channel vector) of the volume is read exactly once
    by the reduction jobs and once by the streaming jobs, inside the volume."""
    p = g.gn_plan_query_cl(N, C, S, G)
    Cv, B, vps, R = C // VEC, p["block"], p["voxels_per_round"], p["rounds_per_step"]
    assert B % Cv == 0 and vps == B // Cv
    t = np.arange(B)
    cv, vo = t % Cv, t // Cv
    assert (p["chunk"] % (R * vps) == 0) or p["jobs_per_sample"] == 1
    for chunk, K, rounds in ((p["chunk"], p["jobs_per_sample"], R), (p["apply_chunk"], p["apply_jobs_per_sample"], p["apply_rounds"])):
        assert (K - 1) * chunk < S <= K * chunk
        seen = np.zeros((N, S, Cv), dtype=np.int32)
        for n in range(N):
            for k in range(K):
                v0, v1 = k * chunk, min((k + 1) * chunk, S)
                step = rounds * vps
                for s0 in range(v0, v1, step):
                    for r in range(rounds):
                        vox = s0 + r * vps + vo
                        ok = vox < v1
                        if not ok.any():
                            continue
                        off = (n * S + vox[ok]) * C + cv[ok] * VEC
                        assert off.min() >= 0 and (off + VEC).max() <= N * S * C
                        np.add.at(seen, (n, vox[ok], cv[ok]), 1)
        assert (seen == 1).all()


@pytest.mark.parametrize("N,C,S,G", CL_SHAPES)
def test_channels_last_slots_and_holders(N, C, S, G):
    """The lane's slots name the right groups, and the workgroup merge of group g (holder
    lanes of each wave after the strided shuffle tree) takes exactly the lanes whose channel
    vector holds g, each once."""
    p = g.gn_plan_query_cl(N, C, S, G)
    Cg, Cv, B, NGL = C // G, C // VEC, p["block"], p["groups_per_vector"]
    W = VEC // NGL
    for cvi in range(Cv):
        g0 = cvi * VEC // Cg
        for i in range(VEC):
            assert (cvi * VEC + i) // Cg == g0 + i // W
    reps = min(Cv, 64)
    # lanes each holder represents after the strided tree (off = 32, 16, ..., Cv)
    def represented(w, l):
        if Cv >= 64:
            return [w * 64 + l]
        return [w * 64 + l + q * Cv for q in range(64 // Cv)]

    def holder(c, w):
        l = ((c - 64 * w) % Cv + Cv) % Cv
        return l if l < 64 else -1

    for grp in range(G):
        if Cg < VEC:
            lo, hi, slot = grp * Cg // VEC, grp * Cg // VEC + 1, (grp * Cg % VEC) // Cg
        else:
            lo, hi, slot = grp * Cg // VEC, (grp + 1) * Cg // VEC, 0
        got = []
        for w in range(B // 64):
            for c in range(lo, hi):
                l = holder(c, w)
                if l >= 0:
                    assert l < reps and (w * 64 + l) * NGL + slot < B * NGL
                    got += represented(w, l)
        want = [tt for tt in range(B) if lo <= tt % Cv < hi]
        assert sorted(got) == want
        # the slot of lane vector c that holds group grp
        assert (lo * VEC // Cg) + slot == grp
    # workspace areas: partials (jobs x C float2), per-channel float2, per-group float4
    assert p["workspace_bytes"] >= p["jobs"] * (C + G) * 8 + N * C * 8 + N * G * 16


CL_RES_SHAPES = [
    (1, 256, 16 ** 3, 32), (1, 512, 8 ** 3, 32), (4, 512, 8 ** 3, 32), (2, 64, 4 ** 3, 8),
    (1, 256, 64, 4), (3, 128, 10, 8), (1, 32, 2 ** 15, 4), (8, 64, 64, 1), (1, 2048, 64, 16),
    (1, 1024, 64, 8), (2, 16, 1000, 4), (1, 64, 4097, 8), (70, 64, 64, 8), (1, 8, 1000, 1),
]


def _cl_res_expect(N, C, S, G):
    Cg = C // G
    cvg = Cg // 8
    ok = Cg % 8 == 0 and 1 <= cvg <= 8 and (cvg & (cvg - 1)) == 0
    vg = S * cvg
    fwd = ok and vg <= 1024 and N <= 65535
    bwd = ok and vg % 64 == 0 and N * vg <= 1024 and N * Cg <= 512
    return fwd, bwd


@pytest.mark.parametrize("N,C,S,G", CL_RES_SHAPES)
def test_channels_last_resident_choice_and_indexing(N, C, S, G):
    """cl_res_fwd_kernel / cl_res_bwd_kernel restated: the resident choice, every vector of
    every group covered once and inside the volume, each lane's channel vector fixed,
    backward waves wholly inside one sample, and every LDS index inside its array."""
    p = g.gn_plan_query_cl(N, C, S, G)
    fwd, bwd = _cl_res_expect(N, C, S, G)
    assert (p["resident_forward"], p["resident_backward"]) == (int(fwd), int(bwd))
    Cg = C // G
    cvg = max(Cg // 8, 1)
    l = cvg.bit_length() - 1
    vg = S * cvg
    total = N * S * C
    if fwd:
        blk, V = p["resident_block_forward"], p["resident_vectors_forward"]
        assert blk % 64 == 0 and blk <= 1024 and blk % cvg == 0 and V in (1, 2, 4) and blk * V >= vg
        seen = np.zeros(total, dtype=np.int32)
        t = np.arange(blk)
        for n in range(N):
            for gg in range(G):
                for u in range(V):
                    w = u * blk + t
                    w = w[w < vg]
                    s, k = w >> l, w & (cvg - 1)
                    assert (k == (w % blk) % cvg).all()
                    off = (n * S + s) * C + gg * Cg + 8 * k
                    assert (off + 8 <= total).all()
                    for e in range(8):
                        np.add.at(seen, off + e, 1)
        assert (seen == 1).all()
    if bwd:
        blk, V = p["resident_block_backward"], p["resident_vectors_backward"]
        nvt = N * vg
        nw = blk // 64
        assert blk % 64 == 0 and blk <= 1024 and V in (1, 2, 4) and blk * V >= nvt
        assert nw <= 16 and cvg <= 8 and N * Cg <= 512 and N <= 64
        seen = np.zeros(total, dtype=np.int32)
        for gg in range(G):
            for u in range(V):
                for wave in range(nw):
                    wb = u * blk + wave * 64
                    if wb >= nvt:
                        continue
                    assert wb + 64 <= nvt and (wb + 63) // vg == wb // vg
                    nn = wb // vg
                    w = wb + np.arange(64) - nn * vg
                    s, k = w >> l, w & (cvg - 1)
                    assert (k == np.arange(wave * 64, wave * 64 + 64) % cvg).all()
                    off = (nn * S + s) * C + gg * Cg + 8 * k
                    assert (off + 8 <= total).all()
                    for e in range(8):
                        np.add.at(seen, off + e, 1)
        assert (seen == 1).all()
