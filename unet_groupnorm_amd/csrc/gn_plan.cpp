// gn_plan.cpp -- shape -> launch plan (see gn_plan.hpp).
#include "gn_plan.hpp"

namespace gn {

namespace {

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Lane vectors (1, 2 or 4) and threads (a multiple of 64, at most kResMaxBlock) of a
// resident workgroup covering nv vectors.
void resident_shape(int64_t nv, int* block, int* vecs)
{
    int v = 1;
    while (v < kResMaxLaneVecs && nv > int64_t(kResMaxBlock) * v) v *= 2;
    const int64_t b = round_up(ceil_div(nv, v), 64);
    *vecs = v;
    *block = int(b < 64 ? 64 : b);
}

}  // namespace

int make_plan(int64_t N, int64_t C, int64_t S, int64_t G, Plan* p)
{
    if (N <= 0 || C <= 0 || S <= 0 || G <= 0) return 2;
    if (C % G != 0) return 3;
    // N*C*S must not overflow and must stay below kMaxNumel.
    if (N > kMaxNumel / C || N * C > kMaxNumel / S) return 2;
    const int64_t Cg = C / G;
    // A single value per normalization set (N == 1 and M == 1) is rejected, as the stock
    // operator does; M == 1 with N > 1 is legal and answered exactly.
    if (N * Cg * S == 1) return 2;
    // Finalize launches take one workgroup per group (and per channel).
    if (N > ((int64_t(1) << 31) - 1 - C) / G) return 2;

    Plan q;
    q.N = N; q.C = C; q.S = S; q.G = G;
    q.Cg = Cg;
    q.M = Cg * S;
    q.rows = N * C;

    // Block size: the smallest of 64/128/256 threads whose step covers a whole row, so
    // that short rows (8^3 voxels) do not leave most lanes idle.
    const int64_t row_vecs = ceil_div(S, kVec) + 1;  // +1: a row need not start on a vector
    int block = 64;
    while (block < kRedBlock && int64_t(block) * kStepVecs < row_vecs) block *= 2;
    const int64_t step = int64_t(block) * kStepVecs * kVec;  // elements per workgroup step

    // Chunking: a whole row per job, halved while the launch has fewer than kTargetJobs
    // jobs and a chunk still holds at least one full step (then possibly one step back,
    // below). Chunks other than the last of a row are whole steps.
    int64_t K = 1, chunk = S;
    while (chunk > kMaxChunk) {
        K *= 2;
        chunk = round_up(ceil_div(S, K), step);
        K = ceil_div(S, chunk);
    }
    while (q.rows * K < kTargetJobs) {
        const int64_t c2 = round_up(ceil_div(S, K * 2), step);
        const int64_t k2 = ceil_div(S, c2);
        if (k2 <= K) break;
        K = k2;
        chunk = c2;
    }
    // Half as many jobs when that makes them kLongChunk elements or longer and leaves at
    // least kMinJobs of them.
    if (K >= 2 && chunk < kLongChunk) {
        const int64_t c2 = round_up(ceil_div(S, K / 2), step);
        const int64_t k2 = ceil_div(S, c2);
        if (c2 >= kLongChunk && q.rows * k2 >= kMinJobs) {
            K = k2;
            chunk = c2;
        }
    }
    q.K = K;
    q.chunk = chunk;
    q.jobs = q.rows * K;
    q.P = Cg * K;
    q.block = block;

    // Streaming jobs: kApplyVecs vectors per lane, the block sized (64..256) to the row.
    int block_a = 64;
    while (block_a < 256 && int64_t(block_a) * kApplyVecs < row_vecs) block_a *= 2;
    const int64_t step_a = int64_t(block_a) * kApplyVecs * kVec;
    q.block_a = block_a;
    q.chunk_a = S <= step_a ? S : step_a;
    q.K_a = ceil_div(S, q.chunk_a);
    q.jobs_a = q.rows * q.K_a;

    // Folded streaming jobs: the reduction jobs, split further where they exceed kFoldChunk.
    q.chunk_f = chunk <= kFoldChunk ? chunk : kFoldChunk;
    q.K_f = ceil_div(S, q.chunk_f);
    q.jobs_f = q.rows * q.K_f;

    // Resident path: rows of whole vectors (so every vector lies in one row and every row
    // starts on a vector) and a workgroup's share within kResMaxVecs.
    // The forward's grid is (G, N), so N stays within the y extent every device accepts.
    if (S % kVec == 0 && G <= (int64_t(1) << 30)) {
        const int64_t vg = q.M / kVec;
        if (vg <= kResMaxVecs && N <= 65535) {
            q.res_fwd = true;
            resident_shape(vg, &q.res_block_f, &q.res_vecs_f);
        }
        if (N <= kResMaxVecs / vg) {
            q.res_bwd = true;
            if (N > 1) {
                // the largest workgroup: its own vg vectors plus, for n = 0, ceil(Cg/N)
                // channels of each of the other N - 1 samples
                q.res_bwd_split = true;
                resident_shape(vg + (N - 1) * ceil_div(Cg, N) * (S / kVec), &q.res_block_b, &q.res_vecs_b);
            } else {
                resident_shape(N * vg, &q.res_block_b, &q.res_vecs_b);
            }
        }
    }

    q.ws_coef_offset = size_t(round_up(q.jobs * 8, 256));
    q.ws_bytes = q.ws_coef_offset + size_t(round_up(q.rows * 32, 256));
    *p = q;
    return 0;
}

int make_plan_cl(int64_t N, int64_t C, int64_t S, int64_t G, PlanCL* p)
{
    Plan base;
    const int rc = make_plan(N, C, S, G, &base);
    if (rc) return rc;
    const int64_t Cg = C / G;
    if (C % kVec != 0) return 4;
    const int64_t Cv = C / kVec;
    if (Cv > kClBlock || kClBlock % Cv != 0) return 4;
    if (!(Cg % kVec == 0 || kVec % Cg == 0)) return 4;

    PlanCL q;
    q.N = N; q.C = C; q.S = S; q.G = G;
    q.Cg = Cg;
    q.M = Cg * S;
    q.Cv = Cv;
    q.vps = kClBlock / Cv;
    q.ngl = int(Cg >= kVec ? 1 : kVec / Cg);
    // Reduction jobs: whole samples split until the launch has kTargetJobs jobs or a job is
    // one step. A job's count per group (chunk * C/G elements) stays within kMaxChunk, so
    // every in-job count fits 32 bits.
    const int64_t step = kClRounds * q.vps;
    const int64_t max_chunk = kMaxChunk / (Cg > kVec ? Cg : kVec);
    int64_t K = 1, chunk = round_up(S, step);
    while (chunk > max_chunk) {
        K *= 2;
        chunk = round_up(ceil_div(S, K), step);
        K = ceil_div(S, chunk);
    }
    while (N * K < kClTargetJobs) {
        const int64_t c2 = round_up(ceil_div(S, K * 2), step);
        const int64_t k2 = ceil_div(S, c2);
        if (k2 <= K) break;
        K = k2;
        chunk = c2;
    }
    q.K = K;
    q.chunk = chunk;
    q.jobs = N * K;
    q.chunk_a = kClApplyRounds * q.vps;
    q.K_a = ceil_div(S, q.chunk_a);
    q.jobs_a = N * q.K_a;
    // Resident path: every group is whole vectors (C/G a multiple of 8) and fits one
    // workgroup; the backward's workgroup also holds all samples, whose vectors start on
    // wave boundaries (S * C/(8G) a multiple of 64), within kClResMaxRows rows.
    const int64_t cvg = Cg / kVec;
    if (Cg % kVec == 0 && cvg <= kClResMaxGroupVecs && (cvg & (cvg - 1)) == 0) {
        const int64_t vg = S * cvg;
        int l = 0;
        while ((int64_t(1) << l) < cvg) ++l;
        q.lcvg = l;
        if (vg <= kClResMaxVecs && N <= 65535) {
            q.res_fwd = true;
            resident_shape(vg, &q.res_block_f, &q.res_vecs_f);
        }
        if (vg % 64 == 0 && N <= kClResMaxVecs / vg && N * Cg <= kClResMaxRows) {
            q.res_bwd = true;
            resident_shape(N * vg, &q.res_block_b, &q.res_vecs_b);
        }
    }
    q.ws_partg_offset = size_t(round_up(q.jobs * C * 8, 256));
    q.ws_coefc_offset = q.ws_partg_offset + size_t(round_up(q.jobs * G * 8, 256));
    q.ws_coefg_offset = q.ws_coefc_offset + size_t(round_up(N * C * 8, 256));
    q.ws_bytes = q.ws_coefg_offset + size_t(round_up(N * G * 16, 256));
    *p = q;
    return 0;
}

}  // namespace gn
