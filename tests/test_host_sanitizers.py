"""The host-side C units built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc and
g++, host code only, every report fatal): the fp64 oracle over small volumes of each input
type, special values and single-element groups included, and the launch plan of both layouts
over a sweep of valid and invalid shapes. Each runs as its own executable, so a report ends
it with a nonzero status and the report's text."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "gn_oracle.c")
CSRC = os.path.join(ROOT, "unet_groupnorm_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]

ORACLE_DRIVER = r"""
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int gno_group_stats(const void*, int, int64_t, int64_t, int64_t, int64_t, float, double*, double*, double*);
int gno_forward(const void*, int, const float*, const float*, int64_t, int64_t, int64_t, int64_t, float, int,
                double*, double*, double*, double*);
int gno_forward_at(const void*, int, const float*, const float*, int64_t, int64_t, int64_t, int64_t, int,
                   const double*, const double*, const int64_t*, int64_t, double*);
int gno_backward(const void*, int, const void*, int, const float*, const float*, int, int64_t, int64_t,
                 int64_t, int64_t, float, double*, double*, double*, double*, double*, double*, double*);
int gno_backward_at(const void*, int, const void*, int, const float*, const float*, int, int64_t, int64_t,
                    int64_t, int64_t, const double*, const double*, const double*, const double*,
                    const int64_t*, int64_t, double*);
int gno_channel_abs_sums(const void*, int, const void*, int, const float*, const float*, int, int64_t,
                         int64_t, int64_t, int64_t, const double*, const double*, double*, double*);
void gno_round_bf16_array(const double*, int64_t, uint16_t*);
void gno_round_f16_array(const double*, int64_t, uint16_t*);
void gno_round_f32_array(const double*, int64_t, float*);

static uint32_t state = 12345u;
static float rnd(void)  /* a value in [-4, 4) */
{
    state = state * 1664525u + 1013904223u;
    return (float)((state >> 8) & 0xffff) / 8192.0f - 4.0f;
}
static uint16_t to_bf16(float f) { uint32_t u; memcpy(&u, &f, 4); return (uint16_t)(u >> 16); }
static uint16_t to_f16(float f)  /* a normal binary16 near f (sign, exponent 14..16, 10 bits) */
{
    uint16_t s = f < 0.0f ? 0x8000u : 0u;
    uint16_t e = (uint16_t)(14 + ((state >> 3) % 3));
    return (uint16_t)(s | (e << 10) | ((state >> 11) & 0x3ffu));
}

/* dt: 0 fp32, 1 bf16, 2 fp64, 3 fp16 */
static void* make(int dt, int64_t n, int special)
{
    size_t sz = dt == 0 ? 4 : dt == 2 ? 8 : 2;
    char* p = (char*)malloc((size_t)n * sz);
    for (int64_t i = 0; i < n; ++i) {
        float v = rnd();
        if (dt == 0) ((float*)p)[i] = v;
        else if (dt == 2) ((double*)p)[i] = v;
        else if (dt == 1) ((uint16_t*)p)[i] = to_bf16(v);
        else ((uint16_t*)p)[i] = to_f16(v);
    }
    if (special && n > 3) {
        if (dt == 0) { ((float*)p)[1] = 1.0f / 0.0f; ((float*)p)[2] = 0.0f / 0.0f; }
        else if (dt == 1) { ((uint16_t*)p)[1] = 0x7f80u; ((uint16_t*)p)[2] = 0x7fc0u; }
        else if (dt == 3) { ((uint16_t*)p)[1] = 0x7c00u; ((uint16_t*)p)[2] = 0x7e00u; }
    }
    return p;
}

static int run(int64_t N, int64_t C, int64_t S, int64_t G, int xdt, int ddt, int act, int special)
{
    const int64_t n = N * C * S, ng = N * G;
    void* x = make(xdt, n, special);
    void* dy = make(ddt, n, 0);
    float* gamma = (float*)malloc(sizeof(float) * C);
    float* beta = (float*)malloc(sizeof(float) * C);
    for (int64_t c = 0; c < C; ++c) { gamma[c] = 1.0f + rnd() / 16.0f; beta[c] = rnd() / 16.0f; }
    double *y = malloc(sizeof(double) * n), *dx = malloc(sizeof(double) * n);
    double *m = malloc(sizeof(double) * ng), *v = malloc(sizeof(double) * ng), *r = malloc(sizeof(double) * ng);
    double *m2 = malloc(sizeof(double) * ng), *r2 = malloc(sizeof(double) * ng);
    double *c1 = malloc(sizeof(double) * ng), *c2 = malloc(sizeof(double) * ng);
    double *dg = malloc(sizeof(double) * C), *db = malloc(sizeof(double) * C);
    double *ad = malloc(sizeof(double) * C), *adx = malloc(sizeof(double) * C);
    int64_t* idx = malloc(sizeof(int64_t) * n);
    double *ya = malloc(sizeof(double) * n), *dxa = malloc(sizeof(double) * n);
    uint16_t* h = malloc(sizeof(uint16_t) * n);
    float* f = malloc(sizeof(float) * n);
    for (int64_t i = 0; i < n; ++i) idx[i] = (i * 7919) % n;
    int rc = 0;
    rc |= gno_group_stats(x, xdt, N, C, S, G, 1e-5f, m, v, r);
    rc |= gno_group_stats(x, xdt, N, C, S, G, 1e-5f, NULL, NULL, r);
    rc |= gno_forward(x, xdt, gamma, beta, N, C, S, G, 1e-5f, act, y, m, v, r);
    rc |= gno_forward(x, xdt, NULL, NULL, N, C, S, G, 0.0f, act, y, m, v, r);
    rc |= gno_forward_at(x, xdt, gamma, beta, N, C, S, G, act, m, r, idx, n, ya);
    rc |= gno_backward(dy, ddt, x, xdt, gamma, beta, act, N, C, S, G, 1e-5f, dx, dg, db, m2, r2, c1, c2);
    rc |= gno_backward(dy, ddt, x, xdt, NULL, beta, act, N, C, S, G, 1e-5f, NULL, dg, db, m2, r2, c1, c2);
    rc |= gno_backward(dy, ddt, x, xdt, gamma, beta, act, N, C, S, G, 1e-5f, dx, dg, db, m2, r2, c1, c2);
    rc |= gno_backward_at(dy, ddt, x, xdt, gamma, beta, act, N, C, S, G, m2, r2, c1, c2, idx, n, dxa);
    rc |= gno_channel_abs_sums(dy, ddt, x, xdt, gamma, beta, act, N, C, S, G, m2, r2, ad, adx);
    gno_round_bf16_array(y, n, h);
    gno_round_f16_array(dx, n, h);
    gno_round_f32_array(ya, n, f);
    free(x); free(dy); free(gamma); free(beta); free(y); free(dx); free(m); free(v); free(r); free(m2);
    free(r2); free(c1); free(c2); free(dg); free(db); free(ad); free(adx); free(idx); free(ya); free(dxa);
    free(h); free(f);
    return rc;
}

int main(void)
{
    static const int64_t shapes[][4] = {
        {1, 4, 7, 2}, {2, 6, 5, 3}, {2, 3, 1, 3}, {3, 8, 33, 4}, {1, 16, 64, 16}, {4, 2, 9, 1}};
    static const int dts[] = {0, 1, 2, 3};
    int bad = 0, runs = 0;
    for (int s = 0; s < 6; ++s)
        for (int a = 0; a < 4; ++a)
            for (int b = 0; b < 4; ++b)
                for (int act = 0; act < 2; ++act) {
                    bad |= run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], dts[a], dts[b], act,
                               (s + a + b) % 2);
                    ++runs;
                }
    /* refusals: a bad shape returns before touching anything */
    double m[4], v[4], r[4];
    float xf[4] = {0};
    bad |= gno_group_stats(xf, 0, 0, 4, 1, 2, 1e-5f, m, v, r) == 0;
    bad |= gno_group_stats(xf, 0, 1, 6, 1, 4, 1e-5f, m, v, r) == 0;
    printf("oracle runs %d bad %d\n", runs, bad);
    return bad;
}
"""

PLAN_DRIVER = r"""
#include <cstdint>
#include <cstdio>

#include "gn_plan.hpp"

int main()
{
    const int64_t Ns[] = {-1, 0, 1, 2, 3, 4, 64, 100000};
    const int64_t Cs[] = {0, 1, 3, 8, 24, 32, 64, 96, 512, 4096, 1 << 20};
    const int64_t Ss[] = {0, 1, 7, 8, 100, 4096, 32768, 2097152, (int64_t(1) << 28) + 64, int64_t(1) << 40};
    const int64_t Gs[] = {0, 1, 2, 3, 4, 8, 16, 32};
    int ok = 0, refused = 0, bad = 0;
    for (int64_t N : Ns)
        for (int64_t C : Cs)
            for (int64_t S : Ss)
                for (int64_t G : Gs) {
                    gn::Plan p;
                    const int rc = gn::make_plan(N, C, S, G, &p);
                    if (rc == 0) {
                        ++ok;
                        // the reduction jobs cover every row's elements once
                        if (p.K * p.chunk < S || (p.K - 1) * p.chunk >= S) ++bad;
                        if (p.jobs != N * C * p.K || p.ws_bytes == 0) ++bad;
                        if (p.block != 64 && p.block != 128 && p.block != 256) ++bad;
                    } else {
                        ++refused;
                    }
                    gn::PlanCL q;
                    const int rq = gn::make_plan_cl(N, C, S, G, &q);
                    if (rq == 0) {
                        if (q.K * q.chunk < S || (q.K - 1) * q.chunk >= S || q.jobs != N * q.K) ++bad;
                        if (q.ws_bytes == 0) ++bad;
                    }
                }
    std::printf("plans ok %d refused %d bad %d\n", ok, refused, bad);
    return bad != 0;
}
"""


def _build_and_run(tmp_path, compiler, sources, extra, name):
    exe = str(tmp_path / name)
    cmd = [compiler] + SAN + extra + sources + ["-o", exe] + (["-lm"] if compiler == "gcc" else [])
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    drv = tmp_path / "oracle_driver.c"
    drv.write_text(ORACLE_DRIVER)
    r = _build_and_run(tmp_path, "gcc", [ORACLE_C, str(drv)], ["-std=c11"], "oracle_san")
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "bad 0" in r.stdout and "runtime error" not in r.stderr, r.stderr[-4000:]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    drv = tmp_path / "plan_driver.cpp"
    drv.write_text(PLAN_DRIVER)
    r = _build_and_run(tmp_path, "g++", [os.path.join(CSRC, "gn_plan.cpp"), str(drv)],
                       ["-std=c++17", "-I", CSRC], "plan_san")
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "bad 0" in r.stdout and "runtime error" not in r.stderr, r.stderr[-4000:]
