#!/usr/bin/env python3
"""GroupNorm fwd+bwd throughput on one MI355X, as achieved HBM GB/s.

One step is the whole hot path on one batch: gn_forward (statistics + normalize) then
gn_backward (reduction + dx), on the 128^3, C=32, G=8 bf16 UNet site with inputs
resident in HBM. Throughput counts the two-pass method's bytes per element:
forward 2*b_x + b_y, backward 2*(b_x + b_dy) + b_dx (16 B/element in bf16).

Printed: one JSON line with the headline value, the dominant kernel's roofline
(timed live with HIP events on the stream the kernels run on), the fp64 CPU oracle
timed on this host as a baseline, and side figures (per-kernel times, compulsory-byte
rate, a run with the 256 MiB last-level cache flushed between steps, a run whose inputs
were rewritten just before each call as a producer kernel would leave them, a plain copy
kernel's rate, and the 256^3 site).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak
METRIC = "GroupNorm fwd+bwd achieved HBM GB/s (% of MI355X peak), bf16 128³/256³ C=32 G=8"
KERNEL_SOURCES = ["unet_groupnorm_amd/csrc/gn_kernels.hip", "unet_groupnorm_amd/csrc/gn_device.hpp",
                  "unet_groupnorm_amd/csrc/gn_plan.cpp", "unet_groupnorm_amd/csrc/gn_plan.hpp",
                  "unet_groupnorm_amd/csrc/gn_launch.hpp", "unet_groupnorm_amd/csrc/gn_api.cpp"]


# Workloads --trace-case runs: name -> (case, layout, activation); "census" runs the 18 sites.
TRACE_CASES = {
    "tiny": ("TINY", "ncdhw", None),
    "deep": ("DEEP", "ncdhw", None),
    "deep_f32out": ("DEEP_F32OUT", "ncdhw", None),
    "scale7_ndhwc": ("SCALE7", "ndhwc", None),
    "scale7_fp16": ("SCALE7_F16", "ncdhw", None),
    "scale7_relu": ("SCALE7", "ncdhw", "relu"),
    "census": (None, "ncdhw", None),
    "shard8": (None, "ncdhw", None),  # one rank's share of the 256^3 site split in 8
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="headline, roofline and baseline only")
    ap.add_argument("--workload", choices=["scale7", "scale8"], default="scale7",
                    help="the 128^3 (default) or 256^3 C=32 G=8 bf16 site")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed steps before the warmup steps (the first timed window "
                         "otherwise reads 2-4%% slow on a GPU that was idle a moment before)")
    ap.add_argument("--trace-case", choices=sorted(TRACE_CASES),
                    help="only run --steps steps (after --warmup) of this workload and print its "
                         "time per step: a short program for a profiler's kernel trace")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB bf16 device copy 5 times (a kernel of known traffic "
                         "for scaling profiler byte counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def bytes_per_elem(x_dtype, y_dtype, dy_dtype):
    import torch
    sz = {torch.bfloat16: 2, torch.float16: 2, torch.float32: 4}
    bx, by, bdy = sz[x_dtype], sz[y_dtype], sz[dy_dtype]
    phases = {"stats": bx, "apply": bx + by, "bwd_reduce": bx + bdy, "bwd_apply": bx + bdy + bx}
    return phases, sum(phases.values())


class Runner:
    """Holds one workload resident on the GPU with preallocated outputs."""

    def __init__(self, case, activation=None, layout="ncdhw"):
        import torch

        import unet_groupnorm_amd as gn
        import workloads
        self.torch, self.gn, self.case, self.act = torch, gn, case, activation
        inp = workloads.make(case, "cuda")
        self.inp = inp
        self.x, self.dy, self.G, self.eps = inp["x"], inp["dy"], inp["G"], inp["eps"]
        if layout == "ndhwc":
            self.x, self.dy = gn.as_layout(self.x, layout), gn.as_layout(self.dy, layout)
        self.gamma, self.beta = inp["gamma"], inp["beta"]
        self.y = torch.empty_like(self.x, dtype=inp["out_dtype"])
        N = case.N
        self.mean = torch.empty((N, self.G), dtype=torch.float32, device="cuda")
        self.rstd = torch.empty_like(self.mean)
        self.dx = torch.empty_like(self.x)
        self.dgamma = torch.empty(case.C, dtype=torch.float32, device="cuda")
        self.dbeta = torch.empty_like(self.dgamma)
        self.ws = gn.workspace_for(self.x, self.G)
        self.phase_bytes, self.bpe = bytes_per_elem(self.x.dtype, self.y.dtype, self.dy.dtype)
        self.step_bytes = self.bpe * case.numel

    def step(self):
        gn = self.gn
        gn.gn_forward(self.x, self.gamma, self.beta, self.G, self.eps, activation=self.act,
                      workspace=self.ws, out=self.y, mean=self.mean, rstd=self.rstd)
        gn.gn_backward(self.dy, self.x, self.mean, self.rstd, self.gamma, self.G, beta=self.beta,
                       activation=self.act, workspace=self.ws, dx=self.dx, dgamma=self.dgamma,
                       dbeta=self.dbeta)

    def phases(self):
        """The same step as its four kernels, one call each (gn_forward = partials + finish,
        gn_backward likewise): stats_kernel, apply_fin_kernel, bwd_reduce_kernel and
        bwd_apply_fin_kernel, the kernels step() launches."""
        gn = self.gn
        return [
            ("stats", lambda: gn.gn_forward_partials(self.x, self.G, self.ws)),
            ("apply", lambda: gn.gn_forward_finish(self.x, self.gamma, self.beta, self.G, self.eps,
                                                   self.y, self.mean, self.rstd, self.ws, self.act)),
            ("bwd_reduce", lambda: gn.gn_backward_partials(self.dy, self.x, self.mean, self.rstd,
                                                           self.gamma, self.G, self.ws, beta=self.beta,
                                                           activation=self.act)),
            ("bwd_apply", lambda: gn.gn_backward_finish(self.dy, self.x, self.mean, self.rstd,
                                                        self.gamma, self.G, self.dx, self.dgamma,
                                                        self.dbeta, self.ws, beta=self.beta,
                                                        activation=self.act)),
        ]

    def settle(self, seconds):
        """Untimed steps for `seconds` of wall time; returns how many ran."""
        torch = self.torch
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(20):
                self.step()
            torch.cuda.synchronize()
            n += 20
        return n

    def timed_steps(self, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    def timed_phases(self, reps):
        """Average duration of each kernel, from HIP events on the stream the kernels run on
        (torch's current stream, which the binding passes down): after one full step, each
        kernel is launched `reps` times back to back between two events. Every kernel reads
        only what the earlier ones left, so the repeats redo identical work."""
        torch = self.torch
        ph = self.phases()
        for _, f in ph:
            f()
        torch.cuda.synchronize()
        out = {}
        for name, f in ph:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            out[name] = e0.elapsed_time(e1) / reps
        return out  # ms

    def graph_steps(self, per_graph=10, replays=20):
        """Steps replayed from a captured HIP graph of `per_graph` steps: microseconds per
        step without the host's per-call launch cost."""
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                self.step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (replays * per_graph)

    def flushed_steps(self, steps, flush_bytes=512 << 20):
        """Each step timed alone after overwriting a buffer twice the size of the 256 MiB
        last-level cache, so that no input starts the step in that cache."""
        torch = self.torch
        buf = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda")
        total = 0.0
        for _ in range(steps):
            buf.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            self.step()
            e1.record()
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
        return total / steps

    def produced_steps(self, steps):
        """Steps whose inputs were just written, as in a training step where a convolution
        writes x right before the forward and dy right before the backward: x and dy are
        rewritten from twins (a read and a write of each) before each call, and only the two
        GroupNorm calls are timed (HIP events around each, all steps enqueued back to back)."""
        torch = self.torch
        gn = self.gn
        xs, dys = self.x.clone(), self.dy.clone()
        ev = []
        for _ in range(steps + 1):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            self.x.copy_(xs)
            e[0].record()
            gn.gn_forward(self.x, self.gamma, self.beta, self.G, self.eps, activation=self.act,
                          workspace=self.ws, out=self.y, mean=self.mean, rstd=self.rstd)
            e[1].record()
            self.dy.copy_(dys)
            e[2].record()
            gn.gn_backward(self.dy, self.x, self.mean, self.rstd, self.gamma, self.G, beta=self.beta,
                           activation=self.act, workspace=self.ws, dx=self.dx, dgamma=self.dgamma,
                           dbeta=self.dbeta)
            e[3].record()
            ev.append(e)
        torch.cuda.synchronize()
        # the first step is dropped: the host enqueues it while the GPU is idle
        total = sum(e[0].elapsed_time(e[1]) + e[2].elapsed_time(e[3]) for e in ev[1:])
        return total / steps


def census(steps=10, warmup=3):
    """The 18 GroupNorm sites of a scale-7 UNet, fwd+bwd each, back to back: aggregate rate
    on method bytes, called eagerly and replayed from one captured HIP graph of the pass, and
    whether 10 repeats of every site are bitwise identical."""
    import torch

    import workloads
    runs = [Runner(c) for c in workloads.census_cases()]
    for r in runs:
        for _ in range(warmup):
            r.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        for r in runs:
            r.step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    total = sum(r.step_bytes for r in runs)
    # the same pass captured once in a HIP graph and replayed: no per-call host cost
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for r in runs:
            r.step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in runs:
            r.step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    pass_gms = e0.elapsed_time(e1) / steps
    del graph
    # determinism: 10 repeats per site, every output compared bitwise with the first
    identical = True
    for r in runs:
        r.step()
        ref = [t.clone() for t in (r.y, r.mean, r.rstd, r.dx, r.dgamma, r.dbeta)]
        for _ in range(9):
            r.step()
            for a, b in zip(ref, (r.y, r.mean, r.rstd, r.dx, r.dgamma, r.dbeta)):
                identical &= bool(torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                                              b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32)))
    # one site of each distinct shape on its own: fwd+bwd microseconds and method-byte rate
    per_shape = {}
    for r in runs:
        key = f"c{r.case.C}_g{r.case.G}_{r.case.spatial[0]}cube"
        if key in per_shape:
            continue
        r.settle(0.25)
        sms, _ = r.timed_steps(max(steps, 20), warmup)
        gms = r.graph_steps()
        per_shape[key] = {"us_per_step": round(sms * 1e3, 2),
                          "value": round(r.step_bytes / (sms * 1e-3) / 1e9, 1),
                          "graph_us_per_step": round(gms * 1e3, 2)}
    return {"sites": len(runs), "elements": sum(r.case.numel for r in runs), "ms_per_pass": round(ms, 4),
            "value": round(total / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
            "graph_ms_per_pass": round(pass_gms, 4),
            "graph_value": round(total / (pass_gms * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * total / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
            "bitwise_identical_10_repeats": identical, "per_shape": per_shape}


def spatial_shard(steps=30, warmup=5, nshards=8):
    """One rank's share of the 256^3, C=32, G=8 bf16 volume split in 8 along D
    (1 x 32 x 32 x 256 x 256), run through the spatial-shard entry points as that rank would:
    its statistics record, the shard-order merge of all ranks' records, the normalize; its
    per-row backward sums, their merge, dx. The records of the other ranks (what an
    all-gather of 128 B and 256 B would bring) are this shard's own, gathered once before
    timing; the all-gather itself is not run (one GPU)."""
    import torch

    import unet_groupnorm_amd as gn
    import workloads
    case = workloads.custom(1, 32, 8, (256 // nshards, 256, 256), torch.bfloat16, dist="unet", seed=1208)
    inp = workloads.make(case, "cuda")
    x, dy, G, eps, gamma, beta = inp["x"], inp["dy"], inp["G"], inp["eps"], inp["gamma"], inp["beta"]
    ws = gn.workspace_for(x, G)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    rec0 = gn.gn_forward_shard_stats(x, G, workspace=ws)
    recs = torch.stack([rec0] * nshards).contiguous()
    mean, rstd = gn.gn_forward_shard_merge(recs, gamma, beta, x.shape, G, eps, workspace=ws)
    sums0 = gn.gn_backward_shard_sums(dy, x, mean, rstd, gamma, G, beta=beta, workspace=ws)
    sums = torch.stack([sums0] * nshards).contiguous()
    S_total = case.S * nshards
    dg = torch.empty(case.C, dtype=torch.float32, device="cuda")
    db = torch.empty_like(dg)

    def step():
        gn.gn_forward_shard_stats(x, G, moments=recs[0], workspace=ws)
        gn.gn_forward_shard_merge(recs, gamma, beta, x.shape, G, eps, workspace=ws, mean=mean, rstd=rstd)
        gn.gn_forward_apply(x, G, y, ws)
        gn.gn_backward_shard_sums(dy, x, mean, rstd, gamma, G, beta=beta, sums=sums[0], workspace=ws)
        gn.gn_backward_shard_merge(sums, mean, rstd, gamma, x.shape, S_total, G, workspace=ws, beta=beta,
                                   dgamma=dg, dbeta=db)
        gn.gn_backward_apply(dy, x, G, dx, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 16 * case.numel
    return {"workload": f"scale8_256cube_c32_g8 split in {nshards} along D, one rank's share "
                        f"{tuple(case.shape)}, global statistics (records merged in shard order)",
            "us_per_step": round(ms * 1e3, 2), "method_bytes_per_step": nbytes,
            "value": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "note": "the all-gather of the records (N*G*16 B) and sums (N*C*8 B) is not run: one GPU"}


def small_configs(steps=50, warmup=10):
    """The launch-bound configurations, timed as fwd+bwd microseconds per step: eager (one
    call per direction from Python) and replayed from a captured graph."""
    import workloads
    out = {}
    for case in (workloads.TINY, workloads.DEEP, workloads.DEEP_F32OUT):
        r = Runner(case)
        r.settle(0.25)
        sms, _ = r.timed_steps(steps, warmup)
        gms = r.graph_steps()
        out[case.name] = {"us_per_step": round(sms * 1e3, 2),
                          "value": round(r.step_bytes / (sms * 1e-3) / 1e9, 1),
                          "bytes_per_step": r.step_bytes,
                          "graph_us_per_step": round(gms * 1e3, 2),
                          "graph_value": round(r.step_bytes / (gms * 1e-3) / 1e9, 1)}
        del r
    return out


def copy_ceiling_gbps(nbytes=1 << 30, reps=20):
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9


def cpu_baseline(runner, min_seconds=10.0, max_reps=40):
    """The fp64 oracle, as it stands, on this host: forward + backward on the same volume."""
    import numpy as np  # noqa: F401

    from oracle import oracle as O
    x, dy = runner.x.cpu(), runner.dy.cpu()
    gamma, beta = runner.gamma.cpu(), runner.beta.cpu()
    G, eps = runner.G, runner.eps
    reps, t_total = 0, 0.0
    while reps < max_reps and (reps == 0 or t_total < min_seconds):
        t0 = time.perf_counter()
        O.forward(x, G, gamma, beta, eps=eps)
        O.backward(dy, x, G, gamma, eps=eps)
        t_total += time.perf_counter() - t0
        reps += 1
    per = t_total / reps
    return {
        "value": round(runner.step_bytes / per / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"the whole {runner.case.name} volume ({runner.case.numel} elements): fp64 "
                   f"forward + backward (outputs in fp64), {reps} repetition(s), "
                   f"{per:.2f} s each, one thread"),
        "seconds_per_step": round(per, 3),
        "host_cpu": _cpu_model(),
        "host_cores_available": os.cpu_count(),
        "threads": _oracle_threads(runner),
    }


def _oracle_threads(runner, min_seconds=5.0, max_reps=60):
    """The same oracle spread over the host's cores: each (n, g) group, taken as its channel
    slice, is a GroupNorm with one group, so one oracle call per group (forward, then
    backward) runs in a thread pool (the oracle's C calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor

    from oracle import oracle as O
    x, dy = runner.x.cpu(), runner.dy.cpu()
    gamma, beta = runner.gamma.cpu(), runner.beta.cpu()
    G, eps, N, C = runner.G, runner.eps, runner.case.N, runner.case.C
    Cg = C // G
    units = [(n, g) for n in range(N) for g in range(G)]
    slices = [(x[n:n + 1, g * Cg:(g + 1) * Cg].contiguous(), dy[n:n + 1, g * Cg:(g + 1) * Cg].contiguous(),
               gamma[g * Cg:(g + 1) * Cg], beta[g * Cg:(g + 1) * Cg]) for n, g in units]
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    workers = max(1, min(cores, 16, len(units)))

    def one(u):
        xs, ds, gs, bs = u
        O.forward(xs, 1, gs, bs, eps=eps)
        O.backward(ds, xs, 1, gs, eps=eps)

    reps, t_total = 0, 0.0
    with ThreadPoolExecutor(max_workers=workers) as pool:
        while reps < max_reps and (reps == 0 or t_total < min_seconds):
            t0 = time.perf_counter()
            list(pool.map(one, slices))
            t_total += time.perf_counter() - t0
            reps += 1
    per = t_total / reps
    return {"value": round(runner.step_bytes / per / 1e9, 3), "unit": "GB/s", "cores": workers,
            "sample": (f"the same volume as {len(units)} one-group oracle calls (one per (n, g) "
                       f"group), forward + backward, on {workers} threads, {reps} repetition(s), "
                       f"{per:.3f} s each"),
            "seconds_per_step": round(per, 3)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def load_traffic(workload):
    """HBM bytes per launch of the dominant kernel from committed rocprofv3 counter runs,
    used only while the kernel sources still hash to the value recorded with them."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None, "no counter run committed"
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return rec, "ok"


def trace_case(args):
    """--trace-case: W warmup steps, then K timed steps of one workload (all 18 sites back to
    back for "census"); prints one JSON line with the time per step."""
    import torch

    import workloads
    if args.trace_case == "shard8":
        r = spatial_shard(steps=args.steps, warmup=args.warmup)
        if args.copy_probe:
            log("copy probe: 5 copies of 1 GiB")
            copy_ceiling_gbps(reps=5)
        print(json.dumps({"trace_case": args.trace_case, **r}), flush=True)
        return
    name, layout, act = TRACE_CASES[args.trace_case]
    cases = workloads.census_cases() if name is None else [getattr(workloads, name)]
    runs = [Runner(c, activation=act, layout=layout) for c in cases]
    log(f"trace case {args.trace_case}: {len(runs)} workload(s), {args.warmup} warmup and {args.steps} timed steps")
    for _ in range(args.warmup):
        for r in runs:
            r.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        for r in runs:
            r.step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    total = sum(r.step_bytes for r in runs)
    if args.copy_probe:
        log("copy probe: 5 copies of 1 GiB")
        copy_ceiling_gbps(reps=5)
    print(json.dumps({"trace_case": args.trace_case, "workloads": [c.name for c in cases], "layout": layout,
                      "activation": act, "steps": args.steps, "us_per_step": round(ms * 1e3, 2),
                      "method_bytes_per_step": total,
                      "gbps": round(total / (ms * 1e-3) / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the path would shard over samples or space, which is not built here)", file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.trace_case:
        trace_case(args)
        return
    case = workloads.SCALE7 if args.workload == "scale7" else workloads.SCALE8
    log(f"workload {case.name} {case.shape}; generating inputs on the GPU")
    run = Runner(case)
    settled = run.settle(args.settle) if args.settle > 0 else 0
    log(f"timing {args.steps} steps after {settled} settling and {args.warmup} warmup steps")
    ms, wall = run.timed_steps(args.steps, args.warmup)
    value = run.step_bytes / (ms * 1e-3) / 1e9

    log("timing each kernel with HIP events")
    ph_ms = run.timed_phases(max(args.steps, 20))
    dom = "bwd_apply"
    dom_bytes = run.phase_bytes[dom] * case.numel
    dom_gbps = dom_bytes / (ph_ms[dom] * 1e-3) / 1e9
    traffic, traffic_note = load_traffic(case.name)
    roofline = {
        "bound": "hbm",
        "kernel": "bwd_apply_fin_kernel<bf16,bf16> (dx pass with the backward finalize folded in: "
                  "reads x and dy, writes dx)",
        "achieved": round(dom_gbps, 1),
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": round(dom_gbps / PEAK_HBM_GBPS, 4),
        "traffic": (traffic or {}).get("bytes_per_launch"),
        "traffic_note": traffic_note if traffic is None else traffic.get("note", "ok"),
        "algorithmic_bytes_per_launch": dom_bytes,
        "avg_launch_us": round(ph_ms[dom] * 1e3, 2),
        "timing": "HIP events on the kernels' stream around back-to-back repeats of the kernel, "
                  "after one full step",
    }
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": case.name, "N": case.N, "C": case.C, "G": case.G, "spatial": list(case.spatial),
            "x_dtype": "bf16", "y_dtype": "bf16", "dy_dtype": "bf16", "dx_dtype": "bf16",
            "stats_dtype": "fp32", "bytes_per_step": run.step_bytes,
            "byte_model": "two-pass method bytes: fwd 2*bx+by, bwd 2*(bx+bdy)+bdx = 16 B/element",
        },
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "roofline": roofline,
        "kernels_us": {k: round(v * 1e3, 2) for k, v in ph_ms.items()},
        "kernel_source_hash": kernel_source_hash(),
        "settle": {"seconds": args.settle, "steps": settled},
    }
    if not args.no_extras:
        compulsory = 10 * case.numel
        out["compulsory_bytes_gbps"] = round(compulsory / (ms * 1e-3) / 1e9, 1)
        log("timing steps with the last-level cache flushed before each")
        fms = run.flushed_steps(max(10, args.steps // 5))
        out["llc_flushed"] = {"ms_per_step": round(fms, 5),
                              "value": round(run.step_bytes / (fms * 1e-3) / 1e9, 1)}
        log("timing steps whose inputs were just rewritten (x before the forward, dy before the backward)")
        pms = run.produced_steps(max(10, args.steps // 5))
        out["inputs_just_written"] = {"ms_per_step": round(pms, 5),
                                      "value": round(run.step_bytes / (pms * 1e-3) / 1e9, 1)}
        log("copy kernel ceiling")
        out["copy_kernel_gbps"] = round(copy_ceiling_gbps(), 1)
        log("the same step with the relu fused into the normalize store and the backward gate")
        run.act = "relu"
        rms, _ = run.timed_steps(max(10, args.steps // 2), 3)
        out["relu_fused"] = {"ms_per_step": round(rms, 5),
                             "value": round(run.step_bytes / (rms * 1e-3) / 1e9, 1)}
        run.act = None
        log("the same site in channels-last (NDHWC) memory")
        rcl = Runner(case, layout="ndhwc")
        cms, _ = rcl.timed_steps(max(10, args.steps // 2), 3)
        out["channels_last"] = {"ms_per_step": round(cms, 5),
                                "value": round(rcl.step_bytes / (cms * 1e-3) / 1e9, 1)}
        del rcl
        log("the same site with fp16 activations")
        r16 = Runner(workloads.SCALE7_F16)
        fms16, _ = r16.timed_steps(max(10, args.steps // 2), 3)
        out["fp16"] = {"workload": workloads.SCALE7_F16.name, "ms_per_step": round(fms16, 5),
                       "value": round(r16.step_bytes / (fms16 * 1e-3) / 1e9, 1)}
        del r16
    if not args.no_cpu_baseline:
        log("timing the fp64 CPU oracle on this host")
        out["cpu_baseline"] = cpu_baseline(run)
    if args.copy_probe:
        log("copy probe: 5 copies of 1 GiB")
        copy_ceiling_gbps(reps=5)
    if not args.no_extras and args.workload == "scale7":
        del run
        torch.cuda.empty_cache()
        c8 = workloads.SCALE8
        log(f"secondary workload {c8.name}")
        r8 = Runner(c8)
        r8.settle(0.5)
        ms8, _ = r8.timed_steps(max(5, args.steps // 5), 3)
        ph8 = r8.timed_phases(10)
        fms8 = r8.flushed_steps(5)
        out["scale8"] = {
            "workload": c8.name, "ms_per_step": round(ms8, 4),
            "value": round(r8.step_bytes / (ms8 * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * r8.step_bytes / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
            "kernels_us": {k: round(v * 1e3, 1) for k, v in ph8.items()},
            "llc_flushed": {"ms_per_step": round(fms8, 4),
                            "value": round(r8.step_bytes / (fms8 * 1e-3) / 1e9, 1)},
        }
        del r8
        torch.cuda.empty_cache()
        log("census: 18 GroupNorm sites of a scale-7 UNet")
        out["census"] = census()
        log("small configurations (tiny, deep)")
        out["small_configs"] = small_configs()
        log("one rank's share of the 256^3 site split in 8, global statistics")
        out["spatial_shard"] = spatial_shard()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
