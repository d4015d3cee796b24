#!/usr/bin/env python3
"""GroupNorm fwd+bwd throughput on one MI355X, as achieved HBM GB/s.

One step is the whole hot path on one batch: gn_forward (statistics + normalize) then
gn_backward (reduction + dx), on the 128^3, C=32, G=8 bf16 UNet site with inputs
resident in HBM. Throughput counts the two-pass method's bytes per element:
forward 2*b_x + b_y, backward 2*(b_x + b_dy) + b_dx (16 B/element in bf16).

Printed: one JSON line with the headline value (K steps between two HIP events), the
same steps timed one by one (median, and the minimum over 7 trials of the median of 20),
the dominant kernel's roofline (its duration inside the step, from HIP events on the
stream the kernels run on), the device's streaming ceiling measured with the committed
probe kernels (libgn_probe.so: read, write, copy) and every kernel's time against the
bound that ceiling gives for its own reads and writes, the fp64 CPU oracle timed on this
host per direction on one core and on all of them, the achieved accuracy against the
oracle, and side figures (the step with the last-level cache flushed, with inputs just
written, the relu fused, channels-last, fp16, the 256^3 site with its own roofline, the
18-site census, the small configurations and one rank's share of a spatially sharded
256^3 volume).
"""
import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E peak
METRIC = "GroupNorm fwd+bwd achieved HBM GB/s (% of MI355X peak), bf16 128³/256³ C=32 G=8"
# Every source compiled into libgn.so: a change to any of them marks committed counter
# records stale.
KERNEL_SOURCES = ["include/gn.h", "unet_groupnorm_amd/csrc/gn_kernels.hip", "unet_groupnorm_amd/csrc/gn_kernels_cl.hip",
                  "unet_groupnorm_amd/csrc/gn_kernels_shard.hip", "unet_groupnorm_amd/csrc/gn_device.hpp",
                  "unet_groupnorm_amd/csrc/gn_plan.cpp", "unet_groupnorm_amd/csrc/gn_plan.hpp",
                  "unet_groupnorm_amd/csrc/gn_launch.hpp", "unet_groupnorm_amd/csrc/gn_api.cpp"]
PAGES_FP32_STATS_VS_FP64 = [1.1e-7, 1.9e-7]  # "Optimize GroupNorm", paragraph folding seven launches into four


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


def parse(argv=None):
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
                    help="also run the probe copy kernel over 1 GiB 5 times (a kernel of known traffic "
                         "for scaling profiler byte counters)")
    return ap.parse_args(argv)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def phase_rw(x_dtype, y_dtype, dy_dtype):
    """Algorithmic (read, write) bytes per element of each kernel of a step."""
    import torch
    sz = {torch.bfloat16: 2, torch.float16: 2, torch.float32: 4}
    bx, by, bdy = sz[x_dtype], sz[y_dtype], sz[dy_dtype]
    return {"stats": (bx, 0), "apply": (bx, by), "bwd_reduce": (bx + bdy, 0), "bwd_apply": (bx + bdy, bx)}


def bytes_per_elem(x_dtype, y_dtype, dy_dtype):
    rw = phase_rw(x_dtype, y_dtype, dy_dtype)
    phases = {k: r + w for k, (r, w) in rw.items()}
    return phases, sum(phases.values())


def _events(n):
    """n timing events, each recorded once already: torch creates a HIP event at its first
    record, and that creation, left inside a timed loop, could hold the host up long enough
    for the GPU to run dry between two events."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    return ev


# ----------------------------------------------------------------------------- probe kernels

_PROBE = None


def probe_lib():
    """libgn_probe.so: the streaming probes and the atomic negative control (not libgn.so)."""
    global _PROBE
    if _PROBE is None:
        path = os.path.join(ROOT, "unet_groupnorm_amd", "libgn_probe.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing; build first (python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        P, I, I64, SZ, U32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_uint32
        lib.gnp_read.argtypes = [P, SZ, I, I, U32, P, I64, P]
        lib.gnp_write.argtypes = [P, SZ, I, I, U32, I64, P]
        lib.gnp_copy.argtypes = [P, P, SZ, I, I, I, I64, P]
        lib.gnp_atomic_group_sums.argtypes = [P, I64, I64, I64, P, P]
        for f in (lib.gnp_read, lib.gnp_write, lib.gnp_copy, lib.gnp_atomic_group_sums):
            f.restype = I
        _PROBE = lib
    return _PROBE


def _stream_ptr():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def ceiling(nbytes=1 << 30, reps=10, grids=(1024, 2048, 4096, 8192, 16384, 32768), vecs=(2, 4, 8, 16)):
    """HBM rates of pure streams over `nbytes` buffers (far larger than the 256 MiB last-level
    cache), with plain and nontemporal loads and stores, each at the best of a sweep of grid
    sizes and vectors in flight per lane: the rates the device delivers for the traffic the
    GroupNorm kernels generate."""
    import torch
    lib = probe_lib()
    src = torch.full((nbytes // 4,), 7, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    st = _stream_ptr()
    magic = 0x5EED5EED
    variants = {
        "read_nontemporal": (lambda g, v: lib.gnp_read(src.data_ptr(), nbytes, 1, v, magic, sink.data_ptr(), g, st),
                             nbytes),
        "read_plain": (lambda g, v: lib.gnp_read(src.data_ptr(), nbytes, 0, v, magic, sink.data_ptr(), g, st), nbytes),
        "write_nontemporal": (lambda g, v: lib.gnp_write(dst.data_ptr(), nbytes, 1, v, 3, g, st), nbytes),
        "write_plain": (lambda g, v: lib.gnp_write(dst.data_ptr(), nbytes, 0, v, 3, g, st), nbytes),
        "copy_nontemporal": (lambda g, v: lib.gnp_copy(src.data_ptr(), dst.data_ptr(), nbytes, 1, 1, v, g, st),
                             2 * nbytes),
        "copy_plain": (lambda g, v: lib.gnp_copy(src.data_ptr(), dst.data_ptr(), nbytes, 0, 0, v, g, st), 2 * nbytes),
        "copy_nt_loads_plain_stores": (lambda g, v: lib.gnp_copy(src.data_ptr(), dst.data_ptr(), nbytes, 1, 0, v, g,
                                                                 st), 2 * nbytes),
    }
    out = {}
    for name, (fn, moved) in variants.items():
        best = None
        for v in vecs:
            for g in grids:
                for _ in range(2):
                    assert fn(g, v) == 0, name
                e0, e1 = _events(2)
                e0.record()
                for _ in range(reps):
                    fn(g, v)
                e1.record()
                torch.cuda.synchronize()
                gbps = moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
                if best is None or gbps > best[0]:
                    best = (gbps, g, v)
        out[name] = {"gbps": round(best[0], 1), "grid": best[1], "vecs": best[2]}
    assert int(sink.sum().item()) == 0  # the magic value was never read, so nothing was written
    read = max(out["read_nontemporal"]["gbps"], out["read_plain"]["gbps"])
    write = max(out["write_nontemporal"]["gbps"], out["write_plain"]["gbps"])
    copy = max(out[k]["gbps"] for k in out if k.startswith("copy"))
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "read_gbps": read, "write_gbps": write, "copy_gbps": copy,
            # a copy moves equal bytes each way: what pricing reads and writes separately predicts
            "copy_predicted_gbps": round(2 / (1 / read + 1 / write), 1),
            "variants": out, "kernels": "libgn_probe.so gnp_read / gnp_write / gnp_copy (16-byte vectors, "
                                        "256-thread workgroups; best of 2-16 vectors a lane in flight and "
                                        "1024-32768 workgroups)"}


def kernel_bounds(rw, numel, kernel_us, ceil):
    """Each kernel's time against the bound of the measured ceiling for its own traffic:
    read bytes at the read rate plus written bytes at the write rate."""
    out = {}
    for k, (r, w) in rw.items():
        bound_us = (r * numel / (ceil["read_gbps"] * 1e9) + w * numel / (ceil["write_gbps"] * 1e9)) * 1e6
        out[k] = {"us": round(kernel_us[k], 2), "bound_us": round(bound_us, 2),
                  "frac_of_bound": round(bound_us / kernel_us[k], 4)}
    tot_b = sum(v["bound_us"] for v in out.values())
    tot = sum(kernel_us[k] for k in rw)
    out["all"] = {"us": round(tot, 2), "bound_us": round(tot_b, 2), "frac_of_bound": round(tot_b / tot, 4)}
    return out


# ----------------------------------------------------------------------------- one workload

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
        self.rw = phase_rw(self.x.dtype, self.y.dtype, self.dy.dtype)
        self.phase_bytes, self.bpe = bytes_per_elem(self.x.dtype, self.y.dtype, self.dy.dtype)
        self.step_bytes = self.bpe * case.numel

    def fwd(self):
        self.gn.gn_forward(self.x, self.gamma, self.beta, self.G, self.eps, activation=self.act,
                           workspace=self.ws, out=self.y, mean=self.mean, rstd=self.rstd)

    def bwd(self):
        self.gn.gn_backward(self.dy, self.x, self.mean, self.rstd, self.gamma, self.G, beta=self.beta,
                            activation=self.act, workspace=self.ws, dx=self.dx, dgamma=self.dgamma,
                            dbeta=self.dbeta)

    def step(self):
        self.fwd()
        self.bwd()

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
        """Mean step time of `steps` back-to-back steps between two HIP events."""
        torch = self.torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        e0, e1 = _events(2)
        t0 = time.perf_counter()
        e0.record()
        for _ in range(steps):
            self.step()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return e0.elapsed_time(e1) / steps, wall

    def step_protocol(self, trials=7, per_trial=20):
        """Every step timed on its own (an event between consecutive steps, all enqueued back
        to back): the median over all steps, and the minimum over `trials` trials of the
        median of `per_trial` steps ("Optimize GroupNorm", paragraph folding seven launches
        into four: min of 7 medians-of-20)."""
        torch = self.torch
        medians, every = [], []
        for _ in range(trials):
            ev = _events(per_trial + 1)
            ev[0].record()
            for i in range(per_trial):
                self.step()
                ev[i + 1].record()
            torch.cuda.synchronize()
            t = [ev[i].elapsed_time(ev[i + 1]) for i in range(per_trial)]
            every += t
            medians.append(statistics.median(t))
        return {"trials": trials, "steps_per_trial": per_trial, "timed_steps": trials * per_trial,
                "median_ms": round(statistics.median(every), 5), "min_of_medians_ms": round(min(medians), 5),
                "max_of_medians_ms": round(max(medians), 5)}

    def in_step_kernels(self, steps=50, backlog=4):
        """Each kernel's average duration inside the step: events between the step's four
        kernels (launched through the two-call halves of gn_forward and gn_backward, the
        same kernels as step()), over `steps` steps enqueued back to back. Each figure
        includes one event packet's latency. The events exist before the first is recorded
        and `backlog` untimed steps are queued ahead of them, so the GPU is never left
        waiting on the host between two events (a wait would land in one kernel's figure)."""
        torch = self.torch
        ph = self.phases()
        n = len(ph)
        for _ in range(3):
            for _, f in ph:
                f()
        torch.cuda.synchronize()
        ev = _events(steps * n + 1)
        for _ in range(backlog):
            for _, f in ph:
                f()
        ev[0].record()
        k = 0
        for _ in range(steps):
            for _, f in ph:
                f()
                k += 1
                ev[k].record()
        torch.cuda.synchronize()
        return {name: sum(ev[s * n + i].elapsed_time(ev[s * n + i + 1]) for s in range(steps)) / steps
                for i, (name, _) in enumerate(ph)}

    def back_to_back_kernels(self, reps):
        """Each kernel launched `reps` times back to back between two events, after one full
        step (every kernel reads only what the earlier ones left, so repeats redo identical
        work; the last-level cache then holds what the repeats touch, not what a step does)."""
        torch = self.torch
        ph = self.phases()
        for _, f in ph:
            f()
        torch.cuda.synchronize()
        out = {}
        for name, f in ph:
            e0, e1 = _events(2)
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
        e0, e1 = _events(2)
        e0.record()
        for _ in range(replays):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (replays * per_graph)

    def _flush(self, mode, flush_bytes):
        """A callable that evicts the 256 MiB last-level cache by touching a buffer twice its
        size: mode "read" reads it (the cache is left holding clean lines, and whatever a
        step left dirty is written back inside the flush), mode "write" overwrites it (the
        cache is left full of dirty lines that the next kernel's misses must write back)."""
        torch = self.torch
        buf = torch.ones(flush_bytes // 4, dtype=torch.int32, device="cuda")
        if mode == "read":
            sink = torch.empty((), dtype=torch.int64, device="cuda")
            return lambda: torch.sum(buf, dim=0, out=sink)
        if mode == "write":
            return lambda: buf.fill_(1)
        raise ValueError(mode)

    def flushed_steps(self, steps, flush_bytes=512 << 20, mode="read"):
        """Each step timed alone after a flush of the last-level cache (see _flush), so that
        no input starts the step in that cache."""
        torch = self.torch
        flush = self._flush(mode, flush_bytes)
        total = 0.0
        e0, e1 = _events(2)
        for _ in range(steps):
            flush()
            e0.record()
            self.step()
            e1.record()
            torch.cuda.synchronize()
            total += e0.elapsed_time(e1)
        return total / steps

    def flushed_kernels(self, steps, flush_bytes=512 << 20, mode="read"):
        """The step's four kernels (the two-call halves of gn_forward and gn_backward, as
        in_step_kernels launches them) timed one by one after the same flush as
        flushed_steps: each step starts with no input in the last-level cache, and its
        kernels then see what the earlier ones left there. Mean milliseconds per kernel."""
        torch = self.torch
        ph = self.phases()
        n = len(ph)
        flush = self._flush(mode, flush_bytes)
        ev = _events(n + 1)
        total = [0.0] * n
        for _ in range(steps):
            flush()
            ev[0].record()
            for i, (_, f) in enumerate(ph):
                f()
                ev[i + 1].record()
            torch.cuda.synchronize()
            for i in range(n):
                total[i] += ev[i].elapsed_time(ev[i + 1])
        return {name: total[i] / steps for i, (name, _) in enumerate(ph)}

    def produced_steps(self, steps, fresh=True):
        """Steps whose inputs were just written, as in a training step where a convolution
        writes x right before the forward and dy right before the backward: x and dy are
        rewritten from twins (a read and a write of each) before each call, and only the two
        GroupNorm calls are timed (HIP events around each, all steps enqueued back to back).
        With fresh=False the same events bracket the same calls without the rewrites."""
        torch = self.torch
        xs, dys = (self.x.clone(), self.dy.clone()) if fresh else (None, None)
        ev = [_events(4) for _ in range(steps + 1)]
        for e in ev:
            if fresh:
                self.x.copy_(xs)
            e[0].record()
            self.fwd()
            e[1].record()
            if fresh:
                self.dy.copy_(dys)
            e[2].record()
            self.bwd()
            e[3].record()
        torch.cuda.synchronize()
        # the first step is dropped: the host enqueues it while the GPU is idle
        total = sum(e[0].elapsed_time(e[1]) + e[2].elapsed_time(e[3]) for e in ev[1:])
        return total / steps


def site_roofline(run, ceil, steps):
    """The dominant kernel (bwd_apply_fin_kernel: reads x and dy, writes dx; 6 of the 16
    bytes an element) timed inside the step, and every kernel against the ceiling's bound.

    An event recorded between two kernels delays the second by the event's own latency, so
    each bracketed kernel reads long by that much: the latency is measured as the four
    bracketed kernels' sum minus the same steps timed without the inner events (step time
    between two events around `steps` steps), divided by four, and taken off each kernel.
    The in-step figures are the least of three measurements (by their sum). The rocprofv3
    kernel trace of the same command, which times the kernels themselves, gives the same
    in-step averages."""
    step_ms, _ = run.timed_steps(steps, 3)
    # three measurements; the one with the smallest total has the fewest host-side gaps
    ks = min((run.in_step_kernels(steps) for _ in range(3)), key=lambda d: sum(d.values()))
    step_ms = (step_ms + run.timed_steps(steps, 0)[0]) / 2
    b2b = run.back_to_back_kernels(20)
    dom = "bwd_apply"
    raw_us = {k: v * 1e3 for k, v in ks.items()}
    event_us = max(0.0, (sum(raw_us.values()) - step_ms * 1e3) / len(raw_us))
    us = {k: v - event_us for k, v in raw_us.items()}
    dom_bytes = run.phase_bytes[dom] * run.case.numel
    dom_gbps = dom_bytes / (us[dom] * 1e-6) / 1e9
    kb = kernel_bounds(run.rw, run.case.numel, us, ceil) if ceil else None
    return {
        "bound": "hbm",
        "kernel": "bwd_apply_fin_kernel<bf16,bf16> (dx pass with the backward finalize folded in: "
                  "reads x and dy, writes dx)",
        "achieved": round(dom_gbps, 1),
        "peak": PEAK_HBM_GBPS,
        "unit": "GB/s",
        "frac": round(dom_gbps / PEAK_HBM_GBPS, 4),
        "algorithmic_bytes_per_launch": dom_bytes,
        "avg_launch_us": round(us[dom], 2),
        "timing": f"HIP events between the four kernels of each of {steps} back-to-back steps on the kernels' "
                  "stream (queued behind untimed steps; the least of three runs), less one event's latency (the "
                  "bracketed kernels' sum minus the step timed without the inner events, over four)",
        "event_latency_us": round(event_us, 2),
        "step_us_without_inner_events": round(step_ms * 1e3, 2),
        "ceiling_frac": kb[dom]["frac_of_bound"] if kb else None,
        "kernels_in_step_us": {k: round(v, 2) for k, v in us.items()},
        "kernels_in_step_with_event_us": {k: round(v, 2) for k, v in raw_us.items()},
        "kernels_back_to_back_us": {k: round(v * 1e3, 2) for k, v in b2b.items()},
        "kernels_vs_ceiling": kb,
    }


# ----------------------------------------------------------------------------- more workloads

def census(steps=10, warmup=3):
    """The 18 GroupNorm sites of a scale-7 UNet, fwd+bwd each, back to back: aggregate rate
    on method bytes, called eagerly and replayed from one captured HIP graph of the pass, the
    pass with every input just written (events around the GroupNorm calls, and the same
    events without the rewrites for comparison), every site's step after a last-level cache
    flush, and whether 10 repeats of every site are bitwise identical."""
    import torch

    import workloads
    runs = [Runner(c) for c in workloads.census_cases()]
    for r in runs:
        for _ in range(warmup):
            r.step()
    torch.cuda.synchronize()
    e0, e1 = _events(2)
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
    # inputs just written, and the same event pattern on resident inputs
    fresh_ms = sum(r.produced_steps(3, fresh=True) for r in runs)
    warm_ev_ms = sum(r.produced_steps(3, fresh=False) for r in runs)
    # every site's step after the last-level cache was flushed
    flushed_ms = sum(r.flushed_steps(3) for r in runs)
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
            "inputs_just_written": {"ms_per_pass": round(fresh_ms, 4),
                                    "value": round(total / (fresh_ms * 1e-3) / 1e9, 1),
                                    "same_events_resident_inputs_ms": round(warm_ev_ms, 4),
                                    "timing": "HIP events around each GroupNorm call (36 a pass)"},
            "llc_flushed": {"ms_per_pass": round(flushed_ms, 4),
                            "value": round(total / (flushed_ms * 1e-3) / 1e9, 1),
                            "timing": "each site's fwd+bwd step timed alone after a 512 MiB read"},
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
    e0, e1 = _events(2)
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
    call per direction from Python), replayed from a captured graph, and each step alone
    after a last-level cache flush."""
    import workloads
    out = {}
    for case in (workloads.TINY, workloads.DEEP, workloads.DEEP_F32OUT):
        r = Runner(case)
        r.settle(0.25)
        sms, _ = r.timed_steps(steps, warmup)
        gms = r.graph_steps()
        fms = r.flushed_steps(10)
        out[case.name] = {"us_per_step": round(sms * 1e3, 2),
                          "value": round(r.step_bytes / (sms * 1e-3) / 1e9, 1),
                          "bytes_per_step": r.step_bytes,
                          "graph_us_per_step": round(gms * 1e3, 2),
                          "graph_value": round(r.step_bytes / (gms * 1e-3) / 1e9, 1),
                          "llc_flushed_us_per_step": round(fms * 1e3, 2)}
        del r
    return out


def probe_copy(nbytes=1 << 30, reps=5):
    """The probe copy kernel over nbytes, reps times: a kernel of known traffic (nbytes read,
    nbytes written a launch) for scaling profiler byte counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        assert probe_lib().gnp_copy(src.data_ptr(), dst.data_ptr(), nbytes, 1, 1, 8, 4096, _stream_ptr()) == 0
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------- CPU baseline (the oracle)

def _timed(fn, min_seconds, max_reps):
    reps, total, out = 0, 0.0, None
    while reps < max_reps and (reps == 0 or total < min_seconds):
        t0 = time.perf_counter()
        out = fn()
        total += time.perf_counter() - t0
        reps += 1
    return total / reps, reps, out


def _host_cores():
    return len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)


def cpu_baseline(runner, min_seconds=4.0, max_reps=30):
    """The fp64 oracle, as it stands, on this host, on the whole volume of the headline site:
    the forward and the backward timed separately on one thread, then on all host cores
    (oracle_all_cores). Returns the baseline and the oracle's outputs of the last repetition."""
    from oracle import oracle as O
    x, dy = runner.x.cpu(), runner.dy.cpu()
    gamma, beta = runner.gamma.cpu(), runner.beta.cpu()
    G, eps = runner.G, runner.eps
    numel = runner.case.numel
    fwd_bytes = (runner.phase_bytes["stats"] + runner.phase_bytes["apply"]) * numel
    bwd_bytes = (runner.phase_bytes["bwd_reduce"] + runner.phase_bytes["bwd_apply"]) * numel
    tf, nf, f = _timed(lambda: O.forward(x, G, gamma, beta, eps=eps), min_seconds, max_reps)
    tb, nb, b = _timed(lambda: O.backward(dy, x, G, gamma, eps=eps), min_seconds, max_reps)
    allc = oracle_all_cores(x, dy, gamma, beta, G, eps, min_seconds=min_seconds / 2)
    import numpy as np
    o = allc.pop("_outputs")
    allc["outputs_bitwise_equal_to_one_thread"] = bool(
        all(np.array_equal(o[k], f[k]) for k in ("mean", "rstd", "y")) and
        all(np.array_equal(o[k], b[k]) for k in ("dx", "dgamma", "dbeta")))
    del o
    base = {
        "value": round(runner.step_bytes / (tf + tb) / 1e9, 3),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"the whole {runner.case.name} volume ({numel} elements): the fp64 oracle's forward "
                   f"({nf} repetitions, {tf:.3f} s each) and backward ({nb} repetitions, {tb:.3f} s each), "
                   "outputs in fp64, one thread; GB/s on the same method bytes as the GPU step"),
        "forward": {"seconds": round(tf, 4), "gbps": round(fwd_bytes / tf / 1e9, 3)},
        "backward": {"seconds": round(tb, 4), "gbps": round(bwd_bytes / tb / 1e9, 3)},
        "host_cpu": _cpu_model(),
        "host_cores_available": _host_cores(),
        "all_cores": {**allc,
                      "value": round(runner.step_bytes / (allc["forward"]["seconds"] + allc["backward"]["seconds"])
                                     / 1e9, 3),
                      "unit": "GB/s"},
    }
    base["all_cores"]["forward"]["gbps"] = round(fwd_bytes / allc["forward"]["seconds"] / 1e9, 3)
    base["all_cores"]["backward"]["gbps"] = round(bwd_bytes / allc["backward"]["seconds"] / 1e9, 3)
    return base, f, b


def oracle_all_cores(x, dy, gamma, beta, G, eps, min_seconds=2.0, max_reps=20, workers=None):
    """The same oracle spread over the host's cores (at most 16 threads; its C calls release
    the GIL), each direction in two phases of independent calls:
      forward:  the statistics of each (n, g) group (gno_group_stats on the group's channel
                slice, a one-group volume), then y of each (n, c) channel (gno_forward_at on the
                channel's row with its group's statistics);
      backward: the statistics, c1, c2 and per-channel sums of each (n, g) group (gno_backward
                without dx on the group's slice), then dx of each (n, c) channel
                (gno_backward_at on the row with its group's coefficients);
    dgamma/dbeta sum the groups' per-channel results over the samples in order. Every output
    is bitwise the whole-volume call's (the definition's sums run over the same elements in
    the same order). Returns the timings and the outputs."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from oracle import oracle as O
    N, C = int(x.shape[0]), int(x.shape[1])
    S = x.numel() // (N * C)
    Cg = C // G
    xr, dyr = x.reshape(N, C, S), dy.reshape(N, C, S)
    gam, bet = gamma.numpy().astype(np.float32), beta.numpy().astype(np.float32)
    groups = [(n, g) for n in range(N) for g in range(G)]
    rows = [(n, c) for n in range(N) for c in range(C)]
    idx = np.arange(S, dtype=np.int64)
    workers = workers or max(1, min(_host_cores(), 16))

    def fwd_stats(u):
        n, g = u
        return O.group_stats(xr[n:n + 1, g * Cg:(g + 1) * Cg], 1, eps)

    def fwd_rows(u, st):
        n, c = u
        m, _, r = st[n * G + c // Cg]
        return O.forward_at(xr[n:n + 1, c:c + 1], 1, idx, m, r, gam[c:c + 1], bet[c:c + 1])

    def bwd_groups(u):
        n, g = u
        sl = slice(g * Cg, (g + 1) * Cg)
        return O.backward(dyr[n:n + 1, sl], xr[n:n + 1, sl], 1, gam[sl], eps=eps, want_dx=False)

    def bwd_rows(u, bg):
        n, c = u
        b = bg[n * G + c // Cg]
        return O.backward_at(dyr[n:n + 1, c:c + 1], xr[n:n + 1, c:c + 1], 1, idx, b["mean"], b["rstd"], b["c1"],
                             b["c2"], gam[c:c + 1])

    with ThreadPoolExecutor(max_workers=workers) as pool:
        def forward():
            st = list(pool.map(fwd_stats, groups))
            return st, list(pool.map(lambda u: fwd_rows(u, st), rows))

        def backward():
            bg = list(pool.map(bwd_groups, groups))
            return bg, list(pool.map(lambda u: bwd_rows(u, bg), rows))

        tf, nf, (st, ys) = _timed(forward, min_seconds, max_reps)
        tb, nb, (bg, dxs) = _timed(backward, min_seconds, max_reps)
    dgamma, dbeta = np.zeros(C), np.zeros(C)
    for n in range(N):
        for g in range(G):
            b = bg[n * G + g]
            dgamma[g * Cg:(g + 1) * Cg] += b["dgamma"]
            dbeta[g * Cg:(g + 1) * Cg] += b["dbeta"]
    out = {"mean": np.array([s[0][0, 0] for s in st]).reshape(N, G),
           "rstd": np.array([s[2][0, 0] for s in st]).reshape(N, G),
           "y": np.stack(ys).reshape(x.shape), "dx": np.stack(dxs).reshape(x.shape),
           "dgamma": dgamma, "dbeta": dbeta}
    return {"cores": workers,
            "sample": (f"the same volume on {workers} threads: {len(groups)} (n, g) group calls then "
                       f"{len(rows)} (n, c) row calls per direction; forward {nf} and backward {nb} repetitions"),
            "forward": {"seconds": round(tf, 4)}, "backward": {"seconds": round(tb, 4)},
            "_outputs": out}


def accuracy(runner, f, b):
    """The GPU's outputs on the headline site against the oracle's (f: forward, b: backward
    of the same inputs), and dgamma/dbeta on the same site with a dy whose channel sums do
    not cancel, next to the accuracy the pages report for fp32 statistics against float64."""
    import numpy as np
    import torch

    import workloads
    from oracle import oracle as O
    runner.act = None
    runner.step()
    torch.cuda.synchronize()

    def bits(t):
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).reshape(-1)

    def ulp_dist(a, b):
        a, b = a.astype(np.int32), b.astype(np.int32)
        oa = np.where(a & 0x8000, -(a & 0x7FFF), a)
        ob = np.where(b & 0x8000, -(b & 0x7FFF), b)
        return np.abs(oa - ob)

    m = runner.mean.cpu().numpy().astype(np.float64)
    r = runner.rstd.cpu().numpy().astype(np.float64)
    sigma = np.sqrt(f["var"])
    yref = O.round_bf16(f["y"].reshape(-1))
    ybits = bits(runner.y)
    ydist = ulp_dist(ybits, yref)
    # elements beyond 1 ulp are those whose fp32 terms cancel near y = 0; they are held to the
    # fp32 bar instead, 1e-5 * max(|y64|, |gamma_c| + |beta_c|)
    far = np.nonzero(ydist > 1)[0]
    y_fallback = 0.0
    if far.size:
        c = (far // runner.case.S) % runner.case.C
        gm, bt = runner.gamma.cpu().numpy().astype(np.float64), runner.beta.cpu().numpy().astype(np.float64)
        y64 = f["y"].reshape(-1)[far]
        got = (ybits[far].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        bar = 1e-5 * np.maximum(np.abs(y64), np.abs(gm[c]) + np.abs(bt[c]))
        y_fallback = float(np.max(np.abs(got - y64) / bar))
    dx64 = b["dx"].reshape(-1)
    dxg = (bits(runner.dx).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dxdist = ulp_dist(bits(runner.dx), O.round_bf16(dx64))
    x, dy = runner.x.cpu(), runner.dy.cpu()
    a_dy, a_dyx = O.channel_abs_sums(dy, x, runner.G, b["mean"], b["rstd"])
    dg = runner.dgamma.cpu().numpy().astype(np.float64)
    db = runner.dbeta.cpu().numpy().astype(np.float64)
    out = {
        "pages_fp32_statistics_vs_float64": PAGES_FP32_STATS_VS_FP64,
        "workload": runner.case.name,
        "mean_max_rel_err": float(np.max(np.abs(m - f["mean"]) / np.abs(f["mean"]))),
        "mean_max_err_of_sigma": float(np.max(np.abs(m - f["mean"]) / sigma)),
        "rstd_max_rel_err": float(np.max(np.abs(r - f["rstd"]) / f["rstd"])),
        "y_max_ulp_from_fp64_rounded_once": int(ydist.max()),
        "y_frac_equal_to_fp64_rounded_once": float(np.mean(ydist == 0)),
        "y_beyond_1_ulp": int(np.sum(ydist > 1)),
        "y_beyond_1_ulp_max_err_of_fp32_bar": y_fallback,
        "dx_max_err_of_max_abs_dx": float(np.max(np.abs(dxg - dx64)) / np.max(np.abs(dx64))),
        "dx_max_ulp_from_fp64_rounded_once": int(dxdist.max()),
        "zero_mean_dy": {"dgamma_max_err_of_sum_abs_terms": float(np.max(np.abs(dg - b["dgamma"]) / a_dyx)),
                         "dbeta_max_err_of_sum_abs_terms": float(np.max(np.abs(db - b["dbeta"]) / a_dy)),
                         "note": "zero-mean dy: every channel sum cancels to ~1/sqrt(S) of its terms, so the "
                                 "error is stated against the sum of the terms' magnitudes"},
    }
    # dgamma/dbeta where the channel sums do not cancel: relative errors that mean something
    case = workloads.SCALE7_DY_OFFSET
    ro = Runner(case)
    ro.step()
    torch.cuda.synchronize()
    bo = O.backward(ro.dy.cpu(), ro.x.cpu(), ro.G, ro.gamma.cpu(), eps=ro.eps, want_dx=False)
    dgo = ro.dgamma.cpu().numpy().astype(np.float64)
    dbo = ro.dbeta.cpu().numpy().astype(np.float64)
    out["offset_dy"] = {"workload": case.name,
                        "dgamma_max_rel_err": float(np.max(np.abs(dgo - bo["dgamma"]) / np.abs(bo["dgamma"]))),
                        "dbeta_max_rel_err": float(np.max(np.abs(dbo - bo["dbeta"]) / np.abs(bo["dbeta"]))),
                        "bar": 1e-4}
    del ro
    return out


def _bf16_ulp_dist(a, b):
    """Distance in bf16 units in the last place between two arrays of bf16 bit patterns
    (sign-magnitude mapped onto a line, so that +0 and -0 are 0 apart)."""
    import numpy as np
    a, b = a.astype(np.int32), b.astype(np.int32)
    oa = np.where(a & 0x8000, -(a & 0x7FFF), a)
    ob = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(oa - ob)


def accuracy_streamed(runner, workers=None):
    """The GPU's outputs on a bf16 NCDHW volume too large to hold in fp64 at once, against
    the oracle group by group and channel by channel, the calls oracle_all_cores makes:
    mean and rstd of each (n, g) against the oracle's group statistics; y and dx of each
    (n, c) row as bf16 ulp distances from the fp64 value rounded once (y beyond 1 ulp held
    to the fp32 bar 1e-5 * max(|y|, |gamma_c| + |beta_c|), as on the headline site); dgamma
    and dbeta against the sums of their terms' magnitudes (dy has zero mean, so the channel
    sums cancel). Only per-row summaries are kept."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import torch

    from oracle import oracle as O
    runner.act = None
    runner.step()
    torch.cuda.synchronize()
    case = runner.case
    N, C, G, S = case.N, case.C, runner.G, case.S
    Cg = C // G
    x, dy = runner.x.cpu().reshape(N, C, S), runner.dy.cpu().reshape(N, C, S)

    def bits(t):
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).reshape(N, C, S)

    ybits, dxbits = bits(runner.y), bits(runner.dx)
    gam, bet = runner.gamma.cpu().numpy(), runner.beta.cpu().numpy()
    m_gpu = runner.mean.cpu().numpy().astype(np.float64).reshape(-1)
    r_gpu = runner.rstd.cpu().numpy().astype(np.float64).reshape(-1)
    dg_gpu = runner.dgamma.cpu().numpy().astype(np.float64)
    db_gpu = runner.dbeta.cpu().numpy().astype(np.float64)
    idx = np.arange(S, dtype=np.int64)
    groups = [(n, g) for n in range(N) for g in range(G)]
    rows = [(n, c) for n in range(N) for c in range(C)]
    workers = workers or max(1, min(_host_cores(), 16))

    def group(u):
        n, g = u
        sl = slice(g * Cg, (g + 1) * Cg)
        st = O.group_stats(x[n:n + 1, sl], 1, runner.eps)
        b = O.backward(dy[n:n + 1, sl], x[n:n + 1, sl], 1, gam[sl], eps=runner.eps, want_dx=False)
        a_dy, a_dyx = O.channel_abs_sums(dy[n:n + 1, sl], x[n:n + 1, sl], 1, b["mean"], b["rstd"])
        return st, b, a_dy, a_dyx

    def row(u, gs):
        n, c = u
        st, b, _, _ = gs[n * G + c // Cg]
        xr, dyr = x[n:n + 1, c:c + 1], dy[n:n + 1, c:c + 1]
        y64 = O.forward_at(xr, 1, idx, st[0], st[2], gam[c:c + 1], bet[c:c + 1])
        yd = _bf16_ulp_dist(ybits[n, c], O.round_bf16(y64))
        far = np.nonzero(yd > 1)[0]
        yfb = 0.0
        if far.size:
            got = (ybits[n, c][far].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            bar = 1e-5 * np.maximum(np.abs(y64[far]), abs(float(gam[c])) + abs(float(bet[c])))
            yfb = float(np.max(np.abs(got - y64[far]) / bar))
        dx64 = O.backward_at(dyr, xr, 1, idx, b["mean"], b["rstd"], b["c1"], b["c2"], gam[c:c + 1])
        dxd = _bf16_ulp_dist(dxbits[n, c], O.round_bf16(dx64))
        dxg = (dxbits[n, c].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return {"y_max_ulp": int(yd.max()), "y_equal": int(np.sum(yd == 0)), "y_beyond_1": int(far.size),
                "y_fallback": yfb, "dx_max_ulp": int(dxd.max()), "dx_max_err": float(np.max(np.abs(dxg - dx64))),
                "dx_max_abs": float(np.max(np.abs(dx64)))}

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=workers) as pool:
        gs = list(pool.map(group, groups))
        rs = list(pool.map(lambda u: row(u, gs), rows))
    mean64 = np.array([g[0][0][0, 0] for g in gs])
    sigma64 = np.sqrt(np.array([g[0][1][0, 0] for g in gs]))
    rstd64 = np.array([g[0][2][0, 0] for g in gs])
    dg64, db64, a_dy, a_dyx = np.zeros(C), np.zeros(C), np.zeros(C), np.zeros(C)
    for (n, g), (_, b, ad, adx) in zip(groups, gs):
        sl = slice(g * Cg, (g + 1) * Cg)
        dg64[sl] += b["dgamma"]
        db64[sl] += b["dbeta"]
        a_dy[sl] += ad
        a_dyx[sl] += adx
    return {
        "workload": case.name,
        "method": (f"the oracle per (n, g) group and per (n, c) row on {workers} threads "
                   f"({len(groups)} groups, {len(rows)} rows, {time.perf_counter() - t0:.1f} s); no fp64 "
                   "tensor of the whole volume is formed"),
        "mean_max_rel_err": float(np.max(np.abs(m_gpu - mean64) / np.abs(mean64))),
        "mean_max_err_of_sigma": float(np.max(np.abs(m_gpu - mean64) / sigma64)),
        "rstd_max_rel_err": float(np.max(np.abs(r_gpu - rstd64) / rstd64)),
        "y_max_ulp_from_fp64_rounded_once": max(r["y_max_ulp"] for r in rs),
        "y_frac_equal_to_fp64_rounded_once": sum(r["y_equal"] for r in rs) / case.numel,
        "y_beyond_1_ulp": sum(r["y_beyond_1"] for r in rs),
        "y_beyond_1_ulp_max_err_of_fp32_bar": max(r["y_fallback"] for r in rs),
        "dx_max_err_of_max_abs_dx": max(r["dx_max_err"] for r in rs) / max(r["dx_max_abs"] for r in rs),
        "dx_max_ulp_from_fp64_rounded_once": max(r["dx_max_ulp"] for r in rs),
        "zero_mean_dy": {"dgamma_max_err_of_sum_abs_terms": float(np.max(np.abs(dg_gpu - dg64) / a_dyx)),
                         "dbeta_max_err_of_sum_abs_terms": float(np.max(np.abs(db_gpu - db64) / a_dy))},
    }


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
            probe_copy()
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
    e0, e1 = _events(2)
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
        probe_copy()
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
    ceil = None
    if not args.no_extras:
        log("streaming ceiling: probe read, write and copy kernels over 1 GiB")
        ceil = ceiling()
    log(f"workload {case.name} {case.shape}; generating inputs on the GPU")
    run = Runner(case)
    settled = run.settle(args.settle) if args.settle > 0 else 0
    log(f"timing {args.steps} steps after {settled} settling and {args.warmup} warmup steps")
    ms, wall = run.timed_steps(args.steps, args.warmup)
    value = run.step_bytes / (ms * 1e-3) / 1e9
    log("the same steps timed one by one: 7 trials of 20")
    proto = run.step_protocol()

    log("timing each kernel inside the step with HIP events")
    roofline = site_roofline(run, ceil, max(args.steps, 50))
    traffic, traffic_note = load_traffic(case.name)
    roofline["traffic"] = (traffic or {}).get("bytes_per_launch")
    roofline["traffic_note"] = traffic_note if traffic is None else traffic.get("note", "ok")
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
        "step_protocol": {**proto,
                          "value_at_median": round(run.step_bytes / (proto["median_ms"] * 1e-3) / 1e9, 1),
                          "value_at_min_of_medians": round(run.step_bytes / (proto["min_of_medians_ms"] * 1e-3) / 1e9,
                                                           1)},
        "roofline": roofline,
        "ceiling": ceil,
        "kernel_source_hash": kernel_source_hash(),
        "settle": {"seconds": args.settle, "steps": settled},
    }
    if not args.no_extras:
        out["compulsory_bytes_gbps"] = round(10 * case.numel / (ms * 1e-3) / 1e9, 1)
        log("timing steps with the last-level cache flushed before each")
        nfl = max(10, args.steps // 5)

        def flushed(mode):
            fms = run.flushed_steps(nfl, mode=mode)
            fk = run.flushed_kernels(nfl, mode=mode)
            return {
                "ms_per_step": round(fms, 5),
                "value": round(run.step_bytes / (fms * 1e-3) / 1e9, 1),
                "pct_of_peak": round(100 * run.step_bytes / (fms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
                "compulsory_bytes_gbps": round(10 * case.numel / (fms * 1e-3) / 1e9, 1),
                "kernels": {name: {"us": round(1e3 * t, 2),
                                   "gbps": round(run.phase_bytes[name] * case.numel / (t * 1e-3) / 1e9, 1)}
                            for name, t in fk.items()},
            }

        out["llc_flushed"] = {"flush": "512 MiB read before each step (clean eviction)", **flushed("read")}
        out["llc_flushed_dirty"] = {"flush": "512 MiB overwritten before each step (the cache left dirty)",
                                    **flushed("write")}
        log("timing steps whose inputs were just rewritten (x before the forward, dy before the backward)")
        pms = run.produced_steps(max(10, args.steps // 5))
        out["inputs_just_written"] = {"ms_per_step": round(pms, 5),
                                      "value": round(run.step_bytes / (pms * 1e-3) / 1e9, 1)}
        log("the same step with the relu fused into the normalize store and the backward gate")
        run.act = "relu"
        rms, _ = run.timed_steps(max(10, args.steps // 2), 3)
        out["relu_fused"] = {"ms_per_step": round(rms, 5),
                             "value": round(run.step_bytes / (rms * 1e-3) / 1e9, 1)}
        run.act = None
        log("the same site in channels-last (NDHWC) memory")
        rcl = Runner(case, layout="ndhwc")
        rcl.settle(0.3)
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
        log("timing the fp64 CPU oracle on this host (one core, then all cores) and the GPU's accuracy against it")
        base, f, b = cpu_baseline(run)
        out["cpu_baseline"] = base
        out["accuracy"] = accuracy(run, f, b)
        del f, b
    if args.copy_probe:
        log("copy probe: 5 copies of 1 GiB")
        probe_copy()
    if not args.no_extras and args.workload == "scale7":
        del run
        torch.cuda.empty_cache()
        c8 = workloads.SCALE8
        log(f"secondary workload {c8.name}")
        r8 = Runner(c8)
        r8.settle(0.5)
        ms8, _ = r8.timed_steps(max(5, args.steps // 5), 3)
        proto8 = r8.step_protocol(trials=7, per_trial=5)
        roof8 = site_roofline(r8, ceil, 10)
        traffic8, note8 = load_traffic(c8.name)
        roof8["traffic"] = (traffic8 or {}).get("bytes_per_launch")
        roof8["traffic_note"] = note8 if traffic8 is None else traffic8.get("note", "ok")
        fms8 = r8.flushed_steps(5)
        pms8 = r8.produced_steps(5)
        out["scale8"] = {
            "workload": c8.name, "ms_per_step": round(ms8, 4),
            "value": round(r8.step_bytes / (ms8 * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * r8.step_bytes / (ms8 * 1e-3) / 1e9 / PEAK_HBM_GBPS, 2),
            "step_protocol": proto8,
            "roofline": roof8,
            "llc_flushed": {"ms_per_step": round(fms8, 4),
                            "value": round(r8.step_bytes / (fms8 * 1e-3) / 1e9, 1)},
            "inputs_just_written": {"ms_per_step": round(pms8, 4),
                                    "value": round(r8.step_bytes / (pms8 * 1e-3) / 1e9, 1)},
        }
        if not args.no_cpu_baseline:
            log(f"the GPU's accuracy on {c8.name} against the oracle, group by group and row by row")
            out["scale8"]["accuracy"] = accuracy_streamed(r8)
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
