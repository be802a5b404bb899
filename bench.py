#!/usr/bin/env python3
"""Benchmark of the depthwise causal conv1d decode update on one MI355X.

One step is one decode-update call (slot routing, x/state/weight loads, shift and
write-back, 4-tap dot, activation, BF16 store) over one batch of the large decode
workload: N=256 rows, D=8192 channels, W=4, L=3, S=256 slots, x row stride 8200,
SiLU, no bias, no index table.  Inputs are seeded synthetic BF16 data already in
HBM.  The call runs through the library's C ABI on torch's current stream.

Cold-cache timing: the working set of one call (about 21 MB) fits in the 256 MB
Infinity Cache, so consecutive steps cycle through enough independent buffer sets
(x, state, weight, output) to exceed it; every step then reads from HBM.

Timing: a timed region is exactly K steps, bracketed by device
synchronisations and timed with HIP events (created without the system-scope
fence, which the timed work does not need) on the stream that launches the
kernels.  Up to 32 steps the region's launches go straight to the stream
behind a busy kernel (every SIMD running arithmetic) that holds the GPU until
the host has enqueued them all, so the steps run back to back on a chip at its
working clocks; a HIP graph replay would add about 7 us per region here,
a third of a microsecond per step at K = 20.  Longer regions are
replayed from HIP graphs (several, when the buffer sets outnumber K, so the
regions keep cycling through every set).  The per-step time reported is the
median over the regions, with p10 and p90.  A plain copy of the same byte count
(the library's measurement-control copy, same buffer rotation, same launch
method) is timed right after the update's regions, as many regions, as a
control.

Achieved bandwidth is the algorithmic byte count of a call (x + selected state
read + state write + weight + bias + output + index table) divided by the
median time per step.

Prints exactly one JSON line on stdout; details go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s + decode rows/s, conv1d_update N=256 D=8192 W=4"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "depthwise_causal_conv1d_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _code_only(text: str) -> str:
    """C++ source without comments, blank lines and runs of white space (an edit
    of those leaves the compiled kernel, and so its counters, unchanged)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(line.split()) for line in text.splitlines() if line.strip())


def kernel_source_hash(kernel: str) -> str:
    """Hash of the code a kernel is compiled from (its file and the shared device
    helpers, comments left out), so stale counter summaries are recognised."""
    main = ("update_ring.hip" if kernel.startswith("tokens_ring") else
            "update_tokens.hip" if kernel.startswith("tokens_") else
            "prefill.hip" if kernel.startswith("prefill_") else
            "update_ring.hip" if kernel.startswith("update_ring") else "update.hip")
    h = hashlib.sha256()
    for name in (main, "device_common.h"):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none or the kernel source changed since the counters were taken."""
    safe = kernel.split("<")[0].replace("_edges", "")  # a prefill call is edges + chunks: "prefill_v8"
    path = os.path.join(PROFILES, f"traffic_{safe}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash(kernel) or vals.get("kernel") != kernel:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Workload:
    """Device buffer sets for one synthetic workload, cycled per step."""

    def __init__(self, spec, rotate_bytes: float, dev):
        import numpy as np
        import torch
        from depthwise_causal_conv1d_amd import workloads as wl

        self.spec = spec
        data = wl.make(spec)
        self.host = data

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

        self.tokens = spec.T if spec.one_call else 1
        set_bytes = (data["x"][0].nbytes * self.tokens + data["state"].nbytes + data["weight"].nbytes
                     + 2 * spec.N * spec.D * self.tokens + (data["bias"].nbytes if data["bias"] is not None else 0))
        self.n_sets = min(128, max(1, int(math.ceil(rotate_bytes / set_bytes))))
        self.sets = []
        x_all = up(data["x"])  # [T, N, ld]
        idx = None if data["indices"] is None else torch.from_numpy(data["indices"]).to(dev)
        self.seqlens = None if data.get("seqlens") is None else torch.from_numpy(data["seqlens"]).to(dev)
        for i in range(self.n_sets):
            st = up(data["state"])
            if spec.layout == "channel_last":
                st = st.permute(0, 2, 1)
            self.sets.append(dict(
                x=x_all.clone(),
                state=st,
                weight=up(data["weight"]),
                bias=None if data["bias"] is None else up(data["bias"]),
                idx=idx,
                out=torch.empty(spec.N, self.tokens, spec.D, dtype=torch.bfloat16, device=dev)))
        self.set_bytes = set_bytes
        active = spec.N if data["indices"] is None else int((data["indices"] >= 0).sum())
        self.active = active  # rows with a slot (the rest are padding)
        self.bytes_per_call = wl.algorithmic_bytes(spec.N, spec.D, spec.W, spec.L, active,
                                                   data["bias"] is not None, data["indices"] is not None,
                                                   spec.layout, self.tokens, spec.ring)

    def step(self, i: int):
        import depthwise_causal_conv1d_amd as dc

        s = self.sets[i % self.n_sets]
        D = self.spec.D
        if self.spec.one_call:
            # x [T, N, ld] seen as [N, D, T]; out [N, T, D] seen as [N, D, T]
            dc.causal_conv1d_update_tokens(s["x"][:, :, :D].permute(1, 2, 0), s["state"], s["weight"], s["bias"],
                                           self.spec.act, out=s["out"].permute(0, 2, 1),
                                           conv_state_indices=s["idx"], cache_seqlens=self.seqlens)
            return
        t = (i // self.n_sets) % self.spec.T
        dc.causal_conv1d_update_out(s["x"][t, :, :D], s["state"], s["weight"], s["bias"],
                                    self.spec.act, out=s["out"][:, 0, :], conv_state_indices=s["idx"],
                                    cache_seqlens=self.seqlens)


class PrefillWorkload:
    """Device buffer sets for one prefill workload (x, out and the state pool),
    cycled per step; the state's initial values change from step to step (each
    call's final state is the next one's initial state), which the cost does not
    depend on."""

    def __init__(self, spec, rotate_bytes: float, dev):
        import numpy as np
        import torch
        from depthwise_causal_conv1d_amd import workloads as wl

        self.spec = spec
        data = wl.make_prefill(spec)
        self.host = data

        def up(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

        total, D = data["total"], spec.D
        set_bytes = 4 * total * D + (data["state"].nbytes if data["state"] is not None else 0)
        self.n_sets = min(128, max(1, int(math.ceil(rotate_bytes / set_bytes))))
        self.set_bytes = set_bytes
        self.tokens = 1
        self.rows = total
        packed = spec.lens is not None
        self.weight = up(data["weight"])
        self.bias = None if data["bias"] is None else up(data["bias"])
        self.idx = None if data["indices"] is None else torch.from_numpy(data["indices"]).to(dev)
        self.has_init = None if data["has_init"] is None else torch.from_numpy(data["has_init"]).to(dev)
        self.starts = None if data["starts"] is None else torch.from_numpy(data["starts"]).to(dev)
        self.sets = []
        for _ in range(self.n_sets):
            xb = up(data["x"])
            x = xb.view(1, total, D).permute(0, 2, 1) if packed else xb.permute(0, 2, 1)
            ob = torch.empty_like(xb)
            out = ob.view(1, total, D).permute(0, 2, 1) if packed else ob.permute(0, 2, 1)
            st = None
            if data["state"] is not None:
                st = up(data["state"])
                if spec.layout == "channel_last":
                    st = st.permute(0, 2, 1)
            self.sets.append(dict(x=x, out=out, state=st))
        self.bytes_per_call = wl.prefill_algorithmic_bytes(spec, data["has_init"])

    def step(self, i: int):
        import depthwise_causal_conv1d_amd as dc

        s = self.sets[i % self.n_sets]
        dc.causal_conv1d(s["x"], self.weight, self.bias, self.spec.act, conv_state=s["state"],
                         conv_state_indices=self.idx, has_initial_state=self.has_init, seq_starts=self.starts,
                         out=s["out"])


class Head:
    """A busy kernel enqueued ahead of a timed region: while every SIMD runs
    arithmetic (the library's ``dcconv_busy_spin``, timed by the device's wall
    clock), the host finishes enqueueing the region's launches, so the start
    event is followed directly by the first step, the steps run back to back,
    and the region starts on a chip at its working clocks.  (Behind a one-thread
    spin the chip idles and the packed prefill region measured about 3 % slower;
    the decode regions measured the same behind either.)  ``__call__(us)``
    spins for about ``us`` microseconds."""

    available = True

    def __call__(self, us: float):
        import depthwise_causal_conv1d_amd as dc

        dc.busy_spin(us)


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    does not write back and invalidate the caches (a system-scope fence the
    timed work does not need), which HIP documents as making timings between
    events more precise.  The region is still closed by a device
    synchronisation, which is a full fence."""

    _hip = None

    def __init__(self):
        import ctypes

        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self.ev = ctypes.c_void_p()
        rc = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(0x20000000))
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self, stream):
        import ctypes

        rc = TimingEvent._hip.hipEventRecord(self.ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_us(self, end) -> float:
        import ctypes

        ms = ctypes.c_float()
        rc = TimingEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value * 1e3

    def __del__(self):
        hip = TimingEvent._hip if TimingEvent is not None else None
        if hip is not None and self.ev:
            hip.hipEventDestroy(self.ev)


# Up to this many steps a timed region is launched directly on the stream behind
# the busy head (every launch then fits in the hardware queue while the GPU
# spins); longer regions are replayed from a HIP graph.  A replay costs about
# 7 us once behind the busy head, and a graph node 0.14-0.48 us less than a
# direct launch, so graphs win from about 35 steps on (large decode: 20 steps
# 6.41 direct against 6.58 as a graph, 100 steps 6.43 against 6.29).
EAGER_MAX_STEPS = 32


def timing_mode(launch: str, steps: int, head_available: bool) -> str:
    """How a region of ``steps`` steps is launched: ``eager`` when asked for,
    else direct launches behind the head (``eager+head``) up to EAGER_MAX_STEPS
    steps, else ``graph``."""
    if launch == "graph" and steps <= EAGER_MAX_STEPS and head_available:
        return "eager+head"
    return launch


class Timer:
    """Times regions of exactly K steps: K launches between two timing events,
    bracketed by device synchronisations, returning microseconds per step."""

    def __init__(self, step, first: int, steps: int, n_sets: int, launch: str, head: Head):
        self.step, self.first, self.steps, self.head = step, first, steps, head
        self.mode = timing_mode(launch, steps, head.available)
        self.graphs = capture(step, first, steps, n_sets) if self.mode == "graph" else []
        self.n_regions = max(1, min(16, math.ceil(n_sets / steps)))
        # host time to enqueue one step, for sizing the spin ahead of an eager region
        import torch

        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(min(steps, 32)):
            step(first + i)
        self.host_us = (time.perf_counter() - t0) * 1e6 / min(steps, 32)
        torch.cuda.synchronize()

    def region(self, r: int) -> float:
        import torch

        stream = torch.cuda.current_stream()
        start, end = TimingEvent(), TimingEvent()
        torch.cuda.synchronize()
        if self.mode == "graph":
            self.head(200.0)
            start.record(stream)
            self.graphs[r % len(self.graphs)].replay()
        else:
            base = self.first + (r % self.n_regions) * self.steps
            if self.mode == "eager+head":
                self.head(100.0 + 2.0 * self.steps * self.host_us)
            start.record(stream)
            for i in range(self.steps):
                self.step(base + i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_us(end) / self.steps


def capture(step, first: int, steps: int, n_sets: int):
    """Graphs of ``steps`` consecutive steps each, starting at step ``first``, as
    many as it takes for the replays to cycle through all ``n_sets`` buffer sets."""
    import torch

    graphs = []
    n_graphs = max(1, min(16, math.ceil(n_sets / steps)))
    for j in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                step(first + j * steps + i)
        graphs.append(g)
    for g in graphs:  # one untimed replay each: graph upload
        g.replay()
    torch.cuda.synchronize()
    return graphs


def quantiles(v):
    import numpy as np

    a = np.asarray(v, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "median": float(np.median(a)), "p90": float(np.percentile(a, 90))}


class CopyControl:
    """The library's measurement-control copy of ``nbytes`` bytes per call (half
    the call's bytes read, half written), over a rotation of source/destination
    pairs as large as the workload's."""

    def __init__(self, nbytes: int, rotate_bytes: float, dev):
        import torch

        self.half = max(16, (nbytes // 2) // 16 * 16)
        self.n_sets = min(128, max(1, int(math.ceil(rotate_bytes / (2 * self.half)))))
        self.src = [torch.ones(self.half, dtype=torch.uint8, device=dev) for _ in range(self.n_sets)]
        self.dst = [torch.empty(self.half, dtype=torch.uint8, device=dev) for _ in range(self.n_sets)]
        self.bytes_per_call = 2 * self.half

    def step(self, i: int):
        import depthwise_causal_conv1d_amd as dc

        k = i % self.n_sets
        dc.stream_copy(self.dst[k], self.src[k])


def measure(spec, steps: int, warmup: int, rotate_mb: float, launch: str, replays: int, head=None,
            copy: bool = False):
    """Times the workload (and, with ``copy``, the copy control of the same bytes,
    in the same number of regions right after the workload's)."""
    import torch
    import depthwise_causal_conv1d_amd as dc
    from depthwise_causal_conv1d_amd import workloads as wl

    dev = torch.device("cuda", torch.cuda.current_device())
    if isinstance(spec, wl.PrefillSpec):
        wk = PrefillWorkload(spec, rotate_mb * 2 ** 20, dev)
    else:
        wk = Workload(spec, rotate_mb * 2 ** 20, dev)
    for i in range(warmup):
        wk.step(i)
    kernel = dc.dcconv_last_kernel()
    torch.cuda.synchronize()
    if head is None:
        head = Head()
    cc = None
    if copy:
        cc = CopyControl(wk.bytes_per_call, rotate_mb * 2 ** 20, dev)
        for i in range(warmup):
            cc.step(i)
    times, copy_times, t_wall = [], [], 0.0
    timer = Timer(wk.step, warmup, steps, wk.n_sets, launch, head)
    ctimer = Timer(cc.step, warmup, steps, cc.n_sets, launch, head) if cc is not None else None
    # the workload's regions first, then the control's: a copy region's freshly
    # written bytes slowed the workload region right after it (long history,
    # 20-step regions: 5.50 us per call interleaved, 5.17 alone)
    for r in range(replays):
        t0 = time.perf_counter()
        times.append(timer.region(r))
        t_wall += time.perf_counter() - t0
    if ctimer is not None:
        for r in range(replays):
            copy_times.append(ctimer.region(r))
    del timer, ctimer
    q = quantiles(times)
    us = q["median"]
    ms = us * 1e-3
    res = dict(workload=spec.name, kernel=kernel, ms_per_step=ms, us_per_call=us,
               us_p10=q["p10"], us_p90=q["p90"], replays=len(times),
               wall_ms_per_step=t_wall * 1e3 / (steps * len(times)), bytes_per_call=wk.bytes_per_call,
               gbs=wk.bytes_per_call / (ms * 1e-3) / 1e9,
               rows_per_s=getattr(wk, "rows", spec.N * wk.tokens) / (ms * 1e-3),
               tokens_per_call=wk.tokens,
               buffer_sets=wk.n_sets, set_bytes=wk.set_bytes)
    res["timing_mode"] = timing_mode(launch, steps, head.available)
    res["frac"] = res["gbs"] / PEAK_HBM_GBS
    if getattr(wk, "active", spec.N) != spec.N:
        res["active_rows_per_s"] = wk.active * wk.tokens / (ms * 1e-3)
    if copy_times:
        cq = quantiles(copy_times)
        res["copy"] = {"bytes_per_call": cc.bytes_per_call, "us_per_call": cq["median"], "us_p10": cq["p10"],
                       "us_p90": cq["p90"], "gbs": cc.bytes_per_call / (cq["median"] * 1e-6) / 1e9,
                       "buffer_sets": cc.n_sets}
        res["copy"]["frac"] = res["copy"]["gbs"] / PEAK_HBM_GBS
        # the update's rate as a fraction of the copy's (same bytes per call)
        res["frac_of_copy"] = (wk.bytes_per_call / us) / (cc.bytes_per_call / cq["median"])
        del cc
    host = wk.host
    del wk
    torch.cuda.empty_cache()
    return res, host


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except Exception:
        return os.cpu_count() or 1


def _oracle_rows(spec, host, st, a: int, b: int):
    """The oracle's update of rows [a, b) of a decode workload, in place on the
    host state ``st`` (rows of a batch touch distinct slots, so disjoint row
    ranges may run concurrently)."""
    import numpy as np
    import oracle
    from depthwise_causal_conv1d_amd import workloads as wl

    tokens = spec.T if spec.one_call else 1
    strides = wl.state_strides(spec)
    n, ld = b - a, spec.ld
    flat = st.reshape(-1)
    if host["indices"] is None:
        # row r uses slot r: hand over the state from slot a on
        sbuf, S, idx = flat[a * strides[0]:], spec.S - a, None
    else:
        sbuf, S, idx = flat, spec.S, np.ascontiguousarray(host["indices"][a:b])
    xs = host["x"].reshape(-1)  # [T, N, ld]
    if spec.ring:
        sl = np.ascontiguousarray(host["seqlens"][a:b])
        for t in range(tokens):  # a multi-token ring call is its tokens' ring steps in order
            xt = host["x"][t].reshape(-1)[a * ld:]
            oracle.update_ring(xt, n, spec.D, ld, sbuf, S, spec.L, strides, host["weight"], host["bias"], idx,
                               sl + t, spec.act)
    elif tokens == 1:
        oracle.update_strided(xs[a * ld:], n, spec.D, ld, sbuf, S, spec.L, strides, host["weight"], host["bias"],
                              idx, spec.act)
    else:
        oracle.update_tokens(xs[a * ld:], n, spec.D, tokens, (ld, 1, spec.N * ld), sbuf, S, spec.L, strides,
                             host["weight"], host["bias"], idx, spec.act)


def cpu_baseline(spec, host, seconds: float):
    """The oracle as it stands (plain C, one thread per call) on the same workload:
    once on one core, and once on every core of the host (the batch's rows split
    into one contiguous range per core, each range one oracle call on its own
    thread; ctypes releases the interpreter lock during the call)."""
    import concurrent.futures as cf
    import numpy as np
    from depthwise_causal_conv1d_amd import workloads as wl

    if isinstance(spec, wl.PrefillSpec):
        return cpu_baseline_prefill(spec, host, seconds)
    tokens = spec.T if spec.one_call else 1
    active = spec.N if host["indices"] is None else int((host["indices"] >= 0).sum())
    b = wl.algorithmic_bytes(spec.N, spec.D, spec.W, spec.L, active, host["bias"] is not None,
                             host["indices"] is not None, spec.layout, tokens, spec.ring)

    def timed(cores: int, budget: float):
        bounds = [round(i * spec.N / cores) for i in range(cores + 1)]
        ranges = [(bounds[i], bounds[i + 1]) for i in range(cores) if bounds[i + 1] > bounds[i]]
        per, total = [], 0.0
        with cf.ThreadPoolExecutor(max_workers=len(ranges)) as pool:
            while len(per) < 5 or total < budget:
                st = host["state"].copy()
                t0 = time.perf_counter()
                if len(ranges) == 1:
                    _oracle_rows(spec, host, st, 0, spec.N)
                else:
                    for f in [pool.submit(_oracle_rows, spec, host, st, lo, hi) for lo, hi in ranges]:
                        f.result()
                dt = time.perf_counter() - t0
                per.append(dt)
                total += dt
        return float(np.median(per)), len(per), len(ranges)

    one, reps1, _ = timed(1, seconds)
    cores = host_cores()
    many, reps_n, threads = timed(cores, seconds / 2)
    cpu = ""
    try:
        cpu = next(l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name"))
    except Exception:
        pass
    return {"value": b / many / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps_n} full {spec.name} calls (N={spec.N}, D={spec.D}, L={spec.L}, {tokens} token(s)) "
                      f"on host arrays, rows split over {threads} threads, median {many * 1e3:.2f} ms per call",
            "rows_per_s": spec.N * tokens / many, "cpu_model": cpu,
            "single_thread": {"value": b / one / 1e9, "unit": "GB/s", "cores": 1,
                              "sample": f"{reps1} full calls on one thread, median {one * 1e3:.1f} ms per call",
                              "rows_per_s": spec.N * tokens / one}}


def cpu_baseline_prefill(spec, host, seconds: float):
    """The oracle's prefill (single thread) on the first sequences of the workload,
    as many as take about ``seconds``; reported per token."""
    import numpy as np
    import oracle
    from depthwise_causal_conv1d_amd import workloads as wl

    lens = list(spec.lens) if spec.lens is not None else [spec.T] * spec.N
    D = spec.D
    strides = wl.state_strides(spec) if spec.layout != "none" else (0, 0, 0)
    x = host["x"].reshape(-1, D)
    reps, t_total, toks, bytes_done, p0 = 0, 0.0, 0, 0, 0
    for i, t in enumerate(lens):
        xi = np.ascontiguousarray(x[p0:p0 + t])
        p0 += t
        st = None if host["state"] is None else host["state"].copy()
        idx = None if host["indices"] is None else host["indices"][i:i + 1].copy()
        hi = None if host["has_init"] is None else host["has_init"][i:i + 1].copy()
        t0 = time.perf_counter()
        oracle.prefill(xi, 1, D, t, (t * D, 1, D), host["weight"], host["bias"], spec.act, state_buf=st,
                       S=spec.S if st is not None else 0, L=spec.L if st is not None else 0, state_strides=strides,
                       indices=idx if idx is not None else (np.array([i], np.int32) if st is not None else None),
                       has_init=hi)
        t_total += time.perf_counter() - t0
        reps += 1
        toks += t
        bytes_done += 4 * t * D + 2 * D * spec.L
        if t_total >= seconds:
            break
    return {"value": bytes_done / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the first {reps} sequences ({toks} tokens, D={D}) of {spec.name} on host arrays, "
                      f"single thread, {t_total * 1e3 / max(toks, 1):.3f} ms per token",
            "rows_per_s": toks / t_total}


def config_of(spec, res, launch):
    """The workload as a config object (no model keys)."""
    import dataclasses
    cfg = {"workload": spec.name}
    for k, v in dataclasses.asdict(spec).items():
        if k in ("name", "seed"):
            continue
        cfg[k] = list(v) if isinstance(v, tuple) else v
    cfg["activation"] = cfg.pop("act", None) or "identity"
    cfg["accumulate"] = "f32"
    cfg["buffer_sets"] = res["buffer_sets"]
    cfg["launch"] = res.get("timing_mode", launch)
    return cfg


def gpu_clocks():
    """Current shader and memory clock (MHz) of the GPU in use, read from the
    driver's DPM tables in sysfs (the level marked '*'); {} when unreadable."""
    import torch
    try:
        props = torch.cuda.get_device_properties(torch.cuda.current_device())
        bdf = f"{props.pci_domain_id:04x}:{props.pci_bus_id:02x}:{props.pci_device_id:02x}.0"
    except Exception:
        return {}
    clocks = {}
    for key, name in (("sclk_mhz", "pp_dpm_sclk"), ("mclk_mhz", "pp_dpm_mclk")):
        try:
            with open(f"/sys/bus/pci/devices/{bdf}/{name}") as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        clocks[key] = int("".join(ch for ch in line.split(":", 1)[1] if ch.isdigit()))
        except (OSError, ValueError, IndexError):
            pass
    if clocks:
        clocks["pci"] = bdf
    return clocks


def environment():
    import torch
    env = {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip, "torch": torch.__version__}
    try:
        props = torch.cuda.get_device_properties(0)
        env["arch"] = getattr(props, "gcnArchName", "")
        env["cus"] = props.multi_processor_count
    except Exception:
        pass
    env["clocks_after_run"] = gpu_clocks()
    try:
        cpu = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")]
        env["host_cpu"] = cpu[0] if cpu else ""
        env["host_cores_visible"] = len(os.sched_getaffinity(0))
    except Exception:
        pass
    return env


def launch_floor(steps: int, replays: int, launch: str, head) -> dict:
    """Time per launch of a minimal kernel (a 4-byte fill), timed exactly as the
    workload is: the per-call cost no kernel can go below on this system, which
    bounds the measured fraction of peak."""
    import torch
    buf = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(10):
        buf.fill_(0)
    torch.cuda.synchronize()
    timer = Timer(lambda i: buf.fill_(0), 0, steps, 1, launch, head)
    return quantiles([timer.region(r) for r in range(replays)])


def copy_calibration(mb: float):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE
    counters (run under rocprofv3 --pmc)."""
    import torch
    n = int(mb * 2 ** 20)
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copied {n} bytes 5 times")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--replays", type=int, default=0,
                    help="timed replays of the K-step graph (default: enough for 2000 timed steps, at least 5)")
    ap.add_argument("--workload", default="large_decode")
    ap.add_argument("--rotate-mb", type=float, default=1024.0,
                    help="total size of the buffer sets cycled through (beats the 256 MB Infinity Cache)")
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--no-copy-control", action="store_true")
    ap.add_argument("--copy-calibration-mb", type=float, default=0.0)
    ap.add_argument("--only-workload", action="store_true",
                    help="time the workload alone (no copy control, other workloads, CPU baseline, warm-cache "
                         "run or launch floor): for profiling runs")
    ap.add_argument("--keep-copy-control", action="store_true",
                    help="with --only-workload, still time the copy control (a trace then holds both)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the decode "
              "update needs no communication, and a multi-GPU deployment runs one process per GPU on its "
              "own share of the channels.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("--steps must be at least 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import depthwise_causal_conv1d_amd as dc
    from depthwise_causal_conv1d_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dc._load()
    if args.copy_calibration_mb > 0:
        copy_calibration(args.copy_calibration_mb)
        return

    replays = args.replays if args.replays > 0 else min(200, max(5, math.ceil(2000 / args.steps)))
    other_replays = max(5, replays // 2)
    head = Head()
    if args.only_workload:
        args.no_other_workloads = args.no_cpu_baseline = True
        args.no_copy_control = args.no_copy_control or not args.keep_copy_control
    copy = not args.no_copy_control
    spec = wl.BY_NAME[args.workload]
    res, host = measure(spec, args.steps, args.warmup, args.rotate_mb, args.launch, replays, head, copy)
    log(f"[bench] {spec.name}: {res['us_per_call']:.3f} us/call (p10 {res['us_p10']:.3f}, p90 {res['us_p90']:.3f}, "
        f"{res['replays']} replays of {args.steps} steps), {res['gbs']:.1f} GB/s "
        f"({100 * res['frac']:.1f}% of 8 TB/s), {res['rows_per_s'] / 1e6:.2f} M rows/s, kernel {res['kernel']}, "
        f"{res['buffer_sets']} buffer sets, timed {res['timing_mode']}")
    if "copy" in res:
        log(f"[bench] copy control ({res['copy']['bytes_per_call']} B): {res['copy']['us_per_call']:.3f} us/call "
            f"({100 * res['copy']['frac']:.1f}% of 8 TB/s); update at {100 * res['frac_of_copy']:.1f}% of the copy")
    others = []
    if not args.no_other_workloads:
        for other in wl.DECODE_WORKLOADS + wl.EXTRA + wl.PREFILL:
            if other.name == spec.name:
                continue
            # ~0.1 ms prefill calls: fewer steps per replay
            if isinstance(other, wl.PrefillSpec):
                r, _ = measure(other, max(20, args.steps // 5), 5, args.rotate_mb, args.launch, other_replays,
                               head, copy)
            else:
                r, _ = measure(other, args.steps, args.warmup, args.rotate_mb, args.launch, other_replays, head,
                               copy)
            log(f"[bench] {other.name}: {r['us_per_call']:.3f} us/call (p10 {r['us_p10']:.3f}, p90 "
                f"{r['us_p90']:.3f}), {r['gbs']:.1f} GB/s, {r['rows_per_s'] / 1e6:.2f} M rows/s, kernel {r['kernel']}"
                + (f"; copy {r['copy']['us_per_call']:.3f} us, {100 * r['frac_of_copy']:.1f}% of it"
                   if "copy" in r else ""))
            entry = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()
                     if k in ("workload", "kernel", "us_per_call", "us_p10", "us_p90", "gbs", "frac", "rows_per_s",
                              "active_rows_per_s", "bytes_per_call", "tokens_per_call", "frac_of_copy")}
            if "copy" in r:
                entry["copy_us"] = round(r["copy"]["us_per_call"], 4)
            entry["traffic"] = read_traffic(r["kernel"], other.name)
            others.append(entry)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, host, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s on {cpu['cores']} threads ({cpu['sample']}); "
            f"one thread {cpu.get('single_thread', {}).get('value', float('nan')):.3f} GB/s")

    # the same calls on one buffer set, resident in the 256 MB Infinity Cache: a
    # cache figure, reported beside the HBM one and never as a fraction of HBM peak
    # the same workload in 1000-step graph replays: the per-call period of long
    # back-to-back runs, independent of --steps (reported beside the headline,
    # which stays the K-step figure)
    steady = None
    if not args.only_workload and args.steps < 1000:
        steady, _ = measure(spec, 1000, args.warmup, args.rotate_mb, "graph", 5, head)
        log(f"[bench] {spec.name} steady state (1000-step graph replays): {steady['us_per_call']:.3f} us/call, "
            f"{100 * steady['frac']:.1f}% of 8 TB/s")
    warm, floor_us = None, float("nan")
    if not args.only_workload:
        warm, _ = measure(spec, args.steps, args.warmup, 0.0, args.launch, other_replays, head)
        log(f"[bench] {spec.name} warm (one buffer set, Infinity Cache resident): {warm['us_per_call']:.3f} us/call")
        floor_us = launch_floor(args.steps, other_replays, args.launch, head)["median"]
    # under a profiler every launch carries the tracer's own cost, so the floor can
    # reach the call's period; the split is then meaningless
    have_floor = math.isfinite(floor_us)
    if have_floor:
        rest_us = res["us_per_call"] - floor_us
        share = f"{res['bytes_per_call'] / (rest_us * 1e3):.1f} GB/s" if rest_us > 0.1 * res["us_per_call"] else "n/a"
        log(f"[bench] launch floor (empty fill kernel, same launch method): {floor_us:.3f} us/call; "
            f"{spec.name} in-kernel share: {share}")
    traffic = read_traffic(res["kernel"], spec.name)
    line = {
        "metric": METRIC,
        "value": round(res["gbs"], 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": config_of(spec, res, args.launch),
        "rows_per_s": res["rows_per_s"],
        "us_per_call": res["us_per_call"],
        "bytes_per_call": res["bytes_per_call"],
        "kernel": res["kernel"],
        "roofline": {"bound": "hbm", "achieved": round(res["gbs"], 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(res["frac"], 4), "traffic": traffic},
        # every timed region is exactly `steps` steps; ms_per_step is the median over regions
        "timing": {"regions": res["replays"], "steps_per_region": args.steps, "mode": res["timing_mode"],
                   "events": "hipEventDisableSystemFence",
                   "us_per_call": {"p10": round(res["us_p10"], 4), "median": round(res["us_per_call"], 4),
                                   "p90": round(res["us_p90"], 4)}},
        # 1000-step graph replays of the same workload in the same run (context, not the headline)
        "steady_state": None if steady is None else {
            "steps_per_region": 1000, "regions": steady["replays"], "mode": steady["timing_mode"],
            "us_per_call": round(steady["us_per_call"], 4), "gbs": round(steady["gbs"], 1),
            "frac": round(steady["frac"], 4)},
        # the same byte count moved by a plain copy, timed in the same run right after the update
        "copy_control": None if "copy" not in res else {
            **{k: (round(v, 4) if isinstance(v, float) else v) for k, v in res["copy"].items()},
            "frac_of_copy": round(res["frac_of_copy"], 4)},
        # per-call floor of a graph-replayed launch, measured beside the workload: a call of
        # B bytes cannot exceed B / (B / peak + floor), the ceiling the fraction is read against
        "launch_floor_us": round(floor_us, 3) if have_floor else None,
        "warm_cache": None if warm is None else {
            "us_per_call": round(warm["us_per_call"], 4), "gbs": round(warm["gbs"], 1),
            "buffer_sets": warm["buffer_sets"], "note": "Infinity Cache resident, not an HBM figure"},
        "frac_ceiling_at_floor": round(res["bytes_per_call"] / (res["bytes_per_call"] / (PEAK_HBM_GBS * 1e3)
                                                                + floor_us) / (PEAK_HBM_GBS * 1e3), 4)
        if have_floor else None,
        "cpu_baseline": cpu,
        "other_workloads": others,
        "env": environment(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
