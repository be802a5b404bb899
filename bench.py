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

The timed region is K steps captured in one HIP graph and replayed once,
bracketed by synchronisations and timed with HIP events on the stream that
launches the kernels.  Achieved bandwidth is the algorithmic byte count of a call
(x + selected state read + state write + weight + bias + output + index table)
divided by the measured time per step.

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


def measure(spec, steps: int, warmup: int, rotate_mb: float, launch: str):
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
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if launch == "graph":
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                wk.step(warmup + i)
        g.replay()  # one untimed replay: graph upload
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        g.replay()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(steps):
            wk.step(warmup + i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    res = dict(workload=spec.name, kernel=kernel, ms_per_step=ms, us_per_call=ms * 1e3,
               wall_ms_per_step=wall * 1e3 / steps, bytes_per_call=wk.bytes_per_call,
               gbs=wk.bytes_per_call / (ms * 1e-3) / 1e9,
               rows_per_s=getattr(wk, "rows", spec.N * wk.tokens) / (ms * 1e-3),
               tokens_per_call=wk.tokens,
               buffer_sets=wk.n_sets, set_bytes=wk.set_bytes)
    res["frac"] = res["gbs"] / PEAK_HBM_GBS
    if getattr(wk, "active", spec.N) != spec.N:
        res["active_rows_per_s"] = wk.active * wk.tokens / (ms * 1e-3)
    host = wk.host
    del wk
    torch.cuda.empty_cache()
    return res, host


def cpu_baseline(spec, host, seconds: float):
    """The oracle as it stands (single thread, plain C) on the same workload."""
    import numpy as np
    import oracle
    from depthwise_causal_conv1d_amd import workloads as wl

    if isinstance(spec, wl.PrefillSpec):
        return cpu_baseline_prefill(spec, host, seconds)
    tokens = spec.T if spec.one_call else 1
    x = np.ascontiguousarray(host["x"][0]) if tokens == 1 else np.ascontiguousarray(host["x"])
    reps, t_total = 0, 0.0
    while reps < 2 or t_total < seconds:
        st = host["state"].copy()
        t0 = time.perf_counter()
        if spec.ring:
            for t in range(tokens):  # a multi-token ring call is its tokens' ring steps in order
                xt = np.ascontiguousarray(host["x"][t])
                oracle.update_ring(xt, spec.N, spec.D, spec.ld, st, spec.S, spec.L, wl.state_strides(spec),
                                   host["weight"], host["bias"], host["indices"], host["seqlens"] + t, spec.act)
        elif tokens == 1:
            oracle.update_strided(x, spec.N, spec.D, spec.ld, st, spec.S, spec.L, wl.state_strides(spec),
                                  host["weight"], host["bias"], host["indices"], spec.act)
        else:
            oracle.update_tokens(x, spec.N, spec.D, tokens, (spec.ld, 1, spec.N * spec.ld), st, spec.S, spec.L,
                                 wl.state_strides(spec), host["weight"], host["bias"], host["indices"], spec.act)
        t_total += time.perf_counter() - t0
        reps += 1
    active = spec.N if host["indices"] is None else int((host["indices"] >= 0).sum())
    b = wl.algorithmic_bytes(spec.N, spec.D, spec.W, spec.L, active, host["bias"] is not None,
                             host["indices"] is not None, spec.layout, tokens, spec.ring)
    per_call = t_total / reps
    return {"value": b / per_call / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full {spec.name} calls (N={spec.N}, D={spec.D}, L={spec.L}, {tokens} token(s)) "
                      f"on host arrays, single thread, {per_call * 1e3:.1f} ms per call",
            "rows_per_s": spec.N * tokens / per_call}


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
    cfg["launch"] = "hipgraph" if launch == "graph" else "eager"
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


def launch_floor(steps: int = 1000) -> float:
    """Time per launch of a minimal kernel (a 4-byte fill) replayed from one HIP
    graph, the same way the workload is timed: the per-call cost no kernel can go
    below on this system, which bounds the measured fraction of peak."""
    import torch
    buf = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(10):
        buf.fill_(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            buf.fill_(0)
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    g.replay()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps * 1e3


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
    ap.add_argument("--workload", default="large_decode")
    ap.add_argument("--rotate-mb", type=float, default=1024.0,
                    help="total size of the buffer sets cycled through (beats the 256 MB Infinity Cache)")
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true")
    ap.add_argument("--copy-calibration-mb", type=float, default=0.0)
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}): the decode "
              "update needs no communication, and a multi-GPU deployment runs one process per GPU on its "
              "own share of the channels.", file=sys.stderr)
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

    spec = wl.BY_NAME[args.workload]
    res, host = measure(spec, args.steps, args.warmup, args.rotate_mb, args.launch)
    log(f"[bench] {spec.name}: {res['us_per_call']:.3f} us/call, {res['gbs']:.1f} GB/s "
        f"({100 * res['frac']:.1f}% of 8 TB/s), {res['rows_per_s'] / 1e6:.2f} M rows/s, kernel {res['kernel']}, "
        f"{res['buffer_sets']} buffer sets, wall {res['wall_ms_per_step'] * 1e3:.3f} us/step")
    others = []
    if not args.no_other_workloads:
        for other in wl.DECODE_WORKLOADS + wl.EXTRA + wl.PREFILL:
            if other.name == spec.name:
                continue
            # as many steps as the main workload (a replay of a few hundred steps still
            # carries a fixed start-up cost of about 0.25 ms), fewer for ~0.1 ms prefill calls
            if isinstance(other, wl.PrefillSpec):
                r, _ = measure(other, max(100, args.steps // 5), 5, args.rotate_mb, args.launch)
            else:
                r, _ = measure(other, args.steps, args.warmup, args.rotate_mb, args.launch)
            log(f"[bench] {other.name}: {r['us_per_call']:.3f} us/call, {r['gbs']:.1f} GB/s, "
                f"{r['rows_per_s'] / 1e6:.2f} M rows/s, kernel {r['kernel']}")
            entry = {k: (round(v, 4) if isinstance(v, float) else v) for k, v in r.items()
                     if k in ("workload", "kernel", "us_per_call", "gbs", "frac", "rows_per_s",
                              "active_rows_per_s", "bytes_per_call", "tokens_per_call")}
            entry["traffic"] = read_traffic(r["kernel"], other.name)
            others.append(entry)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(spec, host, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s ({cpu['sample']})")

    # the same calls on one buffer set, resident in the 256 MB Infinity Cache: a
    # cache figure, reported beside the HBM one and never as a fraction of HBM peak
    warm, _ = measure(spec, args.steps, args.warmup, 0.0, args.launch)
    log(f"[bench] {spec.name} warm (one buffer set, Infinity Cache resident): {warm['us_per_call']:.3f} us/call")
    floor_us = launch_floor()
    # under a profiler every launch carries the tracer's own cost, so the floor can
    # reach the call's period; the split is then meaningless
    rest_us = res["us_per_call"] - floor_us
    share = f"{res['bytes_per_call'] / (rest_us * 1e3):.1f} GB/s" if rest_us > 0.1 * res["us_per_call"] else "n/a"
    log(f"[bench] launch floor (empty fill kernel, graph replay): {floor_us:.3f} us/call; "
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
        # per-call floor of a graph-replayed launch, measured beside the workload: a call of
        # B bytes cannot exceed B / (B / peak + floor), the ceiling the fraction is read against
        "launch_floor_us": round(floor_us, 3),
        "warm_cache": {"us_per_call": round(warm["us_per_call"], 4), "gbs": round(warm["gbs"], 1),
                       "buffer_sets": warm["buffer_sets"], "note": "Infinity Cache resident, not an HBM figure"},
        "frac_ceiling_at_floor": round(res["bytes_per_call"] / (res["bytes_per_call"] / (PEAK_HBM_GBS * 1e3)
                                                                + floor_us) / (PEAK_HBM_GBS * 1e3), 4),
        "cpu_baseline": cpu,
        "other_workloads": others,
        "env": environment(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
