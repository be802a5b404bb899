"""Host-side logic of the benchmark: the algorithmic byte count that the
roofline fraction divides by, the workload generator's shapes, the single-GPU
refusal and the CPU-baseline leg (runs the oracle; no GPU needed)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from depthwise_causal_conv1d_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_large_decode_bytes_by_hand():
    # x 256*8192*2, state read 3 positions and written 3, weight 8192*4*2, out 256*8192*2
    N, D = 256, 8192
    hand = 2 * N * D + 2 * N * D * 3 + 2 * N * D * 3 + 2 * D * 4 + 2 * N * D
    assert hand == 33619968
    assert wl.algorithmic_bytes(N, D, 4, 3, N, False, False) == hand


def test_bytes_count_padding_rows_bias_and_indices():
    N, D, L = 64, 4096, 3
    full = wl.algorithmic_bytes(N, D, 4, L, N, False, False)
    part = wl.algorithmic_bytes(N, D, 4, L, 56, True, True)
    # 8 padding rows skip x, state read and state write; bias and index table added
    assert full - part == 8 * (2 * D + 2 * D * L * 2) - 2 * D - 4 * N


@pytest.mark.parametrize("L,T,planes", [(3, 1, 3), (3, 7, 3), (4, 1, 3), (8, 1, 7), (8, 3, 5), (8, 5, 3),
                                        (8, 16, 3)])
def test_channel_last_reads_only_needed_planes(L, T, planes):
    N, D = 2, 64
    b = wl.algorithmic_bytes(N, D, 4, L, N, False, False, "channel_last", T)
    assert b == 2 * N * D * T + 2 * N * D * planes + 2 * N * D * L + 2 * D * 4 + 2 * N * D * T


def test_tokens_scale_x_and_out_but_not_state():
    N, D, L = 128, 4096, 8
    one = wl.algorithmic_bytes(N, D, 4, L, N, True, True, "compact", 1)
    sixteen = wl.algorithmic_bytes(N, D, 4, L, N, True, True, "compact", 16)
    assert sixteen - one == 15 * (2 * N * D + 2 * N * D)


def test_workload_shapes_and_padding():
    for spec in wl.DECODE_WORKLOADS + wl.EXTRA:
        if spec.N * spec.D * spec.T > 4_000_000:
            continue
        d = wl.make(spec)
        assert d["x"].shape == (spec.T, spec.N, spec.ld)
        assert np.all(d["x"][:, :, spec.D:] == wl.PAD_SENTINEL)
        assert d["weight"].shape == (spec.D, spec.W)
        shape = (spec.S, spec.D, spec.L) if spec.layout == "compact" else (spec.S, spec.L, spec.D)
        assert d["state"].shape == shape
        if d["indices"] is not None:
            real = d["indices"][d["indices"] >= 0]
            assert len(set(real.tolist())) == len(real) and real.max() < spec.S


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


@pytest.mark.parametrize("name", ["tiny", "long_history_one_call"])
def test_cpu_baseline_leg(name):
    spec = wl.BY_NAME[name]
    res = bench.cpu_baseline(spec, wl.make(spec), seconds=0.0)
    assert res["kind"] == "oracle" and res["cores"] >= 1 and res["unit"] == "GB/s" and res["value"] > 0
    one = res["single_thread"]
    assert one["cores"] == 1 and one["value"] > 0
    json.dumps(res)


_SPLIT_CASES = [
    wl.Spec("split_plain", N=13, D=64, W=4, L=3, S=15, ld=72, bias=False, act="silu", routing="none", seed=7),
    wl.Spec("split_padded", N=16, D=40, W=4, L=4, S=64, ld=40, bias=True, act=None, routing="padded", n_unique=11,
            seed=8),
    wl.Spec("split_tokens", N=9, D=32, W=4, L=5, S=20, ld=32, bias=True, act="silu", routing="unique", T=6,
            seed=9, one_call=True),
    wl.Spec("split_ring", N=10, D=48, W=4, L=3, S=10, ld=48, bias=False, act="silu", routing="none",
            layout="channel_last", ring=True, T=3, one_call=True, seed=10),
    wl.Spec("split_channel_last", N=7, D=24, W=4, L=6, S=9, ld=24, bias=True, act=None, routing="none",
            layout="channel_last", seed=11),
]


@pytest.mark.parametrize("spec", _SPLIT_CASES, ids=lambda s: s.name)
def test_cpu_baseline_row_split_matches_one_call(spec):
    # the all-cores leg runs disjoint row ranges as separate oracle calls; the
    # state they leave must be the one a single whole-batch call leaves
    host = wl.make(spec)
    whole = host["state"].copy()
    bench._oracle_rows(spec, host, whole, 0, spec.N)
    split = host["state"].copy()
    for a, b in ((0, 3), (3, 4), (4, spec.N)):
        bench._oracle_rows(spec, host, split, a, b)
    assert np.array_equal(whole, split)
    assert not np.array_equal(whole, host["state"])


def test_prefill_bytes_by_hand():
    # 8 sequences x 2048 tokens x 8192 channels: x read and out written once,
    # the channel-last L=3 final states written, the weight read; no initial state
    spec = wl.BY_NAME["prefill_batch"]
    tok = 8 * 2048
    assert wl.prefill_algorithmic_bytes(spec, None) == 4 * tok * 8192 + 8 * 2 * 8192 * 3 + 2 * 8192 * 4


def test_prefill_bytes_count_initial_state_reads():
    spec = wl.PrefillSpec("p", N=3, D=64, W=4, L=8, lens=(1, 4, 20), S=3, layout="channel_last", routing="unique")
    none = wl.prefill_algorithmic_bytes(spec, np.zeros(3, np.uint8))
    some = wl.prefill_algorithmic_bytes(spec, np.array([1, 1, 1], np.uint8))
    # planes still needed: L - min(T_i, L - 3) = 7, 4, 3
    assert some - none == 2 * 64 * (7 + 4 + 3)


def test_prefill_workload_shapes():
    for spec in wl.PREFILL:
        d = wl.make_prefill(spec)
        lens = spec.lens if spec.lens is not None else [spec.T] * spec.N
        assert d["total"] == sum(lens)
        assert d["x"].reshape(-1, spec.D).shape == (sum(lens), spec.D)
        if d["starts"] is not None:
            assert d["starts"][0] == 0 and d["starts"][-1] == d["total"] and np.all(np.diff(d["starts"]) >= 0)


def test_cpu_baseline_prefill_leg():
    spec = wl.BY_NAME["prefill_varlen"]
    res = bench.cpu_baseline(spec, wl.make_prefill(spec), seconds=0.0)
    assert res["kind"] == "oracle" and res["value"] > 0 and "sequences" in res["sample"]


def test_ring_bytes_by_hand():
    # large decode batch on a ring: x, 3 newest values read, 1 written, out, weight, counts
    N, D = 256, 8192
    hand = 2 * N * D + 2 * N * D * 3 + 2 * N * D + 2 * N * D + 2 * D * 4 + 4 * N
    assert wl.algorithmic_bytes(N, D, 4, 3, N, False, False, "channel_last", 1, ring=True) == hand


def test_cpu_baseline_ring_leg():
    spec = wl.BY_NAME["large_decode_ring"]
    small = wl.Spec("ring_small", N=8, D=64, W=4, L=3, S=8, ld=64, bias=False, act="silu", routing="none",
                    layout="channel_last", ring=True, seed=4)
    res = bench.cpu_baseline(small, wl.make(small), seconds=0.0)
    assert res["value"] > 0 and spec.ring


def test_ring_tokens_bytes_by_hand():
    N, D, T, L = 256, 8192, 4, 3
    hand = 2 * N * D * T + 2 * N * D * 3 + 2 * N * D * min(T, L) + 2 * N * D * T + 2 * D * 4 + 4 * N
    assert wl.algorithmic_bytes(N, D, 4, L, N, False, False, "channel_last", T, ring=True) == hand


def test_kernel_hash_ignores_comments_but_not_code():
    """A comment edit keeps a counter summary current; a code edit makes it stale."""
    import bench
    code = "int f(int a) {  // adds one\n    /* the\n  sum */ return a + 1;\n}\n"
    assert bench._code_only(code) == bench._code_only(code.replace("adds one", "increments"))
    assert bench._code_only(code) == bench._code_only("int f(int a) {\n\n    return a + 1;\n}\n")
    assert bench._code_only(code) != bench._code_only(code.replace("a + 1", "a + 2"))


def test_timing_mode_direct_up_to_32_steps_then_graphs():
    # short regions go straight to the stream behind the head; longer ones are
    # graph replays; an explicit eager request is kept at any length
    assert bench.timing_mode("graph", 1, True) == "eager+head"
    assert bench.timing_mode("graph", 20, True) == "eager+head"
    assert bench.timing_mode("graph", bench.EAGER_MAX_STEPS, True) == "eager+head"
    assert bench.timing_mode("graph", bench.EAGER_MAX_STEPS + 1, True) == "graph"
    assert bench.timing_mode("graph", 1000, True) == "graph"
    assert bench.timing_mode("graph", 20, False) == "graph"
    assert bench.timing_mode("eager", 1000, True) == "eager"
