"""The benchmark's workloads at full size, launched the way bench.py times them.

Each workload's own buffer-set rotation (bench.Workload / bench.PrefillWorkload)
is captured in one HIP graph of two passes over its sets and replayed; then every
set's outputs and state are compared with the oracle applied twice to the same
initial data (state bit-exact, outputs within one BF16 ulp or the relative bound).
"""
import numpy as np
import pytest
import torch

import bench
import oracle
from depthwise_causal_conv1d_amd import workloads as wl
from parity import assert_outputs_match

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _host(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _two_sets(cls, spec, dev):
    """The workload with exactly two buffer sets (the rotation size is chosen from
    one set's bytes)."""
    one = cls(spec, 1.0, dev)
    set_bytes = one.set_bytes
    del one
    torch.cuda.empty_cache()
    wk = cls(spec, 1.5 * set_bytes, dev)
    assert wk.n_sets == 2
    return wk


def _replay_two_passes(wk):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(2 * wk.n_sets):
            wk.step(i)
    g.replay()
    torch.cuda.synchronize()


DECODE = ["large_decode", "large_decode_channel_last", "large_decode_ring", "large_decode_4tok",
          "long_history_one_call", "large_decode_ring_4tok"]


def _decode_reference(spec, data, state):
    """One call of the workload on host arrays; ``state`` is updated in place."""
    N, D, L, S, ld = spec.N, spec.D, spec.L, spec.S, spec.ld
    strides = wl.state_strides(spec)
    x = data["x"]  # [T, N, ld]
    if spec.one_call and spec.ring:
        outs, outs32 = [], []
        for t in range(spec.T):
            o, o32 = oracle.update_ring(np.ascontiguousarray(x[t]), N, D, ld, state, S, L, strides,
                                        data["weight"], data["bias"], data["indices"],
                                        (data["seqlens"] + t).astype(np.int32), spec.act, want_f32=True)
            outs.append(o)
            outs32.append(o32)
        return np.stack(outs, 1), np.stack(outs32, 1)
    if spec.one_call:
        return oracle.update_tokens(x, N, D, spec.T, (ld, 1, N * ld), state, S, L, strides, data["weight"],
                                    data["bias"], data["indices"], spec.act, want_f32=True)
    if spec.ring:
        o, o32 = oracle.update_ring(np.ascontiguousarray(x[0]), N, D, ld, state, S, L, strides, data["weight"],
                                    data["bias"], data["indices"], data["seqlens"], spec.act, want_f32=True)
    else:
        o, o32 = oracle.update_strided(np.ascontiguousarray(x[0]), N, D, ld, state, S, L, strides, data["weight"],
                                       data["bias"], data["indices"], spec.act, want_f32=True)
    return o[:, None, :], o32[:, None, :]


@pytest.mark.parametrize("name", DECODE)
def test_decode_workload_graph_replay(name):
    spec = wl.BY_NAME[name]
    dev = torch.device("cuda", torch.cuda.current_device())
    wk = _two_sets(bench.Workload, spec, dev)
    print(f"[{name}] {wk.n_sets} sets of {wk.set_bytes / 2**20:.1f} MiB", flush=True)
    _replay_two_passes(wk)
    data = wk.host
    state = data["state"].copy()
    _decode_reference(spec, data, state)
    ref, ref32 = _decode_reference(spec, data, state)
    for k, s in enumerate(wk.sets):
        phys = s["state"] if spec.layout == "compact" else s["state"].permute(0, 2, 1)
        np.testing.assert_array_equal(_host(phys), state, err_msg=f"{name} set {k}: state")
        assert_outputs_match(_host(s["out"]), ref, ref32, what=f"{name} set {k}")


@pytest.mark.parametrize("name", ["prefill_batch", "prefill_varlen"])
def test_prefill_workload_graph_replay(name):
    spec = wl.PREFILL[[p.name for p in wl.PREFILL].index(name)]
    dev = torch.device("cuda", torch.cuda.current_device())
    wk = _two_sets(bench.PrefillWorkload, spec, dev)
    print(f"[{name}] {wk.n_sets} sets of {wk.set_bytes / 2**20:.1f} MiB", flush=True)
    _replay_two_passes(wk)
    data = wk.host
    packed = data["starts"] is not None
    D = spec.D
    n = spec.N
    t, xs = (data["total"], (0, 1, D)) if packed else (spec.T, (spec.T * D, 1, D))
    st_strides = (spec.L * D, 1, D) if spec.layout == "channel_last" else (D * spec.L, spec.L, 1)
    state = data["state"].copy()
    for _ in range(2):
        ref, ref32 = oracle.prefill(data["x"], n, D, t, xs, data["weight"], data["bias"], spec.act,
                                    starts=data["starts"], state_buf=state, S=spec.S, L=spec.L,
                                    state_strides=st_strides, indices=data["indices"], has_init=data["has_init"],
                                    want_f32=True)
    for k, s in enumerate(wk.sets):
        phys = s["state"] if spec.layout == "compact" else s["state"].permute(0, 2, 1)
        np.testing.assert_array_equal(_host(phys), state, err_msg=f"{name} set {k}: state")
        out = s["out"].permute(0, 2, 1)  # back to the token-major buffer
        got = _host(out).reshape(ref.shape)
        assert_outputs_match(got, ref, ref32, what=f"{name} set {k}")
