"""Seeded random sweep of every entry point against the CPU oracle.

The targeted GPU tests pick shapes by hand; this sweep draws them: for each case
number a seeded generator picks the rows, channels (multiples of 8 and not),
history length, state layout, x row stride or token layout, bias, activation,
routing (none, a unique table, a table with padding rows), for the ring forms the
token counts and, for the prefill,
batch or packed sequences (some empty) with or without initial state.  Every
case goes through the C ABI and is held to the usual bar: whole state buffer
bit-exact with guard bands intact, x unwritten, padding rows zero, outputs
within 1 BF16 ulp or 1e-2 * max(1, |ref|) of the FP32 oracle (exact for
identity).  The draw is printed before each case runs, so a failure names it.

Semantics: cuDNN FE-OSS page "Causal Conv1d Decode Update", sections "Causal
Conv1d Decode Update" (update rule, routing, padding, cache_seqlens) and
"Semantic tensor contract" (layouts, row stride, the multi-token form); the
prefill is the whole-sequence form the page names at its top.
"""
import numpy as np
import pytest
import torch

import depthwise_causal_conv1d_amd as dc
from depthwise_causal_conv1d_amd import workloads as wl
from test_gpu_prefill import PrefillCase
from parity import assert_guards_intact, assert_outputs_match, from_dev, guarded_copy, guarded_empty, to_dev
from test_gpu_ring import RingCase, _ring_tokens_reference
from test_gpu_tokens import TokensCase
from test_gpu_update import make_case

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dc._load()
    yield


def _channels(rng, hi):
    """Mostly multiples of 8 (the vector kernels), sometimes not (the scalar ones)."""
    return 8 * int(rng.integers(1, hi // 8 + 1)) if rng.random() < 0.75 else int(rng.integers(1, hi + 1))


def _routing(rng, n, S):
    """(routing, n_pad) valid for n rows over S >= n slots."""
    kind = ["none", "unique", "padded"][int(rng.integers(0, 3))]
    n_pad = int(rng.integers(1, n + 1)) if kind == "padded" else 0
    return kind, n_pad


def _act(rng):
    return [None, "silu"][int(rng.integers(0, 2))]


def _show(kind, k, **cfg):
    print(f"{kind} case {k}: {cfg}", flush=True)


@pytest.mark.parametrize("k", range(100))
def test_update_random(k):
    rng = np.random.default_rng(91000 + k)
    D = _channels(rng, 1500)
    N = int(rng.integers(1, 200))
    L = int(rng.integers(3, 10))
    ld = D if rng.random() < 0.5 else (D + 7) // 8 * 8 + 8 * int(rng.integers(0, 4))
    ld = D if ld == D or ld % 8 else ld
    S = N + int(rng.integers(0, 20))
    routing, n_pad = _routing(rng, N, S)
    cfg = dict(N=N, D=D, L=L, S=S, ld=ld, layout=["compact", "channel_last"][int(rng.integers(0, 2))],
               bias=bool(rng.random() < 0.5), routing=routing, n_pad=n_pad, act=_act(rng),
               status=bool(rng.random() < 0.5))
    _show("update", k, **cfg)
    status = make_case(92000 + k, **cfg).check()
    assert status in (None, 0)


@pytest.mark.parametrize("k", range(100))
def test_tokens_random(k):
    rng = np.random.default_rng(93000 + k)
    D = _channels(rng, 1200)
    N = int(rng.integers(1, 64))
    T = int(rng.integers(1, 41))
    L = int(rng.integers(3, 10))
    S = N + int(rng.integers(0, 10))
    routing, n_pad = _routing(rng, N, S)
    x_layout = ["token_major", "step_major", "channel_major"][int(rng.integers(0, 3))]
    ldx = D + (0 if rng.random() < 0.5 else int(rng.integers(0, 17)))
    cfg = dict(N=N, D=D, T=T, L=L, S=S, layout=["compact", "channel_last"][int(rng.integers(0, 2))],
               x_layout=x_layout, ldx=ldx, out_layout=["token_major", "channel_major"][int(rng.integers(0, 2))],
               bias=bool(rng.random() < 0.5), act=_act(rng), routing=routing, n_pad=n_pad,
               status=bool(rng.random() < 0.5))
    _show("tokens", k, **cfg)
    status = TokensCase(94000 + k, **cfg).check()
    assert status in (None, 0)


@pytest.mark.parametrize("k", range(60))
def test_ring_random(k):
    rng = np.random.default_rng(95000 + k)
    D = _channels(rng, 1500)
    N = int(rng.integers(1, 200))
    L = int(rng.integers(3, 10))
    ld = D if rng.random() < 0.5 else (D + 7) // 8 * 8 + 8 * int(rng.integers(0, 4))
    ld = D if ld == D or ld % 8 else ld
    S = N + int(rng.integers(0, 20))
    routing, n_pad = _routing(rng, N, S)
    cfg = dict(S=S, ld=ld, layout=["compact", "channel_last"][int(rng.integers(0, 2))],
               bias=bool(rng.random() < 0.5), act=_act(rng), routing=routing, n_pad=n_pad,
               max_seen=int(rng.integers(0, 5000)), status=bool(rng.random() < 0.5))
    _show("ring", k, N=N, D=D, L=L, **cfg)
    status = RingCase(96000 + k, N, D, L, **cfg).check()
    assert status in (None, 0)


@pytest.mark.parametrize("k", range(100))
def test_prefill_random(k):
    rng = np.random.default_rng(97000 + k)
    D = _channels(rng, 2048)
    packed = bool(rng.random() < 0.5)
    if packed:
        n = int(rng.integers(1, 20))
        lens = [int(v) for v in rng.integers(0, 200, size=n)]
        shape = dict(lens=lens)
    else:
        n = int(rng.integers(1, 8))
        shape = dict(N=n, T=int(rng.integers(1, 300)))
    state = [None, "compact", "channel_last"][int(rng.integers(0, 3))]
    L = int(rng.integers(3, 10))
    S = n + int(rng.integers(0, 10))
    routing, n_pad = _routing(rng, n, S) if state is not None else ("none", 0)
    cfg = dict(L=L, state=state, S=S, routing=routing, n_pad=n_pad,
               has_init=["none", "all", "mixed"][int(rng.integers(0, 3))], bias=bool(rng.random() < 0.5),
               act=_act(rng), x_layout=["token_major", "channel_major"][int(rng.integers(0, 2))],
               out_layout=["token_major", "channel_major"][int(rng.integers(0, 2))],
               status=bool(rng.random() < 0.5))
    _show("prefill", k, D=D, **shape, **cfg)
    status = PrefillCase(98000 + k, D, **shape, **cfg).check()
    assert status in (None, 0)


@pytest.mark.parametrize("k", range(12))
def test_prefill_random_wide(k):
    """Wider prefill draws (up to 4096 channels and about 12 M elements): the
    sweep form's grid then holds fewer blocks than there are items, so blocks
    take several items in turn, and long packed sequences span many items."""
    rng = np.random.default_rng(99000 + k)
    D = 8 * int(rng.integers(256, 4096 // 8 + 1))
    cap = 12_000_000 // D
    packed = bool(rng.random() < 0.5)
    if packed:
        n = int(rng.integers(1, 24))
        lens = [int(v) for v in rng.integers(0, max(2, 2 * cap // n), size=n)]
        shape = dict(lens=lens)
    else:
        n = int(rng.integers(1, 12))
        shape = dict(N=n, T=int(rng.integers(cap // (2 * n) + 1, cap // n + 2)))
    state = [None, "compact", "channel_last"][int(rng.integers(0, 3))]
    L = int(rng.integers(3, 9))
    S = n + int(rng.integers(0, 10))
    routing, n_pad = _routing(rng, n, S) if state is not None else ("none", 0)
    cfg = dict(L=L, state=state, S=S, routing=routing, n_pad=n_pad,
               has_init=["none", "all", "mixed"][int(rng.integers(0, 3))], bias=bool(rng.random() < 0.5),
               act=_act(rng), status=bool(rng.random() < 0.5))
    _show("prefill-wide", k, D=D, **({"n": n, "tokens": sum(lens)} if packed else shape), **cfg)
    case = PrefillCase(99500 + k, D, **shape, **cfg)
    assert case.check() in (None, 0)
    assert case.kernel.startswith("prefill_sweep_v8<"), case.kernel


@pytest.mark.parametrize("k", range(40))
def test_ring_tokens_random(k):
    rng = np.random.default_rng(99000 + k)
    D = _channels(rng, 1200)
    N = int(rng.integers(1, 64))
    T = int(rng.integers(1, 25))
    L = int(rng.integers(3, 10))
    S = N + int(rng.integers(0, 10))
    routing, n_pad = _routing(rng, N, S)
    layout = ["compact", "channel_last"][int(rng.integers(0, 2))]
    act, bias = _act(rng), bool(rng.random() < 0.5)
    _show("ring tokens", k, N=N, D=D, T=T, L=L, S=S, layout=layout, routing=routing, n_pad=n_pad, act=act,
          bias=bias)
    bf = lambda shape, scale=1.0: wl.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)
                                                       * np.float32(scale))
    x, w, st = bf((N, T, D)), bf((D, 4)), bf((S, D, L))           # st: compact values
    b = bf((D,), 0.1) if bias else None
    idx = None
    if routing == "unique":
        idx = rng.choice(S, N, replace=False).astype(np.int32)
    elif routing == "padded":
        real = rng.choice(S, N - n_pad, replace=False).astype(np.int32)
        idx = np.concatenate([real, np.full(n_pad, -1, np.int32)])[rng.permutation(N)].astype(np.int32)
    seen = rng.integers(0, 3000, size=N).astype(np.int32)
    ref_state = st.copy()
    ref, ref32 = _ring_tokens_reference(x, ref_state, w, b, idx, seen, act)
    phys = st if layout == "compact" else np.ascontiguousarray(st.transpose(0, 2, 1))
    sb, sd = guarded_copy(phys)
    sv = sd if layout == "compact" else sd.permute(0, 2, 1)
    ob, od = guarded_empty((N * T * D,))
    out = torch.as_strided(od, (N, D, T), (T * D, 1, D))
    dc.causal_conv1d_update_tokens(to_dev(x).permute(0, 2, 1), sv, to_dev(w), None if b is None else to_dev(b), act,
                                   conv_state_indices=None if idx is None else torch.from_numpy(idx).cuda(),
                                   cache_seqlens=torch.from_numpy(seen).cuda(), out=out)
    torch.cuda.synchronize()
    assert_guards_intact(sb)
    assert_guards_intact(ob)
    got_state = from_dev(sd)
    if layout == "channel_last":
        got_state = got_state.transpose(0, 2, 1)
    np.testing.assert_array_equal(got_state, ref_state, err_msg="ring not bit-exact")
    got = from_dev(out.permute(0, 2, 1))
    assert_outputs_match(got, ref, ref32, exact=act is None)
    if idx is not None:
        assert np.all(got[idx == -1] == 0), "padding row not zero"
