"""GPU parity of the full-sequence causal convolution (prefill) against the oracle.

The prefill is the operation the cuDNN FE-OSS page "Causal Conv1d Decode Update"
names at its top for whole sequences; its final state is what the decode update
continues (section "Semantic tensor contract": an L=3 state from the prefill is
accepted in place).  Every case runs the HIP library and the CPU oracle on the
same seeded inputs and requires: the whole state buffer bit-exact (final states
of live sequences, every other slot untouched, guard bands intact), x unwritten,
padding sequences zero, and outputs within 1 BF16 ulp or 1e-2 * max(1, |ref|) of
the FP32 oracle (exact for the identity activation).
"""
import numpy as np
import pytest
import torch

import oracle
import depthwise_causal_conv1d_amd as dc
from depthwise_causal_conv1d_amd import workloads as wl
from parity import (GUARD, assert_guards_intact, assert_outputs_match, from_dev, guarded_copy, guarded_empty,
                    to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dc._load()
    yield


def _bf(rng, shape, scale=1.0):
    return wl.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


class PrefillCase:
    """lens=None: batch form of N sequences of T tokens; else packed sequences."""

    def __init__(self, seed, D, *, N=1, T=1, lens=None, L=3, state="compact", S=None, routing="none", n_pad=0,
                 has_init="mixed", bias=False, act="silu", x_layout="token_major", out_layout="token_major",
                 status=False):
        rng = np.random.default_rng(seed)
        self.D, self.L, self.act, self.status, self.state_kind = D, L, act, status, state
        self.packed = lens is not None
        if self.packed:
            self.n = len(lens)
            self.starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            self.B, self.T = 1, int(self.starts[-1])
        else:
            self.n, self.B, self.T, self.starts = N, N, T, None
        B, T = self.B, self.T
        xt = _bf(rng, (B, T, D))                                       # token-major values
        if x_layout == "token_major":
            self.x, xs = np.ascontiguousarray(xt), (T * D, 1, D)
        else:
            self.x, xs = np.ascontiguousarray(xt.transpose(0, 2, 1)), (D * T, T, 1)
        self.xs = xs
        self.out_layout = out_layout
        self.weight = _bf(rng, (D, 4))
        self.bias = _bf(rng, (D,), 0.1) if bias else None
        n = self.n
        self.S = (n if S is None else S) if state is not None else 0
        if state == "compact":
            self.state0, self.st = _bf(rng, (self.S, D, L)), (D * L, L, 1)
        elif state == "channel_last":
            self.state0, self.st = _bf(rng, (self.S, L, D)), (L * D, 1, D)
        else:
            self.state0, self.st = None, (0, 0, 0)
        self.indices = None
        if routing == "unique":
            self.indices = rng.choice(self.S, n, replace=False).astype(np.int32)
        elif routing == "padded":
            real = rng.choice(self.S, n - n_pad, replace=False).astype(np.int32)
            self.indices = np.concatenate([real, np.full(n_pad, -1, np.int32)])[rng.permutation(n)].astype(np.int32)
        self.oracle_indices = self.indices
        if state is None or has_init == "none":
            self.has_init = None
        elif has_init == "all":
            self.has_init = np.ones(n, np.uint8)
        else:
            self.has_init = (rng.random(n) < 0.6).astype(np.uint8)

    def reference(self):
        st = None if self.state0 is None else self.state0.copy()
        xs = (0, self.xs[1], self.xs[2]) if self.packed else self.xs
        out, out32 = oracle.prefill(self.x, self.n, self.D, self.T, xs, self.weight, self.bias, self.act,
                                    starts=self.starts, state_buf=st, S=self.S, L=self.L if st is not None else 0,
                                    state_strides=self.st, indices=self.oracle_indices, has_init=self.has_init,
                                    want_f32=True)
        return out.reshape(self.B, self.T, self.D), out32.reshape(self.B, self.T, self.D), st

    def run_gpu(self, dev="cuda"):
        B, D, T = self.B, self.D, self.T
        xb, xd = guarded_copy(self.x, dev)
        xv = torch.as_strided(xd.reshape(-1), (B, D, T), self.xs)
        sb = sv = None
        if self.state0 is not None:
            sb, sd = guarded_copy(self.state0, dev)
            sv = sd if self.state_kind == "compact" else sd.permute(0, 2, 1)
        ob, od = guarded_empty((B * T * D,), dev)
        ostr = (T * D, 1, D) if self.out_layout == "token_major" else (D * T, T, 1)
        ov = torch.as_strided(od, (B, D, T), ostr)
        wd = to_dev(self.weight, dev)
        bd = None if self.bias is None else to_dev(self.bias, dev)
        idd = None if self.indices is None else torch.from_numpy(self.indices).to(dev)
        hid = None if self.has_init is None else torch.from_numpy(self.has_init).to(dev)
        ssd = None if self.starts is None else torch.from_numpy(self.starts).to(dev)
        stat = torch.zeros(1, dtype=torch.int32, device=dev) if self.status else None
        ret = dc.causal_conv1d(xv, wd, bd, self.act, conv_state=sv, conv_state_indices=idd, has_initial_state=hid,
                               seq_starts=ssd, out=ov, dev_status=stat)
        assert ret is ov
        self.kernel = dc.dcconv_last_kernel()
        torch.cuda.synchronize()
        if sb is not None:
            assert_guards_intact(sb)
        assert_guards_intact(ob)
        assert np.array_equal(from_dev(xb)[GUARD:GUARD + self.x.size].reshape(self.x.shape), self.x), "x was written"
        state = None if sb is None else from_dev(sd)
        return from_dev(ov.permute(0, 2, 1)), state, (int(stat.item()) if stat is not None else None)

    def check(self):
        ref_out, ref32, ref_state = self.reference()
        out, state, status = self.run_gpu()
        if ref_state is not None:
            np.testing.assert_array_equal(state, ref_state, err_msg="state not bit-exact")
        assert_outputs_match(out, ref_out, ref32, exact=self.act in (None, "identity"))
        return status


# ------------------------------------------------------------------- batch form


@pytest.mark.parametrize("L", [3, 4, 8])
@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 70])
def test_prefill_batch_compact(L, T):
    case = PrefillCase(2000 + 10 * L + T, 1096, N=3, T=T, L=L, state="compact", bias=T % 2 == 0,
                       act=None if T % 3 == 0 else "silu")
    case.check()
    assert case.kernel == f"prefill_sweep_v8<L={L},{'identity' if T % 3 == 0 else 'silu'},compact>", case.kernel


@pytest.mark.parametrize("L", [3, 5, 6, 7, 8])
@pytest.mark.parametrize("T", [2, 9, 65])
def test_prefill_batch_channel_last(L, T):
    case = PrefillCase(2100 + 10 * L + T, 1608, N=5, T=T, L=L, state="channel_last", routing="unique", S=9,
                       bias=True, has_init="mixed")
    case.check()
    assert f"L={L}" in case.kernel and "channel_last" in case.kernel, case.kernel


@pytest.mark.parametrize("T", [1, 3, 40])
def test_prefill_stateless(T):
    case = PrefillCase(2200 + T, 520, N=4, T=T, state=None, bias=True)
    case.check()
    assert case.kernel == "prefill_sweep_v8<stateless,silu>", case.kernel


# Which form a call takes: the sweep for rows of at most 4096 channels or
# columns of at most 64 tokens, the chunk (column) form otherwise.  D = 4616 has
# a ragged last tile of one lane.

@pytest.mark.parametrize("layout", ["compact", "channel_last", None])
def test_prefill_column_form(layout):
    case = PrefillCase(2250, 4616, N=8, T=1700, L=4 if layout == "compact" else 3, state=layout,
                       routing="padded" if layout else "none", n_pad=2, S=10, bias=True, has_init="mixed",
                       status=layout is not None)
    assert case.check() in (None, 0)
    assert case.kernel.startswith("prefill_v8<"), case.kernel


def test_prefill_column_form_packed():
    rng = np.random.default_rng(2260)
    lens = [int(v) for v in rng.integers(1500, 3000, size=9)] + [0, 2]
    case = PrefillCase(2260, 4616, lens=lens, L=5, state="compact", routing="unique", S=12, has_init="mixed",
                       status=True)
    assert case.check() == 0
    assert case.kernel.startswith("prefill_v8<L=5,"), case.kernel


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
def test_prefill_sweep_form_wide_short(layout):
    """Wide rows but short columns (64 tokens or fewer per chunk wave) take the sweep."""
    case = PrefillCase(2270, 8192, N=2, T=300, L=3, state=layout, has_init="all", bias=True)
    case.check()
    assert case.kernel.startswith("prefill_sweep_v8<L=3,"), case.kernel


def test_prefill_sweep_packed_many_short_sequences():
    """Packed sequences shorter than a sweep item (16 tokens): items span many
    sequences, and a wave's 4 tokens cross several boundaries (empty and
    one-token sequences among them)."""
    rng = np.random.default_rng(2280)
    lens = [int(v) for v in rng.integers(0, 12, size=700)]
    case = PrefillCase(2280, 1032, lens=lens, L=3, state="channel_last", routing="padded", n_pad=40, S=700,
                       has_init="mixed", status=True, bias=True)
    assert case.check() == 0
    assert case.kernel.startswith("prefill_sweep_v8<"), case.kernel


def test_prefill_zero_tokens_writes_final_states():
    """t = 0: a sequence that continues from its slot keeps it; one that starts
    from zeros ends with a zero state."""
    case = PrefillCase(2300, 512, N=4, T=0, L=4, state="compact", has_init="mixed")
    case.check()


# ------------------------------------------------------------------- packed form


@pytest.mark.parametrize("state", ["compact", "channel_last", None])
def test_prefill_packed_varlen(state):
    lens = [0, 1, 2, 3, 5, 32, 33, 64, 100, 7, 0, 40]
    case = PrefillCase(2400, 2048, lens=lens, L=4 if state == "compact" else 3, state=state,
                       routing="unique" if state else "none", S=16, bias=True)
    case.check()


def test_prefill_packed_padding_and_status():
    lens = [4, 0, 37, 3, 70, 1]
    case = PrefillCase(2410, 1024, lens=lens, L=3, state="channel_last", routing="padded", n_pad=2, S=8,
                       status=True, has_init="all")
    assert case.check() == 0
    pad = case.indices == -1
    out, _, _ = case.run_gpu()
    for i in np.flatnonzero(pad):
        a, e = case.starts[i], case.starts[i + 1]
        assert np.all(wl.bf16_bits_to_f32(out[0, a:e]) == 0)


def test_prefill_bad_and_duplicate_indices():
    case = PrefillCase(2420, 1536, N=6, T=20, L=3, state="compact", routing="unique", S=8, status=True)
    case.indices = case.indices.copy()
    case.indices[1] = case.indices[4]
    case.indices[5] = 8
    oi = case.indices.copy(); oi[[1, 4, 5]] = -1
    case.oracle_indices = oi
    assert case.check() == dc.DCCONV_DEV_BAD_INDEX | dc.DCCONV_DEV_DUP_INDEX


def test_prefill_unordered_seq_starts_set_status_and_stay_in_bounds():
    """A sequence table that is not ordered is flagged; outputs are unspecified,
    but every write stays inside the operands (guards intact) and slots outside
    the flagged sequences keep their values."""
    rng = np.random.default_rng(2430)
    D, L, total = 512, 3, 40
    x = torch.from_numpy(_bf(rng, (1, total, D)).view(np.int16)).cuda().view(torch.bfloat16).permute(0, 2, 1)
    starts = torch.tensor([0, 30, 10, 40], dtype=torch.int32, device="cuda")  # sequence 1 runs backwards
    sb, sd = guarded_copy(_bf(rng, (4, L, D)))
    before = from_dev(sd)
    stat = torch.zeros(1, dtype=torch.int32, device="cuda")
    ob, od = guarded_empty((total * D,))
    out = torch.as_strided(od, (1, D, total), (total * D, 1, D))
    dc.causal_conv1d(x, to_dev(_bf(rng, (D, 4))), None, "silu", conv_state=sd.permute(0, 2, 1),
                     conv_state_indices=torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda"),
                     seq_starts=starts, out=out, dev_status=stat)
    torch.cuda.synchronize()
    assert int(stat.item()) & dc.DCCONV_DEV_BAD_SEQ
    assert_guards_intact(sb)
    assert_guards_intact(ob)
    after = from_dev(sd)
    np.testing.assert_array_equal(after[1], before[1])   # the flagged sequence's slot
    np.testing.assert_array_equal(after[3], before[3])   # nobody's slot


# ------------------------------------------------------------------- scalar path


@pytest.mark.parametrize("x_layout,out_layout,D,L", [("channel_major", "token_major", 512, 3),
                                                      ("token_major", "channel_major", 512, 4),
                                                      ("token_major", "token_major", 100, 3),
                                                      ("channel_major", "channel_major", 37, 9)])
def test_prefill_scalar_path(x_layout, out_layout, D, L):
    case = PrefillCase(2500 + D + L, D, N=3, T=13, L=L, state="compact", routing="padded", n_pad=1, S=5,
                       x_layout=x_layout, out_layout=out_layout, bias=True, status=True)
    assert case.check() == 0
    assert case.kernel == "prefill_scalar<silu>", case.kernel


def test_prefill_scalar_packed_channel_last():
    case = PrefillCase(2510, 44, lens=[3, 0, 9, 1], L=5, state="channel_last", routing="unique", S=6,
                       act=None)
    case.check()
    assert case.kernel == "prefill_scalar<identity>", case.kernel


# ----------------------------------------------------- agreement with the decode path


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
def test_prefill_from_state_equals_multi_token_update(layout):
    """Continuing from the slots == the multi-token decode update, bit for bit."""
    rng = np.random.default_rng(2600)
    N, D, T, L, S = 6, 2048, 19, 4, 9
    xt = _bf(rng, (N, T, D)); w = _bf(rng, (D, 4)); b = _bf(rng, (D,), 0.1)
    st = _bf(rng, (S, D, L) if layout == "compact" else (S, L, D))
    idx = torch.from_numpy(rng.choice(S, N, replace=False).astype(np.int32)).cuda()
    xd = to_dev(xt).permute(0, 2, 1)
    s1, s2 = to_dev(st), to_dev(st)
    v1 = s1 if layout == "compact" else s1.permute(0, 2, 1)
    v2 = s2 if layout == "compact" else s2.permute(0, 2, 1)
    wd, bd = to_dev(w), to_dev(b)
    o1 = dc.causal_conv1d(xd, wd, bd, "silu", conv_state=v1, conv_state_indices=idx,
                          has_initial_state=torch.ones(N, dtype=torch.bool, device="cuda"))
    o2 = dc.causal_conv1d_update_tokens(xd, v2, wd, bd, "silu", conv_state_indices=idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(o1.permute(0, 2, 1)), from_dev(o2.permute(0, 2, 1)))
    np.testing.assert_array_equal(from_dev(s1), from_dev(s2))


def test_prefill_final_state_hands_off_to_decode():
    """Prefill T tokens returning the channel-last L=3 state, then one decode step
    on that state in place == the oracle's prefill of T+1 tokens."""
    rng = np.random.default_rng(2610)
    N, D, T = 4, 4096, 50
    xt = _bf(rng, (N, T + 1, D)); w = _bf(rng, (D, 4)); b = _bf(rng, (D,), 0.1)
    wd, bd = to_dev(w), to_dev(b)
    xd = to_dev(np.ascontiguousarray(xt[:, :T])).permute(0, 2, 1)
    out, state = dc.causal_conv1d(xd, wd, bd, "silu", return_final_state=True)
    assert state.shape == (N, D, 3) and state.stride() == (3 * D, 1, D)
    y = dc.causal_conv1d_update(to_dev(np.ascontiguousarray(xt[:, T])), state, wd, bd, "silu")
    torch.cuda.synchronize()
    ref_st = np.zeros((N, D, 3), np.uint16)
    ref, ref32 = oracle.prefill(np.ascontiguousarray(xt), N, D, T + 1, ((T + 1) * D, 1, D), w, b, "silu",
                                state_buf=ref_st, S=N, L=3, state_strides=(3 * D, 3, 1), want_f32=True)
    assert_outputs_match(from_dev(out.permute(0, 2, 1)), ref[:, :T], ref32[:, :T], what="prefill out")
    assert_outputs_match(from_dev(y), ref[:, T], ref32[:, T], what="decode out")
    np.testing.assert_array_equal(from_dev(state.permute(0, 2, 1)).transpose(0, 2, 1), ref_st)


# ---------------------------------------------------------------- full size


@pytest.mark.parametrize("layout", ["channel_last", "compact"])
def test_prefill_full_size(layout):
    """Two sequences of 2048 tokens over 4096 channels (one prefill batch of the
    width-four short convolution), checked element by element."""
    case = PrefillCase(2700, 4096, N=2, T=2048, L=3, state=layout, has_init="mixed", act="silu")
    case.check()
    assert f"L=3,silu,{layout}" in case.kernel, case.kernel


@pytest.mark.parametrize("T", [200_000, 524_288])
def test_prefill_long_chunks(T):
    """A long sequence at a narrow width: the chunk kernel's per-call chunk
    length grows to its largest values (about 100 and 256 tokens per wave)."""
    case = PrefillCase(2800 + T % 97, 64, N=1, T=T, L=3, state="channel_last", has_init="all", bias=True)
    case.check()


def test_prefill_packed_long_chunks_cross_many_sequences():
    """Packed sequences shorter than a chunk: one wave's chunk spans many of them."""
    rng = np.random.default_rng(2900)
    lens = [int(v) for v in rng.integers(0, 40, size=3000)]
    case = PrefillCase(2900, 64, lens=lens, L=4, state="compact", routing="unique", S=3000, has_init="mixed")
    case.check()


def test_prefill_in_hip_graph_chunked_continuation():
    """A captured prefill that continues every sequence from its slot, replayed
    with fresh tokens: each replay is the next chunk of the same sequences, and
    matches the oracle continuing the same way."""
    rng = np.random.default_rng(3000)
    N, D, T, L = 4, 1024, 37, 3
    st_h = _bf(rng, (N, L, D)); w_h = _bf(rng, (D, 4))
    sd, wd = to_dev(st_h), to_dev(w_h)
    sv = sd.permute(0, 2, 1)
    xbuf = torch.empty(N, T, D, dtype=torch.bfloat16, device="cuda")
    obuf = torch.empty(N, T, D, dtype=torch.bfloat16, device="cuda")
    hi = torch.ones(N, dtype=torch.bool, device="cuda")
    xbuf.copy_(to_dev(_bf(rng, (N, T, D))))
    dc.causal_conv1d(xbuf.permute(0, 2, 1), wd, None, "silu", conv_state=sv, has_initial_state=hi,
                     out=obuf.permute(0, 2, 1))  # warm
    torch.cuda.synchronize()
    ref_state = np.ascontiguousarray(from_dev(sd).transpose(0, 2, 1))   # oracle keeps it compact
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dc.causal_conv1d(xbuf.permute(0, 2, 1), wd, None, "silu", conv_state=sv, has_initial_state=hi,
                         out=obuf.permute(0, 2, 1))
    for step in range(4):
        x_h = _bf(rng, (N, T, D))
        xbuf.copy_(to_dev(x_h))
        g.replay()
        torch.cuda.synchronize()
        ref, ref32 = oracle.prefill(x_h, N, D, T, (T * D, 1, D), w_h, None, "silu", state_buf=ref_state, S=N, L=L,
                                    state_strides=(D * L, L, 1), has_init=np.ones(N, np.uint8), want_f32=True)
        assert_outputs_match(from_dev(obuf), ref, ref32, what=f"replay {step}")
        np.testing.assert_array_equal(from_dev(sd).transpose(0, 2, 1), ref_state)
        _ = (xbuf.float() * 2).sum().item()  # eager work between replays
