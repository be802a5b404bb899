"""GPU parity of the multi-token update x[N, D, T] against the CPU oracle.

The oracle applies the T tokens of each row as T successive single decode steps
(the form the cuDNN FE-OSS page "Causal Conv1d Decode Update" reserves in its
section "Semantic tensor contract"); the library does them in one call.  Each
case requires: the whole state buffer bit-exact (selected slots shifted T
places, every other slot untouched, guard bands intact), x unwritten, padding
rows zero for every token, and outputs within 1 BF16 ulp or
1e-2 * max(1, |ref|) of the FP32 oracle (exact for the identity activation).
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


def _x_phys(rng, N, D, T, x_layout, ldx):
    """x in one of three physical layouts; returns (buffer, element strides (n, c, t))."""
    vals = _bf(rng, (N, T, D))
    if x_layout == "token_major":        # [N, T, ldx]
        buf = np.full((N, T, ldx), wl.PAD_SENTINEL, np.uint16)
        buf[:, :, :D] = vals
        return buf, (T * ldx, 1, ldx)
    if x_layout == "step_major":         # [T, N, ldx], as successive decode batches
        buf = np.full((T, N, ldx), wl.PAD_SENTINEL, np.uint16)
        buf[:, :, :D] = vals.transpose(1, 0, 2)
        return buf, (ldx, 1, N * ldx)
    if x_layout == "channel_major":      # [N, D, T]
        return np.ascontiguousarray(vals.transpose(0, 2, 1)), (D * T, T, 1)
    raise ValueError(x_layout)


def _out_strides(N, D, T, out_layout):
    if out_layout == "token_major":
        return (N * T * D,), (T * D, 1, D)
    if out_layout == "channel_major":
        return (N * D * T,), (D * T, T, 1)
    raise ValueError(out_layout)


class TokensCase:
    def __init__(self, seed, N, D, T, L, S=None, layout="compact", x_layout="token_major", ldx=None,
                 out_layout="token_major", bias=False, act="silu", routing="none", n_pad=0, status=False):
        rng = np.random.default_rng(seed)
        self.N, self.D, self.T, self.L = N, D, T, L
        self.S = N if S is None else S
        self.layout, self.act, self.status, self.out_layout = layout, act, status, out_layout
        self.x, self.xs = _x_phys(rng, N, D, T, x_layout, D if ldx is None else ldx)
        self.weight = _bf(rng, (D, 4))
        self.state0 = _bf(rng, (self.S, D, L) if layout == "compact" else (self.S, L, D))
        self.strides = (D * L, L, 1) if layout == "compact" else (L * D, 1, D)
        self.bias = _bf(rng, (D,), 0.1) if bias else None
        self.indices = None
        if routing == "unique":
            self.indices = rng.choice(self.S, N, replace=False).astype(np.int32)
        elif routing == "padded":
            real = rng.choice(self.S, N - n_pad, replace=False).astype(np.int32)
            self.indices = np.concatenate([real, np.full(n_pad, -1, np.int32)])[rng.permutation(N)].astype(np.int32)
        self.oracle_indices = self.indices

    def reference(self):
        st = self.state0.copy()
        out, out32 = oracle.update_tokens(self.x, self.N, self.D, self.T, self.xs, st, self.S, self.L, self.strides,
                                          self.weight, self.bias, self.oracle_indices, self.act, want_f32=True)
        return out, out32, st

    def run_gpu(self, dev="cuda"):
        N, D, T = self.N, self.D, self.T
        xb, xd = guarded_copy(self.x, dev)
        xv = torch.as_strided(xd.reshape(-1), (N, D, T), self.xs)
        sb, sd = guarded_copy(self.state0, dev)
        sv = sd if self.layout == "compact" else sd.permute(0, 2, 1)
        wd = to_dev(self.weight, dev)
        bd = None if self.bias is None else to_dev(self.bias, dev)
        idd = None if self.indices is None else torch.from_numpy(self.indices).to(dev)
        oshape, ostr = _out_strides(N, D, T, self.out_layout)
        ob, od = guarded_empty(oshape, dev)
        ov = torch.as_strided(od, (N, D, T), ostr)
        stat = torch.zeros(1, dtype=torch.int32, device=dev) if self.status else None
        ret = dc.causal_conv1d_update_tokens(xv, sv, wd, bd, self.act, conv_state_indices=idd, out=ov,
                                             dev_status=stat)
        assert ret is ov
        self.kernel = dc.dcconv_last_kernel()
        torch.cuda.synchronize()
        assert_guards_intact(sb)
        assert_guards_intact(ob)
        assert np.array_equal(from_dev(xb)[GUARD:GUARD + self.x.size].reshape(self.x.shape), self.x), "x was written"
        out = from_dev(ov.permute(0, 2, 1))  # [N, T, D]
        return out, from_dev(sd), (int(stat.item()) if stat is not None else None)

    def check(self):
        ref_out, ref32, ref_state = self.reference()
        out, state, status = self.run_gpu()
        np.testing.assert_array_equal(state, ref_state, err_msg="state not bit-exact")
        assert_outputs_match(out, ref_out, ref32, exact=self.act in (None, "identity"))
        if self.oracle_indices is not None:
            pad = self.oracle_indices == -1
            assert np.all(wl.bf16_bits_to_f32(out[pad]) == 0), "padding row output not zero"
        return status


# ------------------------------------------------------------------ vector path


def _one_row_form(T, L):
    """Kernel-name suffix of the one-row form on a thin grid: a call of at least
    2L tokens splits each row's tokens over two waves, and a wave with 5 to 8
    tokens takes them in one pass."""
    split = T >= 2 * L
    per_wave = T - T // 2 if split else T
    return "R=1" + (",split" if split else "") + (",one pass" if 4 < per_wave <= 8 else "") + ">"


@pytest.mark.parametrize("L", [3, 4, 8])
@pytest.mark.parametrize("T", [1, 2, 3, 7, 8, 9, 16, 33])
def test_tokens_compact(L, T):
    case = TokensCase(1000 + 10 * L + T, N=6, D=1096, T=T, L=L, bias=T % 2 == 1,
                      act="silu" if T % 3 else None)
    case.check()
    assert case.kernel.startswith(f"tokens_v8<L={L},") and case.kernel.endswith("compact," + _one_row_form(T, L)), \
        case.kernel


@pytest.mark.parametrize("L", [5, 6, 7])
def test_tokens_compact_other_history_lengths(L):
    case = TokensCase(1100 + L, N=5, D=520, T=11, L=L, bias=True, act="silu", routing="unique", S=9)
    case.check()
    assert case.kernel == f"tokens_v8<L={L},silu,compact," + _one_row_form(11, L), case.kernel


@pytest.mark.parametrize("L", [3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("T", [1, 4, 7, 17])
def test_tokens_channel_last(L, T):
    case = TokensCase(1200 + 10 * L + T, N=7, D=1608, T=T, L=L, layout="channel_last", bias=L % 2 == 0,
                      act="silu" if T != 4 else None, routing="unique", S=11)
    case.check()
    assert case.kernel.startswith(f"tokens_v8<L={L},") and case.kernel.endswith("channel_last," + _one_row_form(T, L)), \
        case.kernel


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
def test_tokens_step_major_padded_rows(layout):
    """x as T successive decode batches [T, N, ldx] with padded rows (ldx > D)."""
    case = TokensCase(1300, N=9, D=2048, T=6, L=4, layout=layout, x_layout="step_major", ldx=2056, bias=True)
    case.check()
    assert case.kernel.startswith("tokens_v8<L=4,silu,"), case.kernel


def test_tokens_long_history_in_one_call():
    """The long-history workload's 16 decode steps as one multi-token call."""
    spec = wl.BY_NAME["long_history"]
    data = wl.make(spec)
    case = TokensCase(0, N=1, D=8, T=1, L=spec.L)   # shell; fields replaced below
    case.N, case.D, case.T, case.L, case.S = spec.N, spec.D, spec.T, spec.L, spec.S
    case.x, case.xs = data["x"], (spec.ld, 1, spec.N * spec.ld)
    case.weight, case.state0, case.bias = data["weight"], data["state"], data["bias"]
    case.strides = wl.state_strides(spec)
    case.indices = case.oracle_indices = data["indices"]
    case.act, case.layout, case.out_layout, case.status = spec.act, spec.layout, "token_major", True
    assert case.check() == 0
    assert case.kernel == "tokens_v8<L=8,identity,compact,R=1,split,one pass>", case.kernel


def _two_row_form(T):
    """Kernel-name suffix of the two-row form: 5 to 8 tokens go in one pass."""
    return "R=2,one pass>" if 4 < T <= 8 else "R=2>"


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
@pytest.mark.parametrize("T", [4, 8])
def test_tokens_full_size_large_decode(layout, T):
    """The large decode batch (N=256, D=8192, L=3, SiLU) advanced 4 or 8 tokens at
    once, checked element by element against the oracle at full size."""
    case = TokensCase(1400 + T, N=256, D=8192, T=T, L=3, layout=layout, ldx=8200)
    case.check()
    assert case.kernel == f"tokens_v8<L=3,silu,{layout}," + _two_row_form(T), case.kernel


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
@pytest.mark.parametrize("T", [3, 7, 9])
def test_tokens_two_rows_per_wave(layout, T):
    """Enough rows for two per wave: odd N (a lone last row), padding rows,
    bias, L = 4, token counts that leave a partial pass of 4."""
    case = TokensCase(1450 + T, N=191, D=8192, T=T, L=4, layout=layout, bias=True, routing="padded", n_pad=9,
                      S=200, status=True)
    assert case.check() == 0
    assert case.kernel == f"tokens_v8<L=4,silu,{layout}," + _two_row_form(T), case.kernel


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
@pytest.mark.parametrize("L,T", [(3, 6), (3, 7), (4, 8), (8, 16), (8, 17), (6, 33)])
def test_tokens_split_rows(layout, L, T):
    """Thin grid, long call: each row's tokens split over the block's two waves
    (the first reads the state, the second starts from the three tokens before
    its half and writes the final state).  Ragged last tile, padding rows, a
    status word, bias, T = 2L exactly and odd T."""
    case = TokensCase(2300 + 10 * L + T, N=10, D=1096, T=T, L=L, layout=layout, bias=True, routing="padded",
                      n_pad=3, S=14, status=True, act="silu" if T % 2 else None)
    assert case.check() == 0
    assert case.kernel == f"tokens_v8<L={L},{'silu' if T % 2 else 'identity'},{layout}," + _one_row_form(T, L), \
        case.kernel


def test_tokens_one_row_full_grid_does_not_split():
    """A grid of one row per wave that already holds two waves per SIMD keeps
    each row on one wave (L > 4 rules out two rows per wave)."""
    case = TokensCase(2400, N=129, D=8192, T=11, L=5, bias=True, routing="padded", n_pad=5, S=140, status=True)
    assert case.check() == 0
    assert case.kernel == "tokens_v8<L=5,silu,compact,R=1>", case.kernel


# ---------------------------------------------------------- routing and padding


@pytest.mark.parametrize("N", [1, 3, 10])
def test_tokens_padding_rows_write_zeros(N):
    case = TokensCase(1500 + N, N=N, D=1024, T=5, L=3, S=16, routing="padded", n_pad=(N + 1) // 2,
                      bias=True, status=True)
    assert case.check() == 0


def test_tokens_bad_and_duplicate_indices():
    case = TokensCase(1600, N=8, D=1536, T=9, L=4, S=10, routing="unique", status=True)
    case.indices = case.indices.copy()
    case.indices[1] = case.indices[5]
    case.indices[7] = 10
    oi = case.indices.copy(); oi[[1, 5, 7]] = -1
    case.oracle_indices = oi
    assert case.check() == dc.DCCONV_DEV_BAD_INDEX | dc.DCCONV_DEV_DUP_INDEX


# ------------------------------------------------------------------ scalar path


@pytest.mark.parametrize("x_layout,out_layout,D", [("channel_major", "token_major", 1024),
                                                    ("token_major", "channel_major", 1024),
                                                    ("token_major", "token_major", 100),
                                                    ("channel_major", "channel_major", 37)])
def test_tokens_scalar_path(x_layout, out_layout, D):
    case = TokensCase(1700 + D, N=5, D=D, T=7, L=4, x_layout=x_layout, out_layout=out_layout, bias=True,
                      routing="padded", n_pad=1, S=7, status=True)
    assert case.check() == 0
    assert case.kernel == "tokens_scalar<silu>", case.kernel


def test_tokens_scalar_path_channel_last_identity():
    case = TokensCase(1800, N=4, D=44, T=10, L=9, layout="channel_last", act=None, routing="unique", S=6)
    case.check()
    assert case.kernel == "tokens_scalar<identity>", case.kernel


# --------------------------------------------------------- agreement with single steps


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
def test_one_token_call_equals_single_step_entry(layout):
    """T = 1 through the multi-token entry gives the single-step entry's bits."""
    rng = np.random.default_rng(1900)
    N, D, L, S = 12, 3072, 4, 16
    x = _bf(rng, (N, D)); w = _bf(rng, (D, 4)); b = _bf(rng, (D,), 0.1)
    st = _bf(rng, (S, D, L) if layout == "compact" else (S, L, D))
    idx = rng.choice(S, N, replace=False).astype(np.int32)
    dev = "cuda"
    s1, s2 = to_dev(st, dev), to_dev(st, dev)
    v1 = s1 if layout == "compact" else s1.permute(0, 2, 1)
    v2 = s2 if layout == "compact" else s2.permute(0, 2, 1)
    xd, wd, bd, idd = to_dev(x, dev), to_dev(w, dev), to_dev(b, dev), torch.from_numpy(idx).to(dev)
    o1 = dc.causal_conv1d_update(xd, v1, wd, bd, "silu", conv_state_indices=idd)
    o2 = dc.causal_conv1d_update_tokens(xd.unsqueeze(2), v2, wd, bd, "silu", conv_state_indices=idd)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(o2[:, :, 0]), from_dev(o1))
    np.testing.assert_array_equal(from_dev(s2), from_dev(s1))


def test_tokens_equal_successive_single_step_calls_on_gpu():
    """T tokens in one call give the same bits as T calls of the single-step entry."""
    rng = np.random.default_rng(2000)
    N, D, L, T = 16, 2560, 3, 12
    x = _bf(rng, (N, T, D)); w = _bf(rng, (D, 4)); st = _bf(rng, (N, D, L))
    dev = "cuda"
    xd, wd = to_dev(x, dev), to_dev(w, dev)
    s_tok, s_seq = to_dev(st, dev), to_dev(st, dev)
    out_tok = dc.causal_conv1d_update_tokens(xd.permute(0, 2, 1), s_tok, wd, None, "silu")
    outs = [dc.causal_conv1d_update(xd[:, t, :], s_seq, wd, None, "silu") for t in range(T)]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(out_tok.permute(0, 2, 1)), np.stack([from_dev(o) for o in outs], 1))
    np.testing.assert_array_equal(from_dev(s_tok), from_dev(s_seq))


def test_tokens_zero_tokens_leave_everything():
    rng = np.random.default_rng(2100)
    st = _bf(rng, (4, 64, 3))
    sd = to_dev(st, "cuda")
    x = torch.empty(4, 64, 0, dtype=torch.bfloat16, device="cuda")
    out = dc.causal_conv1d_update_tokens(x, sd, to_dev(_bf(rng, (64, 4)), "cuda"))
    torch.cuda.synchronize()
    assert out.shape == (4, 64, 0)
    np.testing.assert_array_equal(from_dev(sd), st)


@pytest.mark.parametrize("T", [5, 9])
def test_tokens_in_hip_graph_replays(T):
    """A captured multi-token call, replayed with fresh tokens each time (copied
    in eagerly between replays), matches the oracle stepping the same way
    (T = 9 takes the split form)."""
    rng = np.random.default_rng(2200 + T)
    N, D, L = 64, 2048, 4
    st_h = _bf(rng, (N, D, L)); w_h = _bf(rng, (D, 4)); b_h = _bf(rng, (D,), 0.1)
    sd, wd, bd = to_dev(st_h), to_dev(w_h), to_dev(b_h)
    xbuf = torch.empty(N, T, D, dtype=torch.bfloat16, device="cuda")
    obuf = torch.empty(N, T, D, dtype=torch.bfloat16, device="cuda")
    x_view, o_view = xbuf.permute(0, 2, 1), obuf.permute(0, 2, 1)
    xbuf.copy_(to_dev(_bf(rng, (N, T, D))))
    dc.causal_conv1d_update_tokens(x_view, sd, wd, bd, "silu", out=o_view)  # warm
    torch.cuda.synchronize()
    ref_state = from_dev(sd)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dc.causal_conv1d_update_tokens(x_view, sd, wd, bd, "silu", out=o_view)
    for step in range(4):
        x_h = _bf(rng, (N, T, D))
        xbuf.copy_(to_dev(x_h))
        g.replay()
        torch.cuda.synchronize()
        ref, ref32 = oracle.update_tokens(x_h, N, D, T, (T * D, 1, D), ref_state, N, L, (D * L, L, 1), w_h, b_h,
                                          None, "silu", want_f32=True)
        assert_outputs_match(from_dev(obuf), ref, ref32, what=f"replay {step}")
        np.testing.assert_array_equal(from_dev(sd), ref_state)
        _ = (xbuf.float() * 2).sum().item()  # eager work between replays
