"""GPU parity of the decode step on circular-buffer state (``cache_seqlens``).

The cuDNN FE-OSS page "Causal Conv1d Decode Update" reserves ``cache_seqlens``
for circular-buffer state (section "Causal Conv1d Decode Update").  Ring
reading: a slot that has seen c tokens keeps token i at position i mod L; the
taps are tokens c-3..c-1 and x, and x replaces the oldest token at c mod L.
Every case runs the HIP library and the CPU oracle on the same seeded inputs
and requires the whole state buffer bit-exact (one value per channel written,
guard bands intact), padding and rejected rows zero, and outputs within 1 BF16
ulp or 1e-2 * max(1, |ref|) of the FP32 oracle (exact for identity).
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


class RingCase:
    def __init__(self, seed, N, D, L, *, S=None, ld=None, layout="channel_last", bias=False, act="silu",
                 routing="none", n_pad=0, max_seen=100, status=False):
        rng = np.random.default_rng(seed)
        self.N, self.D, self.L = N, D, L
        self.S = N if S is None else S
        self.ld = D if ld is None else ld
        self.layout, self.act, self.status = layout, act, status
        self.x = np.full((N, self.ld), wl.PAD_SENTINEL, np.uint16)
        self.x[:, :D] = _bf(rng, (N, D))
        self.weight = _bf(rng, (D, 4))
        self.bias = _bf(rng, (D,), 0.1) if bias else None
        if layout == "compact":
            self.state0, self.st = _bf(rng, (self.S, D, L)), (D * L, L, 1)
        else:
            self.state0, self.st = _bf(rng, (self.S, L, D)), (L * D, 1, D)
        self.indices = None
        if routing == "unique":
            self.indices = rng.choice(self.S, N, replace=False).astype(np.int32)
        elif routing == "padded":
            real = rng.choice(self.S, N - n_pad, replace=False).astype(np.int32)
            self.indices = np.concatenate([real, np.full(n_pad, -1, np.int32)])[rng.permutation(N)].astype(np.int32)
        self.oracle_indices = self.indices
        seen = rng.integers(0, max_seen + 1, size=N).astype(np.int32)
        seen[: min(N, 3)] = np.arange(min(N, 3))          # always cover c = 0, 1, 2 (window wraps)
        self.seqlens = seen
        self.oracle_seqlens = seen

    def reference(self):
        st = self.state0.copy()
        out, out32 = oracle.update_ring(self.x, self.N, self.D, self.ld, st, self.S, self.L, self.st, self.weight,
                                        self.bias, self.oracle_indices, self.oracle_seqlens, self.act, want_f32=True)
        return out, out32, st

    def run_gpu(self, dev="cuda"):
        xb, xd = guarded_copy(self.x, dev)
        sb, sd = guarded_copy(self.state0, dev)
        sv = sd if self.layout == "compact" else sd.permute(0, 2, 1)
        ob, od = guarded_empty((self.N, self.D), dev)
        idd = None if self.indices is None else torch.from_numpy(self.indices).to(dev)
        csd = torch.from_numpy(self.seqlens).to(dev)
        stat = torch.zeros(1, dtype=torch.int32, device=dev) if self.status else None
        dc.causal_conv1d_update_out(xd[:, :self.D], sv, to_dev(self.weight, dev),
                                    None if self.bias is None else to_dev(self.bias, dev), self.act, out=od,
                                    cache_seqlens=csd, conv_state_indices=idd, dev_status=stat)
        self.kernel = dc.dcconv_last_kernel()
        torch.cuda.synchronize()
        assert_guards_intact(sb)
        assert_guards_intact(ob)
        assert np.array_equal(from_dev(xb)[GUARD:GUARD + self.x.size].reshape(self.x.shape), self.x)
        np.testing.assert_array_equal(csd.cpu().numpy(), self.seqlens, err_msg="cache_seqlens was written")
        return from_dev(od), from_dev(sd), (int(stat.item()) if stat is not None else None)

    def check(self):
        ref_out, ref32, ref_state = self.reference()
        out, state, status = self.run_gpu()
        np.testing.assert_array_equal(state, ref_state, err_msg="state not bit-exact")
        assert_outputs_match(out, ref_out, ref32, exact=self.act in (None, "identity"))
        if self.oracle_indices is not None:
            assert np.all(wl.bf16_bits_to_f32(out[self.oracle_indices == -1]) == 0)
        return status


@pytest.mark.parametrize("L", [3, 4, 5, 8, 11])
@pytest.mark.parametrize("act", [None, "silu"])
def test_ring_channel_last(L, act):
    case = RingCase(3000 + L, N=9, D=1096, L=L, bias=L % 2 == 1, act=act, routing="unique", S=13, ld=1104)
    case.check()
    assert case.kernel.startswith("update_ring_v8<"), case.kernel


@pytest.mark.parametrize("L", [3, 4, 8])
def test_ring_compact_takes_the_scalar_kernel(L):
    case = RingCase(3100 + L, N=6, D=520, L=L, layout="compact", bias=True)
    case.check()
    assert case.kernel == "update_ring_scalar<silu>", case.kernel


def test_ring_odd_channels_scalar():
    case = RingCase(3150, N=5, D=37, L=4, layout="channel_last", act=None)
    case.check()
    assert case.kernel == "update_ring_scalar<identity>", case.kernel


def test_ring_padding_bad_and_duplicate_rows():
    case = RingCase(3200, N=10, D=1024, L=3, S=12, routing="padded", n_pad=2, status=True)
    case.indices = case.indices.copy()
    live = np.flatnonzero(case.indices >= 0)
    case.indices[live[1]] = case.indices[live[4]]      # duplicate
    case.indices[live[6]] = 12                         # out of range
    case.seqlens = case.seqlens.copy()
    case.seqlens[live[7]] = -5                         # negative count
    oi = case.indices.copy()
    oi[[live[1], live[4], live[6], live[7]]] = -1
    case.oracle_indices = oi
    cs = case.seqlens.copy(); cs[live[7]] = 0          # the oracle refuses negatives; the row is padding anyway
    case.oracle_seqlens = cs
    status = case.check()
    assert status == dc.DCCONV_DEV_BAD_INDEX | dc.DCCONV_DEV_DUP_INDEX | dc.DCCONV_DEV_BAD_SEQLEN


def test_ring_two_rows_per_wave_rejections():
    """Negative counts, padding and bad indices in the two-rows-per-wave kernel:
    rejected rows are zero and leave their slots alone, whichever row of its wave
    they are."""
    case = RingCase(3250, N=256, D=4096, L=3, S=300, routing="padded", n_pad=20, status=True, max_seen=5000)
    case.indices = case.indices.copy()
    live = np.flatnonzero(case.indices >= 0)
    case.seqlens = case.seqlens.copy()
    neg = live[[3, 4, 50, 51, 200]]                    # both rows of some waves, one row of others
    case.seqlens[neg] = -1 - np.arange(len(neg), dtype=np.int32)
    case.indices[live[100]] = 300                      # out of range
    oi = case.indices.copy()
    oi[neg] = -1
    oi[live[100]] = -1
    case.oracle_indices = oi
    cs = case.seqlens.copy(); cs[neg] = 0              # the oracle refuses negatives; those rows are padding
    case.oracle_seqlens = cs
    status = case.check()
    assert status == dc.DCCONV_DEV_BAD_INDEX | dc.DCCONV_DEV_BAD_SEQLEN
    assert case.kernel == "update_ring_v8<silu,R=2>", case.kernel


def test_ring_full_size_large_decode():
    """The large decode batch (N=256, D=8192, L=3, SiLU, x row stride 8200) on a
    channel-last ring, element by element."""
    case = RingCase(3300, N=256, D=8192, L=3, ld=8200, max_seen=100000)
    case.check()
    assert case.kernel == "update_ring_v8<silu,R=2>", case.kernel


def test_ring_steps_equal_shifting_steps_on_gpu():
    """Caller advances cache_seqlens each step; outputs equal the shifting update
    on a linear copy of the same history, and the ring rotated by c equals it."""
    rng = np.random.default_rng(3400)
    N, D, L, T = 16, 2048, 4, 9
    lin = _bf(rng, (N, L, D))                          # channel-last, position k = age order
    c = rng.integers(0, 40, size=N).astype(np.int32)
    ring = lin.copy()
    for n in range(N):
        for k in range(L):
            ring[n, (c[n] + k) % L] = lin[n, k]
    w, b = to_dev(_bf(rng, (D, 4))), to_dev(_bf(rng, (D,), 0.1))
    ld, rd = to_dev(lin), to_dev(ring)
    cd = torch.from_numpy(c).cuda()
    for t in range(T):
        xd = to_dev(_bf(rng, (N, D)))
        o_lin = dc.causal_conv1d_update(xd, ld.permute(0, 2, 1), w, b, "silu")
        o_ring = dc.causal_conv1d_update(xd, rd.permute(0, 2, 1), w, b, "silu", cache_seqlens=cd)
        cd += 1
        torch.cuda.synchronize()
        np.testing.assert_array_equal(from_dev(o_ring), from_dev(o_lin))
    lin_h, ring_h, c_h = from_dev(ld), from_dev(rd), cd.cpu().numpy()
    for n in range(N):
        for k in range(L):
            np.testing.assert_array_equal(ring_h[n, (c_h[n] + k) % L], lin_h[n, k])


def test_ring_in_hip_graph_with_advancing_counts():
    """One graph holds the ring update and the counter increment; every replay
    matches the oracle stepping the same way."""
    rng = np.random.default_rng(3500)
    N, D, L = 32, 1024, 3
    st_h = _bf(rng, (N, L, D)); w_h = _bf(rng, (D, 4)); c_h = rng.integers(0, 10, size=N).astype(np.int32)
    sd, wd = to_dev(st_h), to_dev(w_h)
    cd = torch.from_numpy(c_h.copy()).cuda()
    xd = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    od = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    xd.copy_(to_dev(_bf(rng, (N, D))))
    dc.causal_conv1d_update_out(xd, sd.permute(0, 2, 1), wd, None, "silu", out=od, cache_seqlens=cd)  # warm
    torch.cuda.synchronize()
    st_h = from_dev(sd); c_h = cd.cpu().numpy().copy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dc.causal_conv1d_update_out(xd, sd.permute(0, 2, 1), wd, None, "silu", out=od, cache_seqlens=cd)
        cd.add_(1)
    ref_state = np.ascontiguousarray(st_h.transpose(0, 2, 1))   # oracle in compact order
    for step in range(4):
        x_h = _bf(rng, (N, D))
        xd.copy_(to_dev(x_h))
        g.replay()
        torch.cuda.synchronize()
        ref, ref32 = oracle.update_ring(x_h, N, D, D, ref_state, N, L, (D * L, L, 1), w_h, None, None, c_h, "silu",
                                        want_f32=True)
        c_h = c_h + 1
        assert_outputs_match(from_dev(od), ref, ref32, what=f"replay {step}")
        np.testing.assert_array_equal(from_dev(sd), ref_state.transpose(0, 2, 1))
        np.testing.assert_array_equal(cd.cpu().numpy(), c_h)
        _ = (xd.float() * 2).sum().item()  # eager work between replays


# ----------------------------------------------------- T tokens per call on a ring


def _ring_tokens_reference(x_ntd, state_compact, weight, bias, indices, seqlens, act):
    """The oracle's ring step applied token by token (count advanced each token)."""
    N, T, D = x_ntd.shape
    S, _, L = state_compact.shape
    outs, outs32 = [], []
    c = seqlens.copy()
    for t in range(T):
        o, o32 = oracle.update_ring(np.ascontiguousarray(x_ntd[:, t]), N, D, D, state_compact, S, L, (D * L, L, 1),
                                    weight, bias, indices, c, act, want_f32=True)
        outs.append(o); outs32.append(o32)
        c = c + 1
    return np.stack(outs, 1), np.stack(outs32, 1)


@pytest.mark.parametrize("layout", ["channel_last", "compact"])
@pytest.mark.parametrize("L,T", [(3, 1), (3, 5), (3, 9), (4, 3), (4, 20), (8, 6), (8, 17)])
def test_ring_tokens(layout, L, T):
    rng = np.random.default_rng(3600 + 10 * L + T)
    N, D, S = 9, 1096, 12
    x = _bf(rng, (N, T, D)); w = _bf(rng, (D, 4)); b = _bf(rng, (D,), 0.1)
    st = _bf(rng, (S, D, L))                                     # compact values
    idx = rng.choice(S, N, replace=False).astype(np.int32)
    idx[4] = -1
    seen = rng.integers(0, 50, size=N).astype(np.int32)
    seen[:3] = [0, 1, 2]
    ref_state = st.copy()
    oi = idx.copy()
    ref, ref32 = _ring_tokens_reference(x, ref_state, w, b, oi, seen, "silu")
    phys = st if layout == "compact" else np.ascontiguousarray(st.transpose(0, 2, 1))
    sb, sd = guarded_copy(phys)
    sv = sd if layout == "compact" else sd.permute(0, 2, 1)
    ob, od = guarded_empty((N * T * D,))
    out = torch.as_strided(od, (N, D, T), (T * D, 1, D))
    dc.causal_conv1d_update_tokens(to_dev(x).permute(0, 2, 1), sv, to_dev(w), to_dev(b), "silu",
                                   conv_state_indices=torch.from_numpy(idx).cuda(),
                                   cache_seqlens=torch.from_numpy(seen).cuda(), out=out)
    kernel = dc.dcconv_last_kernel()
    torch.cuda.synchronize()
    assert_guards_intact(sb)
    assert_guards_intact(ob)
    got_state = from_dev(sd)
    if layout == "channel_last":
        got_state = got_state.transpose(0, 2, 1)
    np.testing.assert_array_equal(got_state, ref_state, err_msg="ring not bit-exact")
    assert_outputs_match(from_dev(out.permute(0, 2, 1)), ref, ref32)
    assert kernel == ("tokens_ring_v8<silu,R=1>" if layout == "channel_last" else "tokens_ring_scalar<silu>"), kernel


def test_ring_tokens_equal_single_ring_steps_on_gpu():
    """T tokens through the multi-token entry == T single ring steps with the
    count advanced in between, bit for bit."""
    rng = np.random.default_rng(3700)
    N, D, L, T = 32, 4096, 3, 7
    x = _bf(rng, (N, T, D)); w = to_dev(_bf(rng, (D, 4)))
    st = _bf(rng, (N, L, D))
    c = rng.integers(0, 100, size=N).astype(np.int32)
    s1, s2 = to_dev(st), to_dev(st)
    xd = to_dev(x)
    o1 = dc.causal_conv1d_update_tokens(xd.permute(0, 2, 1), s1.permute(0, 2, 1), w, None, "silu",
                                        cache_seqlens=torch.from_numpy(c).cuda())
    cd = torch.from_numpy(c).cuda()
    outs = []
    for t in range(T):
        outs.append(dc.causal_conv1d_update(xd[:, t].contiguous(), s2.permute(0, 2, 1), w, None, "silu",
                                            cache_seqlens=cd))
        cd += 1
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(o1.permute(0, 2, 1)), np.stack([from_dev(o) for o in outs], 1))
    np.testing.assert_array_equal(from_dev(s1), from_dev(s2))


def test_ring_tokens_bad_count_rejects_row():
    rng = np.random.default_rng(3800)
    N, D, L, T = 4, 512, 4, 3
    st = _bf(rng, (N, L, D)); sd = to_dev(st)
    seen = torch.tensor([5, -1, 0, 2], dtype=torch.int32, device="cuda")
    stat = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = dc.causal_conv1d_update_tokens(to_dev(_bf(rng, (N, T, D))).permute(0, 2, 1), sd.permute(0, 2, 1),
                                         to_dev(_bf(rng, (D, 4))), None, "silu", cache_seqlens=seen, dev_status=stat)
    torch.cuda.synchronize()
    assert int(stat.item()) == dc.DCCONV_DEV_BAD_SEQLEN
    assert np.all(wl.bf16_bits_to_f32(from_dev(out.permute(0, 2, 1))[1]) == 0)
    np.testing.assert_array_equal(from_dev(sd)[1], st[1])


@pytest.mark.parametrize("L,T", [(3, 3), (3, 5), (3, 6), (4, 8), (4, 9)])
def test_ring_tokens_two_rows_per_wave(L, T):
    """Enough rows for two per wave (odd N, a padding row, bias), partial passes;
    5 to 8 tokens go in one pass."""
    rng = np.random.default_rng(3900 + 10 * L + T)
    N, D, S = 129, 8192, 140
    x = _bf(rng, (N, T, D)); w = _bf(rng, (D, 4)); b = _bf(rng, (D,), 0.1)
    st = _bf(rng, (S, D, L))
    idx = rng.choice(S, N, replace=False).astype(np.int32)
    idx[7] = -1
    seen = rng.integers(0, 1000, size=N).astype(np.int32)
    ref_state = st.copy()
    ref, ref32 = _ring_tokens_reference(x, ref_state, w, b, idx, seen, "silu")
    sb, sd = guarded_copy(np.ascontiguousarray(st.transpose(0, 2, 1)))
    out = dc.causal_conv1d_update_tokens(to_dev(x).permute(0, 2, 1), sd.permute(0, 2, 1), to_dev(w), to_dev(b),
                                         "silu", conv_state_indices=torch.from_numpy(idx).cuda(),
                                         cache_seqlens=torch.from_numpy(seen).cuda())
    kernel = dc.dcconv_last_kernel()
    torch.cuda.synchronize()
    assert_guards_intact(sb)
    np.testing.assert_array_equal(from_dev(sd).transpose(0, 2, 1), ref_state, err_msg="ring not bit-exact")
    assert_outputs_match(from_dev(out.permute(0, 2, 1)), ref, ref32)
    assert kernel == ("tokens_ring_v8<silu,R=2,one pass>" if 4 < T <= 8 else "tokens_ring_v8<silu,R=2>"), kernel
