"""GPU parity of the decode update against the CPU oracle.

Every case runs the HIP library (through the C ABI) and the oracle on the same
seeded inputs and requires: the whole state buffer bit-exact (selected slots
shifted, every other slot untouched, guard bands intact), padding rows zero, and
outputs within 1 BF16 ulp or 1e-2 * max(1, |ref|) of the FP32 oracle; the
identity path must match the oracle's value exactly (its FP32 sum is formed in
the same order, and BF16 products are exact in FP32).

Semantics: cuDNN FE-OSS page "Causal Conv1d Decode Update", sections "Causal
Conv1d Decode Update" (update rule, routing, padding) and "Semantic tensor
contract" / "Current native implementation" (layouts, limits).
"""
import numpy as np
import pytest
import torch

import oracle
import depthwise_causal_conv1d_amd as dc
from depthwise_causal_conv1d_amd import workloads as wl
from parity import (Case, assert_outputs_match, from_dev, guarded_copy, guarded_empty, to_dev,
                    assert_guards_intact, takes_narrow, NARROW_MAX_WAVES)

pytestmark = pytest.mark.gpu


def _bf(rng, shape, scale=1.0):
    return wl.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def _x(rng, N, D, ld):
    x = np.full((N, ld), wl.PAD_SENTINEL, dtype=np.uint16)
    x[:, :D] = _bf(rng, (N, D))
    return x


def make_case(seed, N, D, L, S=None, ld=None, layout="compact", bias=False, routing="none", act="silu",
              status=False, n_pad=0):
    rng = np.random.default_rng(seed)
    S = N if S is None else S
    ld = D if ld is None else ld
    x = _x(rng, N, D, ld)
    w = _bf(rng, (D, 4))
    state = _bf(rng, (S, D, L) if layout == "compact" else (S, L, D))
    b = _bf(rng, (D,), 0.1) if bias else None
    idx = None
    if routing == "unique":
        idx = rng.choice(S, N, replace=False).astype(np.int32)
    elif routing == "padded":
        real = rng.choice(S, N - n_pad, replace=False).astype(np.int32)
        idx = np.concatenate([real, np.full(n_pad, -1, np.int32)])[rng.permutation(N)].astype(np.int32)
    return Case(x, D, w, state, layout=layout, bias=b, indices=idx, act=act, status=status)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dc._load()
    yield


# ------------------------------------------------------------ the five workloads


@pytest.mark.parametrize("spec", wl.DECODE_WORKLOADS[:4], ids=[c.name for c in wl.DECODE_WORKLOADS[:4]])
def test_configs_single_step(spec):
    data = wl.make(spec)
    case = Case(data["x"][0], spec.D, data["weight"], data["state"], bias=data["bias"],
                indices=data["indices"], act=spec.act, status=data["indices"] is not None)
    status = case.check()
    assert status in (None, 0)
    form = "update_narrow" if takes_narrow(spec.N, spec.D) else "update_compact_v8"
    assert case.kernel.startswith(form), case.kernel


def test_config_long_history_sequential():
    """16 successive decode steps on L=8 state: each step's output and the final
    state agree with the oracle stepping the same way."""
    spec = wl.BY_NAME["long_history"]
    data = wl.make(spec)
    x, w, b, idx = data["x"], data["weight"], data["bias"], data["indices"]
    st_host = data["state"].copy()
    dev = "cuda"
    sb, sd = guarded_copy(data["state"], dev)
    wd, bd, idd = to_dev(w, dev), to_dev(b, dev), torch.from_numpy(idx).to(dev)
    xd = to_dev(x, dev)
    for t in range(spec.T):
        ref, ref32 = oracle.update(np.ascontiguousarray(x[t]), st_host, w, b, spec.act,
                                   conv_state_indices=idx, want_f32=True)
        out = dc.causal_conv1d_update(xd[t], sd, wd, bd, spec.act, conv_state_indices=idd)
        assert_outputs_match(from_dev(out), ref, ref32, exact=True, what=f"step {t}")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(sd), st_host)
    assert_guards_intact(sb)


# ------------------------------------------------------------------- edge cases


# Rows for each form at D = 1544 (4 tiles of 512 channels): 5 rows take the
# narrow form, a few more rows than the narrow form's limit allows the
# 512-channel kernel.
FORMS = {"narrow": 5, "wide": NARROW_MAX_WAVES // 4 + 12}
FORM_KERNEL = {"narrow": "update_narrow", "wide": "_v8"}


def test_form_rows_straddle_the_threshold():
    assert takes_narrow(FORMS["narrow"], 1544) and not takes_narrow(FORMS["wide"], 1544)
    assert 4 * FORMS["wide"] > NARROW_MAX_WAVES


@pytest.mark.parametrize("form", ["narrow", "wide"])
@pytest.mark.parametrize("L", [3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("act", [None, "silu"])
def test_vector_path_every_l(L, act, form):
    # D = 1544 = 3 full 512-channel tiles + a 8-channel ragged tail tile
    # (12 full 128-channel tiles + the same tail for the narrow form)
    N = FORMS[form]
    case = make_case(100 + L, N=N, D=1544, L=L, S=N + 4, bias=True, routing="padded", n_pad=2 + N // 10, act=act)
    case.check()
    assert FORM_KERNEL[form] in case.kernel and "compact" in case.kernel, case.kernel


@pytest.mark.parametrize("D", [1, 7, 13, 100, 1001])
@pytest.mark.parametrize("L", [3, 4, 9])
def test_scalar_path_any_d(D, L):
    case = make_case(200 + D + L, N=6, D=D, L=L, S=11, bias=D % 2 == 1, routing="unique", act="silu")
    case.check()
    if D % 8 != 0 or L > 8:
        assert "scalar" in case.kernel


@pytest.mark.parametrize("L", [3, 4, 6])
@pytest.mark.parametrize("act", [None, "silu"])
@pytest.mark.parametrize("form", ["narrow", "wide"])
def test_channel_last_layout(L, act, form):
    N = {"narrow": 7, "wide": NARROW_MAX_WAVES // 3 + 9}[form]  # D = 1032: 3 tiles of 512 (2 full + 8 channels)
    case = make_case(300 + L, N=N, D=1032, L=L, S=N + 5, layout="channel_last", routing="padded", n_pad=3,
                     bias=True, act=act)
    case.check()
    assert FORM_KERNEL[form] in case.kernel and "channel_last" in case.kernel, case.kernel


@pytest.mark.parametrize("form", ["narrow", "wide"])
@pytest.mark.parametrize("L", [5, 7, 8])
def test_channel_last_more_l(L, form):
    N = FORMS[form]
    case = make_case(320 + L, N=N, D=1544, L=L, S=N + 4, layout="channel_last", routing="unique", bias=False,
                     act="silu")
    case.check()
    assert FORM_KERNEL[form] in case.kernel and "channel_last" in case.kernel, case.kernel


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
@pytest.mark.parametrize("act", [None, "silu"])
def test_two_rows_per_wave_odd_n_padding_bias(layout, act):
    """N odd (the last wave has one row and one row past the end), padding rows
    inside row pairs, a bias, an index table, a ragged tile: the two-row kernels."""
    case = make_case(330, N=151, D=8200, L=3, S=300, layout=layout, routing="padded", n_pad=17, bias=True, act=act,
                     status=True)
    assert case.check() == 0
    assert "R=2" in case.kernel, case.kernel


@pytest.mark.parametrize("N,R", [(160, 1), (192, 2), (256, 2)])
def test_rows_per_wave_follow_whole_rounds_of_blocks(N, R):
    """At D = 8192 on 256 CUs: 160 rows take one row per wave (1280 blocks, 5
    rounds) rather than two (640 blocks, 3 rounds of two rows); 192 and 256 rows
    take two.  Results are the same either way."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("the expected choice is worked out for 256 compute units")
    case = make_case(340 + N, N=N, D=8192, L=3, bias=False, act="silu")
    case.check()
    assert case.kernel == f"update_compact_v8<L=3,silu,R={R}>", case.kernel


def test_channel_last_full_size_large_decode():
    """The large decode shape (N=256, D=8192, L=3, ld=8200, SiLU) with the state
    handed over channel-last, checked element by element."""
    spec = wl.Spec("large_decode_cl", N=256, D=8192, W=4, L=3, S=256, ld=8200, bias=False, act="silu",
                   routing="none", weight_dist="uniform", seed=4, layout="channel_last")
    data = wl.make(spec)
    case = Case(data["x"][0], spec.D, data["weight"], data["state"], layout="channel_last", act="silu")
    case.check()
    assert case.kernel == "update_channel_last_v8<L=3,silu,R=2>"


def test_channel_last_scalar_path():
    case = make_case(310, N=4, D=21, L=3, S=4, layout="channel_last", act="silu")
    case.check()
    assert "scalar" in case.kernel


@pytest.mark.parametrize("ld", [1032, 1536])
def test_padded_row_stride_is_never_read(ld):
    case = make_case(400 + ld, N=9, D=1024, L=3, ld=ld, act="silu")
    case.check()


def test_single_row_and_single_channel_group():
    make_case(501, N=1, D=8, L=3, act="silu").check()
    make_case(502, N=1, D=1, L=3, act=None).check()


def test_all_rows_padding():
    case = make_case(503, N=6, D=512, L=3, S=3, routing="padded", n_pad=6, act="silu")
    case.check()


def test_zero_slots_all_padding():
    rng = np.random.default_rng(504)
    x = _x(rng, 3, 64, 64)
    case = Case(x, 64, _bf(rng, (64, 4)), np.zeros((0, 64, 3), np.uint16),
                indices=np.full(3, -1, np.int32), act="silu")
    case.check()


def test_zero_rows_launch_nothing():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    st = torch.zeros(2, 64, 3, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(64, 4, dtype=torch.bfloat16, device="cuda")
    out = dc.causal_conv1d_update(x, st, w, None, "silu")
    assert out.shape == (0, 64) and dc.dcconv_last_kernel() == ""


def test_many_rows_small_d():
    make_case(505, N=3000, D=16, L=4, S=3100, routing="unique", act="silu", bias=True).check()


def test_wide_channels():
    make_case(506, N=2, D=65536, L=3, act="silu").check()


def test_special_state_bits_survive_the_shift():
    """-0.0, denormals and NaN payloads in history positions that only shift
    (L=8: positions 0..4 never reach the taps) are copied bit for bit."""
    rng = np.random.default_rng(507)
    N, D, L = 3, 1024, 8
    case = make_case(507, N=N, D=D, L=L, act="silu")
    specials = np.array([0x8000, 0x0001, 0x807F, 0x7FC3, 0xFFD1, 0x7F80, 0xFF80], np.uint16)
    case.state0[:, :, :5] = rng.choice(specials, size=(N, D, 5))
    case.check()


# -------------------------------------------------------- routing rejections


def test_out_of_range_indices_set_status_and_touch_nothing():
    case = make_case(600, N=8, D=1024, L=3, S=10, routing="unique", act="silu", status=True)
    case.indices = case.indices.copy()
    case.indices[1] = -2
    case.indices[5] = 10
    oi = case.indices.copy(); oi[[1, 5]] = -1
    case.oracle_indices = oi
    status = case.check()
    assert status == dc.DCCONV_DEV_BAD_INDEX


def test_duplicate_indices_with_status_are_rejected_deterministically():
    case = make_case(601, N=8, D=1536, L=4, S=10, routing="unique", act="silu", status=True)
    case.indices = case.indices.copy()
    case.indices[6] = case.indices[2]
    oi = case.indices.copy(); oi[[2, 6]] = -1
    case.oracle_indices = oi
    status = case.check()
    assert status == dc.DCCONV_DEV_DUP_INDEX


def test_duplicates_and_bad_indices_in_scalar_path():
    case = make_case(602, N=6, D=13, L=3, S=8, routing="unique", act=None, status=True)
    case.indices = case.indices.copy()
    case.indices[0] = case.indices[3]
    case.indices[4] = 99
    oi = case.indices.copy(); oi[[0, 3, 4]] = -1
    case.oracle_indices = oi
    status = case.check()
    assert status == dc.DCCONV_DEV_BAD_INDEX | dc.DCCONV_DEV_DUP_INDEX


def test_repeated_padding_is_not_a_duplicate():
    case = make_case(603, N=10, D=512, L=3, S=10, routing="padded", n_pad=4, act="silu", status=True)
    assert case.check() == 0


# ---------------------------------------------------------- streams and graphs


def test_side_stream_with_default_stream_parked():
    """The launch honours the ambient stream: run on a side stream while the
    default stream is busy, then compare bit for bit with a default-stream run."""
    case = make_case(700, N=64, D=4096, L=3, act="silu", bias=True)
    ref_out, _, ref_state = case.reference()
    dev = "cuda"
    xd = to_dev(case.x, dev); sd = to_dev(case.state0, dev); wd = to_dev(case.weight, dev)
    bd = to_dev(case.bias, dev)
    # default-stream result
    s_def = sd.clone()
    out_def = dc.causal_conv1d_update(xd, s_def, wd, bd, "silu")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    s_side = sd.clone()
    torch.cuda.synchronize()
    torch.cuda._sleep(50_000_000)          # park the default stream
    with torch.cuda.stream(side):
        out_side = dc.causal_conv1d_update(xd, s_side, wd, bd, "silu")
        side.synchronize()                 # completes without waiting for the default stream
    torch.cuda.synchronize()
    assert torch.equal(out_side.view(torch.int16), out_def.view(torch.int16))
    assert torch.equal(s_side.view(torch.int16), s_def.view(torch.int16))
    np.testing.assert_array_equal(from_dev(s_side), ref_state)


def test_hip_graph_replays_match_eager_steps():
    """One captured update, replayed several times with eager work and syncs in
    between; every replay equals the oracle advanced by the same number of steps."""
    case = make_case(701, N=16, D=2048, L=4, S=20, routing="unique", act="silu", bias=True)
    dev = "cuda"
    xd = to_dev(case.x, dev); sd = to_dev(case.state0, dev); wd = to_dev(case.weight, dev)
    bd = to_dev(case.bias, dev); idd = torch.from_numpy(case.indices).to(dev)
    out = torch.empty(case.N, case.D, dtype=torch.bfloat16, device=dev)
    st_host = case.state0.copy()
    # warm the specialisation outside capture
    s_warm = sd.clone()
    dc.causal_conv1d_update_out(xd, s_warm, wd, bd, "silu", out=out, conv_state_indices=idd)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dc.causal_conv1d_update_out(xd, sd, wd, bd, "silu", out=out, conv_state_indices=idd)
    # capture does not execute: the state is still the initial one
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(sd), case.state0)
    for step in range(4):
        g.replay()
        torch.cuda.synchronize()
        ref, ref32 = oracle.update(case.x, st_host, case.weight, case.bias, "silu",
                                   conv_state_indices=case.indices, want_f32=True)
        assert_outputs_match(from_dev(out), ref, ref32, what=f"replay {step}")
        np.testing.assert_array_equal(from_dev(sd), st_host)
        _ = (xd.float() * 2).sum().item()  # eager work between replays


# ------------------------------------------------------ refusals on real tensors


def test_refusals_on_device_tensors():
    dev = "cuda"
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device=dev)
    st = torch.zeros(4, 64, 3, dtype=torch.bfloat16, device=dev)
    w = torch.zeros(64, 4, dtype=torch.bfloat16, device=dev)
    with pytest.raises(NotImplementedError):
        dc.causal_conv1d_update(x, st, torch.zeros(64, 3, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        dc.causal_conv1d_update(x, st, w, cache_seqlens=torch.zeros(4, dtype=torch.int64, device=dev))
    with pytest.raises(ValueError):
        dc.causal_conv1d_update(x, st[:3], w)            # S < N without a table
    with pytest.raises(ValueError):
        dc.causal_conv1d_update(x, torch.zeros(4, 64, 2, dtype=torch.bfloat16, device=dev),
                                torch.zeros(64, 4, dtype=torch.bfloat16, device=dev))  # L < W-1
    odd = torch.zeros(900 * 4, dtype=torch.bfloat16, device=dev).as_strided((4, 64, 3), (900, 1, 128))
    with pytest.raises(NotImplementedError):
        dc.causal_conv1d_update(x, odd, w)               # strides neither compact nor channel-last
    xo = torch.zeros(4, 72, dtype=torch.bfloat16, device=dev)[:, 2:66]   # misaligned rows
    with pytest.raises(ValueError):
        dc.causal_conv1d_update(xo, st, w)
    with pytest.raises(ValueError):
        dc.causal_conv1d_update_out(x, st, w, out=x)      # out aliases x
