"""Pins of the CPU oracle against things other than itself.

Each check is chosen so that a plausible slip in the oracle (a dropped tap, a tap
read from the wrong end of the history, a sign, a bias added twice, a padding row
that mutates, a wrong rounding) fails at least one of them:

* a float64 library convolution (``numpy.convolve``) over the initial state
  followed by the tokens, for single steps and for T successive steps;
* one-hot taps (a pure delay line), zero weights (the output is the bias),
  power-of-two scaling of an exact linear map;
* SiLU against torch's float64 ``silu``;
* BF16 conversion against torch's converter on all 65536 patterns and on ties;
* hand-worked examples of the page's update rule (``tests/golden``);
* routing laws: no table == identity table, row permutation, padding rows.

Semantics: cuDNN FE-OSS page "Causal Conv1d Decode Update", sections
"Causal Conv1d Decode Update" and "Semantic tensor contract".
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from depthwise_causal_conv1d_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U32 = 2.0 ** -24  # unit roundoff of FP32


def bf(a):
    return f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def rand_bf(rng, shape, scale=1.0):
    return bf(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


def conv_f64(ext, w):
    """Causal convolution by numpy: y[t] = sum_k w[W-1-k] * ext[t-k], t >= W-1."""
    return np.convolve(ext, w[::-1])


def silu64(a):
    return torch.nn.functional.silu(torch.as_tensor(a, dtype=torch.float64)).numpy()


def check_out(out_bits, out_f32, exact_acc, abs_terms, act):
    """out_f32 within the FP32 error bound of the exact value; out == one RNE rounding."""
    n_terms = 5
    err_acc = n_terms * U32 * abs_terms
    if act == "silu":
        ref = silu64(exact_acc)
        bound = 1.1 * err_acc + 8 * U32 * np.abs(ref) + 1e-37
    else:
        ref = exact_acc
        bound = err_acc + 1e-37
    err = np.abs(out_f32.astype(np.float64) - ref)
    assert np.all(err <= bound), f"max excess {np.max(err - bound)}"
    # the BF16 output is exactly the library RNE rounding of the FP32 value
    np.testing.assert_array_equal(out_bits, bf(out_f32))


# --------------------------------------------------------------------------- BF16


def test_bf16_to_f32_all_patterns():
    # every pattern, NaN payloads and signalling NaNs included, bit for bit
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f32(bits)
    lib = bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(ours.view(np.uint32), lib.view(np.uint32))


def test_f32_to_bf16_matches_library_rne():
    rng = np.random.default_rng(7)
    vals = [rng.standard_normal(3000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 3000)]
    # exact ties: a BF16 value plus half a BF16 ulp (both parities of the kept bit)
    base = rng.integers(0x0080, 0x7F00, 2000).astype(np.uint32) << 16
    vals.append((base | 0x8000).view(np.float32))
    vals.append((base | 0x8000 | 0x10000).view(np.float32))
    vals.append(((base | 0x7FFF)).view(np.float32))
    # denormals, zeros, infinities, values that round up to infinity
    special = np.array([0x00000001, 0x00008000, 0x007FFFFF, 0x80000000, 0x00000000,
                        0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF],
                       dtype=np.uint32).view(np.float32)
    vals.append(special)
    v = np.concatenate(vals).astype(np.float32)
    np.testing.assert_array_equal(oracle.f32_to_bf16(v), bf(v))


def test_f32_to_bf16_nan_stays_nan():
    # quiet and signalling NaNs, with payloads in the kept and in the dropped half
    nans = np.array([0x7FC00000, 0x7F800001, 0xFF800001, 0xFFC00001, 0x7FFFFFFF, 0x7F810000],
                    dtype=np.uint32).view(np.float32)
    out = oracle.f32_to_bf16(nans)
    assert np.all(np.isnan(bf16_bits_to_f32(out)))
    # the sign survives, and a payload in the kept half is kept
    np.testing.assert_array_equal(out >> 15, [0, 0, 1, 1, 0, 0])
    assert out[5] & 0x003F == 0x0001  # below the quiet bit, which is forced on


# ------------------------------------------------------------------- golden cases


def _load_golden():
    with open(os.path.join(GOLDEN, "update_hand_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _load_golden(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    state = bf(case["state"])
    x = bf(case["x"])
    w = bf(case["weight"])
    b = None if case["bias"] is None else bf(case["bias"])
    idx = None if case["indices"] is None else np.array(case["indices"], dtype=np.int32)
    out = oracle.update(x, state, w, b, case["activation"], conv_state_indices=idx)
    np.testing.assert_array_equal(out, bf(case["expected_out"]))
    np.testing.assert_array_equal(state, bf(case["expected_state"]))


# ------------------------------------------------- brute force vs library convolution


@pytest.mark.parametrize("D", [1, 7, 13, 64])
@pytest.mark.parametrize("L", [3, 4, 5, 8])
@pytest.mark.parametrize("act", [None, "silu"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_single_step_vs_f64_convolution(D, L, act, with_bias):
    rng = np.random.default_rng(1000 * D + 10 * L + with_bias)
    W, N, S = 4, 5, 9
    x = rand_bf(rng, (N, D))
    w = rand_bf(rng, (D, W))
    state = rand_bf(rng, (S, D, L))
    bias = rand_bf(rng, (D,), 0.1) if with_bias else None
    idx = np.array([3, -1, 0, 8, -1], dtype=np.int32)
    before = state.copy()
    out, out32 = oracle.update(x, state, w, bias, act, conv_state_indices=idx, want_f32=True)
    for n, s in enumerate(idx):
        if s < 0:
            assert np.all(out[n] == 0) and np.all(out32[n] == 0)
            continue
        for c in range(D):
            ext = np.concatenate([f64(before[s, c]), f64(x[n, c:c + 1])])
            full = conv_f64(ext, f64(w[c]))
            exact = full[L] + (f64(bias[c:c + 1])[0] if with_bias else 0.0)
            terms = np.abs(ext[L + 1 - W:]) @ np.abs(f64(w[c])) + (abs(f64(bias[c:c + 1])[0]) if with_bias else 0)
            check_out(out[n, c:c + 1], out32[n, c:c + 1], np.array([exact]), terms, act)
            # new state: the newest L of the history, as bits
            np.testing.assert_array_equal(state[s, c], np.concatenate([before[s, c, 1:], x[n, c:c + 1]]))
    untouched = [s for s in range(S) if s not in set(idx.tolist())]
    np.testing.assert_array_equal(state[untouched], before[untouched])


@pytest.mark.parametrize("L", [3, 4, 8])
@pytest.mark.parametrize("act", [None, "silu"])
def test_t_steps_equal_full_sequence_convolution(L, act):
    """T successive updates == one causal convolution over concat(state0, x_0..x_{T-1})."""
    rng = np.random.default_rng(40 + L)
    W, N, D, S, T = 4, 6, 9, 16, 7
    idx = rng.choice(S, N, replace=False).astype(np.int32)
    x = rand_bf(rng, (T, N, D))
    w = rand_bf(rng, (D, W))
    state = rand_bf(rng, (S, D, L))
    bias = rand_bf(rng, (D,), 0.1)
    state0 = state.copy()
    outs, outs32 = [], []
    for t in range(T):
        o, o32 = oracle.update(np.ascontiguousarray(x[t]), state, w, bias, act,
                               conv_state_indices=idx, want_f32=True)
        outs.append(o); outs32.append(o32)
    for n, s in enumerate(idx):
        for c in range(D):
            ext = np.concatenate([f64(state0[s, c]), f64(x[:, n, c])])
            full = conv_f64(ext, f64(w[c]))
            b = f64(bias[c:c + 1])[0]
            for t in range(T):
                exact = full[L + t] + b
                terms = np.abs(ext[L + t + 1 - W:L + t + 1]) @ np.abs(f64(w[c])) + abs(b)
                check_out(outs[t][n, c:c + 1], outs32[t][n, c:c + 1], np.array([exact]), terms, act)
            # final state == the last L values of the extended sequence, bit-exact
            ext_bits = np.concatenate([state0[s, c], x[:, n, c]])
            np.testing.assert_array_equal(state[s, c], ext_bits[-L:])


# --------------------------------------------------------------- closed-form pins


@pytest.mark.parametrize("L", [3, 4, 8])
def test_one_hot_tap_is_a_pure_delay(L):
    """weight = e_k gives output history[L+1-W+k]: tap W-1 is the new token, tap k
    looks W-1-k steps back.  Pins the orientation of the taps."""
    rng = np.random.default_rng(L)
    W, N, D = 4, 3, 16
    x = rand_bf(rng, (N, D))
    state = rand_bf(rng, (N, D, L))
    for k in range(W):
        st = state.copy()
        w = np.zeros((D, W), dtype=np.float32); w[:, k] = 1.0
        out = oracle.update(x, st, bf(w), None, None)
        hist = np.concatenate([state, x[:, :, None]], axis=2)  # [N, D, L+1]
        expect = hist[:, :, L + 1 - W + k]
        np.testing.assert_array_equal(f64(out), f64(expect))


@pytest.mark.parametrize("act", [None, "silu"])
def test_zero_weights_give_activated_bias(act):
    rng = np.random.default_rng(3)
    N, D, L = 4, 33, 3
    x = rand_bf(rng, (N, D)); state = rand_bf(rng, (N, D, L)); bias = rand_bf(rng, (D,), 3.0)
    out, o32 = oracle.update(x, state, bf(np.zeros((D, 4))), bias, act, want_f32=True)
    if act is None:
        np.testing.assert_array_equal(out, np.broadcast_to(bias, (N, D)))
    else:
        ref = silu64(f64(bias))
        assert np.all(np.abs(o32 - ref) <= 8 * U32 * np.abs(ref) + 1e-37)


def test_identity_output_scales_exactly_by_two():
    rng = np.random.default_rng(5)
    N, D, L = 4, 40, 4
    x = rand_bf(rng, (N, D)); state = rand_bf(rng, (N, D, L))
    wf = rng.standard_normal((D, 4)).astype(np.float32); bfl = rng.standard_normal(D).astype(np.float32)
    w1, b1 = bf(wf), bf(bfl)
    w2, b2 = bf(f64(w1) * 2), bf(f64(b1) * 2)   # exact doubling of BF16 values
    _, o1 = oracle.update(x, state.copy(), w1, b1, None, want_f32=True)
    _, o2 = oracle.update(x, state.copy(), w2, b2, None, want_f32=True)
    np.testing.assert_array_equal(o2, 2 * o1)


def test_silu_of_zero_is_zero():
    D = 8
    out = oracle.update(bf(np.zeros((1, D))), bf(np.zeros((1, D, 3))), bf(np.ones((D, 4))), None, "silu")
    assert np.all(f64(out) == 0)


# ------------------------------------------------------------------ routing laws


def test_no_table_equals_identity_table():
    rng = np.random.default_rng(11)
    N, D, L, S = 6, 24, 3, 8
    x = rand_bf(rng, (N, D)); w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (S, D, L)); b = rand_bf(rng, (D,), 0.1)
    s1, s2 = st.copy(), st.copy()
    o1 = oracle.update(x, s1, w, b, "silu")
    o2 = oracle.update(x, s2, w, b, "silu", conv_state_indices=np.arange(N, dtype=np.int32))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(s1[N:], st[N:])


def test_row_permutation_permutes_outputs():
    rng = np.random.default_rng(12)
    N, D, L, S = 7, 16, 4, 20
    x = rand_bf(rng, (N, D)); w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (S, D, L))
    idx = np.array([4, -1, 9, 0, -1, 19, 2], dtype=np.int32)
    perm = rng.permutation(N)
    s1, s2 = st.copy(), st.copy()
    o1 = oracle.update(x, s1, w, None, "silu", conv_state_indices=idx)
    o2 = oracle.update(np.ascontiguousarray(x[perm]), s2, w, None, "silu",
                       conv_state_indices=np.ascontiguousarray(idx[perm]))
    np.testing.assert_array_equal(o2, o1[perm])
    np.testing.assert_array_equal(s1, s2)


def test_padding_rows_zero_and_untouched():
    rng = np.random.default_rng(13)
    N, D, L, S = 5, 12, 3, 6
    x = rand_bf(rng, (N, D)); w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (S, D, L))
    idx = np.full(N, -1, dtype=np.int32)
    before = st.copy()
    out = oracle.update(x, st, w, rand_bf(rng, (D,)), "silu", conv_state_indices=idx)
    assert np.all(out == 0)
    np.testing.assert_array_equal(st, before)


@pytest.mark.parametrize("idx,code", [([0, -2], oracle.EINDEX), ([0, 4], oracle.EINDEX),
                                      ([1, 1], oracle.EDUP), ([3, -1, 3], oracle.EDUP)])
def test_invalid_tables_are_refused_before_any_mutation(idx, code):
    rng = np.random.default_rng(14)
    N, D, L, S = len(idx), 8, 3, 4
    x = rand_bf(rng, (N, D)); w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (S, D, L))
    before = st.copy()
    with pytest.raises(oracle.OracleError) as e:
        oracle.update(x, st, w, None, None, conv_state_indices=np.array(idx, dtype=np.int32))
    assert e.value.code == code
    np.testing.assert_array_equal(st, before)


def test_channel_last_strides_equal_compact():
    """The same logical [S, D, L] state stored as physical [S, L, D] gives the same result."""
    rng = np.random.default_rng(15)
    N, D, L, S = 4, 20, 3, 6
    x = rand_bf(rng, (N, D)); w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (S, D, L))
    idx = np.array([5, 0, -1, 2], dtype=np.int32)
    compact = st.copy()
    cl = np.ascontiguousarray(st.transpose(0, 2, 1))  # physical [S, L, D]
    o1 = oracle.update(x, compact, w, None, "silu", conv_state_indices=idx)
    o2 = oracle.update_strided(x, N, D, D, cl, S, L, (L * D, 1, D), w, None, idx, "silu")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(compact, cl.transpose(0, 2, 1))


def test_row_stride_padding_is_never_read():
    rng = np.random.default_rng(16)
    N, D, L, ld = 3, 16, 3, 24
    xp = np.full((N, ld), 0x7FC1, dtype=np.uint16)
    xp[:, :D] = rand_bf(rng, (N, D))
    w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (N, D, L))
    st2 = st.copy()
    out = oracle.update(xp, st, w, None, "silu", d=D, ld=ld)
    assert np.all(np.isfinite(f64(out)))
    # same as the compact copy
    out_c = oracle.update(np.ascontiguousarray(xp[:, :D]), st2, w, None, "silu")
    np.testing.assert_array_equal(out, out_c)
    np.testing.assert_array_equal(st, st2)


# ------------------------------------------------------------- multi-token form


@pytest.mark.parametrize("L", [3, 4, 8])
@pytest.mark.parametrize("act", [None, "silu"])
@pytest.mark.parametrize("x_layout", ["token_major", "channel_major"])
def test_multi_token_equals_full_sequence_convolution(L, act, x_layout):
    """x[N, D, T] applied as T successive steps == one float64 library causal
    convolution over concat(state0, x_0..x_{T-1}); final state bit-exact."""
    rng = np.random.default_rng(60 + L)
    W, N, D, S, T = 4, 5, 11, 9, 6
    idx = np.array([7, -1, 2, 0, -1], dtype=np.int32)
    xt = rand_bf(rng, (N, T, D))                      # token-major values
    if x_layout == "token_major":
        xbuf, xs = np.ascontiguousarray(xt), (T * D, 1, D)
    else:
        xbuf, xs = np.ascontiguousarray(xt.transpose(0, 2, 1)), (D * T, T, 1)
    w = rand_bf(rng, (D, W)); b = rand_bf(rng, (D,), 0.1)
    state = rand_bf(rng, (S, D, L)); state0 = state.copy()
    out, o32 = oracle.update_tokens(xbuf, N, D, T, xs, state, S, L, (D * L, L, 1), w, b, idx, act, want_f32=True)
    for n, s in enumerate(idx):
        if s < 0:
            assert np.all(out[n] == 0)
            continue
        for c in range(D):
            ext = np.concatenate([f64(state0[s, c]), f64(xt[n, :, c])])
            full = conv_f64(ext, f64(w[c]))
            bb = f64(b[c:c + 1])[0]
            for t in range(T):
                terms = np.abs(ext[L + t + 1 - W:L + t + 1]) @ np.abs(f64(w[c])) + abs(bb)
                check_out(out[n, t, c:c + 1], o32[n, t, c:c + 1], np.array([full[L + t] + bb]), terms, act)
            np.testing.assert_array_equal(state[s, c], np.concatenate([state0[s, c], xt[n, :, c]])[-L:])
    untouched = [s for s in range(S) if s not in set(idx.tolist())]
    np.testing.assert_array_equal(state[untouched], state0[untouched])


def test_multi_token_with_one_token_is_the_single_step():
    rng = np.random.default_rng(70)
    N, D, L, S = 4, 24, 4, 6
    x = rand_bf(rng, (N, D)); w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (S, D, L))
    idx = np.array([3, 0, -1, 5], dtype=np.int32)
    s1, s2 = st.copy(), st.copy()
    o1 = oracle.update(x, s1, w, None, "silu", conv_state_indices=idx)
    o2 = oracle.update_tokens(x, N, D, 1, (D, 1, 0), s2, S, L, (D * L, L, 1), w, None, idx, "silu")
    np.testing.assert_array_equal(o2[:, 0, :], o1)
    np.testing.assert_array_equal(s1, s2)


def test_multi_token_longer_than_history_keeps_last_tokens():
    """T > L: the state ends as the last L tokens, bit for bit."""
    rng = np.random.default_rng(71)
    N, D, L, T = 2, 8, 3, 9
    xt = rand_bf(rng, (N, T, D)); w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (N, D, L))
    oracle.update_tokens(np.ascontiguousarray(xt), N, D, T, (T * D, 1, D), st, N, L, (D * L, L, 1), w, None, None, None)
    np.testing.assert_array_equal(st, xt[:, T - L:, :].transpose(0, 2, 1))
