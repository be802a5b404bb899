"""Pins of the oracle's full-sequence causal convolution (prefill).

The prefill is the operation the cuDNN FE-OSS page "Causal Conv1d Decode Update"
points to at its top for full sequences, whose final state the decode update
continues.  Its own page is not among the sources, so the oracle takes the
plainest reading the decode page supports (a causal convolution over the
initial state, or zeros, followed by the tokens; the final state is the newest
L values).  It is pinned here against things other than itself:

* hand-worked examples (``tests/golden/prefill_hand_examples.json``);
* a float64 library convolution (``numpy.convolve``) over varlen sequences of
  lengths 0, 1, 2, ... with and without initial states; final states bit-exact;
* the oracle's decode update applied token by token (a different formulation
  of the same result), bit for bit;
* one-hot taps (a pure delay), stateless == zero initial state, batch form ==
  varlen form, strided layouts == contiguous ones, refusals before mutation.
"""
import json
import os

import numpy as np
import pytest

import oracle
from test_oracle_pins import GOLDEN, bf, check_out, conv_f64, f64, rand_bf


def _golden():
    with open(os.path.join(GOLDEN, "prefill_hand_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    L = case["L"]
    x = bf(case["x"])
    w = bf(case["weight"])
    D = w.shape[0]
    b = None if case["bias"] is None else bf(case["bias"])
    state = bf(case["state"])
    S = state.shape[0]
    idx = None if case["indices"] is None else np.array(case["indices"], np.int32)
    hi = None if case["has_init"] is None else np.array(case["has_init"], np.uint8)
    starts = None if case["starts"] is None else np.array(case["starts"], np.int32)
    t = case["t"]
    xs = (t * D, 1, D) if starts is None else (0, 1, D)
    out = oracle.prefill(x, case["n"], D, t, xs, w, b, case["activation"], starts=starts, state_buf=state, S=S, L=L,
                         state_strides=(D * L, L, 1), indices=idx, has_init=hi)
    np.testing.assert_array_equal(out, bf(case["expected_out"]))
    np.testing.assert_array_equal(state, bf(case["expected_state"]))


@pytest.mark.parametrize("L", [3, 4, 8])
@pytest.mark.parametrize("act", [None, "silu"])
def test_varlen_vs_f64_convolution(L, act):
    rng = np.random.default_rng(300 + L)
    W, D, S = 4, 5, 12
    lens = [0, 1, 2, 3, 5, 17, 4]
    n = len(lens)
    starts = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t = int(starts[-1])
    x = rand_bf(rng, (t, D))
    w = rand_bf(rng, (D, W)); b = rand_bf(rng, (D,), 0.1)
    state = rand_bf(rng, (S, D, L)); state0 = state.copy()
    idx = rng.choice(S, n, replace=False).astype(np.int32)
    hi = np.array([1, 0, 1, 1, 0, 1, 0], np.uint8)
    out, o32 = oracle.prefill(x, n, D, t, (0, 1, D), w, b, act, starts=starts, state_buf=state, S=S, L=L,
                              state_strides=(D * L, L, 1), indices=idx, has_init=hi, want_f32=True)
    for i in range(n):
        a, e = starts[i], starts[i + 1]
        s = idx[i]
        for c in range(D):
            init_bits = state0[s, c] if hi[i] else np.zeros(L, np.uint16)
            ext = np.concatenate([f64(init_bits), f64(x[a:e, c])])
            full = conv_f64(ext, f64(w[c]))
            bb = f64(b[c:c + 1])[0]
            for j in range(e - a):
                terms = np.abs(ext[L + j + 1 - W:L + j + 1]) @ np.abs(f64(w[c])) + abs(bb)
                check_out(out[a + j, c:c + 1], o32[a + j, c:c + 1], np.array([full[L + j] + bb]), terms, act)
            np.testing.assert_array_equal(state[s, c], np.concatenate([init_bits, x[a:e, c]])[-L:])
    untouched = [s for s in range(S) if s not in set(idx.tolist())]
    np.testing.assert_array_equal(state[untouched], state0[untouched])


@pytest.mark.parametrize("L", [3, 5, 8])
def test_prefill_from_state_equals_decode_steps(L):
    """Continuing from the slot's state == the decode update applied to the tokens
    one at a time (two formulations), bit for bit, outputs and final state."""
    rng = np.random.default_rng(320 + L)
    N, D, T, S = 4, 9, 11, 7
    xt = rand_bf(rng, (N, T, D)); w = rand_bf(rng, (D, 4)); b = rand_bf(rng, (D,), 0.1)
    st = rand_bf(rng, (S, D, L))
    idx = np.array([6, -1, 0, 3], np.int32)
    s1, s2 = st.copy(), st.copy()
    o1 = oracle.prefill(np.ascontiguousarray(xt), N, D, T, (T * D, 1, D), w, b, "silu", state_buf=s1, S=S, L=L,
                        state_strides=(D * L, L, 1), indices=idx, has_init=np.ones(N, np.uint8))
    o2 = np.stack([oracle.update(np.ascontiguousarray(xt[:, j]), s2, w, b, "silu", conv_state_indices=idx)
                   for j in range(T)], 1)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_zero_initial_state_equals_stateless_and_zeroed_slots():
    rng = np.random.default_rng(330)
    N, D, T, L = 3, 6, 8, 4
    xt = rand_bf(rng, (N, T, D)); w = rand_bf(rng, (D, 4))
    xb = np.ascontiguousarray(xt)
    stateless = oracle.prefill(xb, N, D, T, (T * D, 1, D), w, None, "silu")
    st = rand_bf(rng, (N, D, L))
    fresh = oracle.prefill(xb, N, D, T, (T * D, 1, D), w, None, "silu", state_buf=st, S=N, L=L,
                           state_strides=(D * L, L, 1))
    zst = np.zeros((N, D, L), np.uint16)
    zeroed = oracle.prefill(xb, N, D, T, (T * D, 1, D), w, None, "silu", state_buf=zst, S=N, L=L,
                            state_strides=(D * L, L, 1), has_init=np.ones(N, np.uint8))
    np.testing.assert_array_equal(stateless, fresh)
    np.testing.assert_array_equal(stateless, zeroed)
    np.testing.assert_array_equal(st, zst)                       # same final states
    np.testing.assert_array_equal(st, xt[:, T - L:, :].transpose(0, 2, 1))


@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_one_hot_tap_is_a_delay(k):
    """weight = e_k: out[j] = ext[L + j - (W-1-k)], i.e. the token W-1-k places back
    (the initial state's values before the sequence start)."""
    rng = np.random.default_rng(340 + k)
    D, T, L = 4, 6, 3
    xt = rand_bf(rng, (1, T, D)); st = rand_bf(rng, (1, D, L)); st0 = st.copy()
    w = np.zeros((D, 4), np.uint16); w[:, k] = bf(1.0)
    out = oracle.prefill(np.ascontiguousarray(xt), 1, D, T, (T * D, 1, D), w, None, None, state_buf=st, S=1, L=L,
                         state_strides=(D * L, L, 1), has_init=np.ones(1, np.uint8))
    ext = np.concatenate([st0[0].T, xt[0]], 0)  # [L + T, D]
    np.testing.assert_array_equal(out[0], ext[L - (3 - k):L - (3 - k) + T])


def test_batch_form_equals_varlen_form():
    rng = np.random.default_rng(350)
    N, D, T, L = 3, 7, 5, 3
    xt = rand_bf(rng, (N, T, D)); w = rand_bf(rng, (D, 4)); b = rand_bf(rng, (D,), 0.1)
    st = rand_bf(rng, (N, D, L)); s1, s2 = st.copy(), st.copy()
    hi = np.array([1, 0, 1], np.uint8)
    o1 = oracle.prefill(np.ascontiguousarray(xt), N, D, T, (T * D, 1, D), w, b, None, state_buf=s1, S=N, L=L,
                        state_strides=(D * L, L, 1), has_init=hi)
    starts = (np.arange(N + 1) * T).astype(np.int32)
    o2 = oracle.prefill(np.ascontiguousarray(xt.reshape(N * T, D)), N, D, N * T, (0, 1, D), w, b, None,
                        starts=starts, state_buf=s2, S=N, L=L, state_strides=(D * L, L, 1), has_init=hi)
    np.testing.assert_array_equal(o1.reshape(N * T, D), o2)
    np.testing.assert_array_equal(s1, s2)


def test_channel_major_x_and_channel_last_state_equal_contiguous():
    rng = np.random.default_rng(360)
    N, D, T, L = 2, 10, 6, 4
    xt = rand_bf(rng, (N, T, D)); w = rand_bf(rng, (D, 4))
    st = rand_bf(rng, (N, D, L))
    hi = np.ones(N, np.uint8)
    s_c = st.copy()
    o_c = oracle.prefill(np.ascontiguousarray(xt), N, D, T, (T * D, 1, D), w, None, "silu", state_buf=s_c, S=N, L=L,
                         state_strides=(D * L, L, 1), has_init=hi)
    s_l = np.ascontiguousarray(st.transpose(0, 2, 1))              # physical [S, L, D]
    o_l = oracle.prefill(np.ascontiguousarray(xt.transpose(0, 2, 1)), N, D, T, (D * T, T, 1), w, None, "silu",
                         state_buf=s_l, S=N, L=L, state_strides=(L * D, 1, D), has_init=hi)
    np.testing.assert_array_equal(o_c, o_l)
    np.testing.assert_array_equal(s_c, s_l.transpose(0, 2, 1))


@pytest.mark.parametrize("starts,idx,code", [
    ([1, 2, 4], [0, 1], oracle.EARGS),     # does not start at 0
    ([0, 3, 2], [0, 1], oracle.EARGS),     # decreasing
    ([0, 2, 3], [0, 1], oracle.EARGS),     # does not end at t
    ([0, 2, 4], [0, 0], oracle.EDUP),
    ([0, 2, 4], [0, 5], oracle.EINDEX),
])
def test_refusals_before_any_mutation(starts, idx, code):
    rng = np.random.default_rng(370)
    D, L, S = 3, 3, 4
    x = rand_bf(rng, (4, D)); w = rand_bf(rng, (D, 4)); st = rand_bf(rng, (S, D, L)); st0 = st.copy()
    with pytest.raises(oracle.OracleError) as e:
        oracle.prefill(x, 2, D, 4, (0, 1, D), w, None, None, starts=np.array(starts, np.int32), state_buf=st, S=S,
                       L=L, state_strides=(D * L, L, 1), indices=np.array(idx, np.int32),
                       has_init=np.ones(2, np.uint8))
    assert e.value.code == code
    np.testing.assert_array_equal(st, st0)
