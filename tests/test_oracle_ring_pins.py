"""Pins of the oracle's circular-buffer decode step (``cache_seqlens``).

The cuDNN FE-OSS page "Causal Conv1d Decode Update" reserves ``cache_seqlens`` for
circular-buffer state and fixes nothing else (section "Causal Conv1d Decode
Update").  The reading: a slot that has seen c tokens keeps token i at position
i mod L; the step's history is the same as the shifting update's, so the ring
step must agree with the shifting update on every output, with the ring rotated
by c.  Pinned against:

* hand-worked examples (``tests/golden/ring_hand_examples.json``);
* the oracle's shifting update over many steps (a different formulation):
  outputs bit for bit, and ring[(c + k) mod L] == linear[k] after every step;
* one-hot taps (a pure delay through the ring); refusals before mutation.
"""
import json
import os

import numpy as np
import pytest

import oracle
from test_oracle_pins import GOLDEN, bf, rand_bf


def _golden():
    with open(os.path.join(GOLDEN, "ring_hand_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    st = bf(case["state"]); S, D, L = st.shape
    x = bf(case["x"]); w = bf(case["weight"])
    b = None if case["bias"] is None else bf(case["bias"])
    idx = None if case["indices"] is None else np.array(case["indices"], np.int32)
    cs = np.array(case["cache_seqlens"], np.int32)
    out = oracle.update_ring(x, x.shape[0], D, D, st, S, L, (D * L, L, 1), w, b, idx, cs, case["activation"])
    np.testing.assert_array_equal(out, bf(case["expected_out"]))
    np.testing.assert_array_equal(st, bf(case["expected_state"]))


@pytest.mark.parametrize("L", [3, 4, 5, 8])
@pytest.mark.parametrize("act", [None, "silu"])
def test_ring_equals_shifting_update_over_many_steps(L, act):
    rng = np.random.default_rng(400 + L)
    N, D, S, T = 5, 7, 9, 13
    idx = np.array([8, 2, -1, 0, 5], np.int32)
    w = rand_bf(rng, (D, 4)); b = rand_bf(rng, (D,), 0.1)
    lin = rand_bf(rng, (S, D, L))
    c = rng.integers(0, 50, size=N).astype(np.int32)
    # the ring holding the same history: token c-L+k (= linear position k) at (c + k) mod L
    ring = lin.copy()
    for n, s in enumerate(idx):
        if s >= 0:
            for k in range(L):
                ring[s, :, (c[n] + k) % L] = lin[s, :, k]
    ring0 = ring.copy()
    for t in range(T):
        x = rand_bf(rng, (N, D))
        o_lin = oracle.update(x, lin, w, b, act, conv_state_indices=idx)
        o_ring = oracle.update_ring(x, N, D, D, ring, S, L, (D * L, L, 1), w, b, idx, c, act)
        np.testing.assert_array_equal(o_ring, o_lin)
        c = c + 1
        for n, s in enumerate(idx):
            if s >= 0:
                for k in range(L):
                    np.testing.assert_array_equal(ring[s, :, (c[n] + k) % L], lin[s, :, k])
    untouched = [s for s in range(S) if s not in set(idx.tolist())]
    np.testing.assert_array_equal(ring[untouched], ring0[untouched])


@pytest.mark.parametrize("k", [0, 1, 2, 3])
def test_one_hot_tap_reads_the_token_k_places_back(k):
    """weight = e_k: the output is token c-(3-k), read at position (c-3+k) mod L
    (the new token itself for k = 3)."""
    rng = np.random.default_rng(410 + k)
    N, D, L = 4, 6, 5
    st = rand_bf(rng, (N, D, L)); st0 = st.copy()
    x = rand_bf(rng, (N, D))
    w = np.zeros((D, 4), np.uint16); w[:, k] = bf(1.0)
    c = np.array([0, 3, 7, 12], np.int32)
    out = oracle.update_ring(x, N, D, D, st, N, L, (D * L, L, 1), w, None, None, c, None)
    for n in range(N):
        want = x[n] if k == 3 else st0[n, :, (c[n] - 3 + k) % L]
        np.testing.assert_array_equal(out[n], want)
        # only position c mod L changed
        changed = np.flatnonzero(np.any(st[n] != st0[n], axis=0))
        assert set(changed.tolist()) <= {c[n] % L}
        np.testing.assert_array_equal(st[n, :, c[n] % L], x[n])


def test_channel_last_ring_equals_compact_ring():
    rng = np.random.default_rng(420)
    N, D, L = 3, 16, 4
    st = rand_bf(rng, (N, D, L)); x = rand_bf(rng, (N, D)); w = rand_bf(rng, (D, 4))
    c = np.array([2, 9, 4], np.int32)
    s1 = st.copy(); s2 = np.ascontiguousarray(st.transpose(0, 2, 1))
    o1 = oracle.update_ring(x, N, D, D, s1, N, L, (D * L, L, 1), w, None, None, c, "silu")
    o2 = oracle.update_ring(x, N, D, D, s2, N, L, (L * D, 1, D), w, None, None, c, "silu")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2.transpose(0, 2, 1))


@pytest.mark.parametrize("idx,cs,code", [([0, 1], [3, -1], oracle.EARGS), ([0, 0], [1, 1], oracle.EDUP),
                                         ([0, 7], [1, 1], oracle.EINDEX)])
def test_refusals_before_any_mutation(idx, cs, code):
    rng = np.random.default_rng(430)
    st = rand_bf(rng, (4, 8, 3)); st0 = st.copy()
    with pytest.raises(oracle.OracleError) as e:
        oracle.update_ring(rand_bf(rng, (2, 8)), 2, 8, 8, st, 4, 3, (24, 3, 1), rand_bf(rng, (8, 4)), None,
                           np.array(idx, np.int32), np.array(cs, np.int32), None)
    assert e.value.code == code
    np.testing.assert_array_equal(st, st0)
