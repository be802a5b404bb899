"""GPU parity at offsets past 2^31 elements and 4 GiB.

The operands of a real decode cache are large: a slot pool of many sequences, or
x rows inside a bigger activation buffer, puts slots and rows gigabytes apart.
These cases place the selected state slots and the x rows of each entry point at
element offsets past 2^31 (byte offsets past 4 GiB) inside one large device
buffer, so that any offset formed in 32 bits would land on another slot or row
(the guard bands and the untouched regions would then change) or outside the
buffer.  Only the regions a call may touch are written and read back; the oracle
runs on compact host copies of them (slots are independent, so the result is the
same), and the bar is the usual one: state bit-exact, outputs within 1 BF16 ulp or
1e-2 * max(1, |ref|) of the FP32 oracle (exact for identity), padding rows zero.

Semantics: cuDNN FE-OSS page "Causal Conv1d Decode Update", sections "Causal
Conv1d Decode Update" (update rule, routing, padding, cache_seqlens) and
"Semantic tensor contract" (layouts, row stride, the multi-token form).
"""
import numpy as np
import pytest
import torch

import oracle
import depthwise_causal_conv1d_amd as dc
from depthwise_causal_conv1d_amd import workloads as wl
from parity import GUARD, assert_outputs_match, from_dev, to_dev, takes_narrow

pytestmark = pytest.mark.gpu

# Slot stride (elements): slot 1 starts at byte 2^32 + 16, so a 32-bit byte
# offset would wrap onto slot 0's first vector.
SLOT_STRIDE = (1 << 31) + 8
# x row stride (elements): row 2 starts at byte 2^32 + 32.
ROW_STRIDE = (1 << 30) + 8
# Routing used throughout: row 0 -> slot 1 (past 4 GiB), row 1 padding, row 2
# (past 4 GiB in x) -> slot 0.
INDICES = np.array([1, -1, 0], np.int32)


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dc._load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _bf(rng, shape, scale=1.0):
    return wl.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(scale))


class SparseBuffer:
    """A large device buffer of which only some regions are written: each region
    is surrounded by GUARD sentinel elements, and only regions and guards are
    ever read back."""

    def __init__(self, elems):
        # room for the guard band above the last region
        self.t = torch.empty(elems + GUARD, dtype=torch.bfloat16, device="cuda")
        self.regions = []

    def put(self, off, bits):
        flat = np.ascontiguousarray(bits).ravel()
        host = np.full(flat.size + 2 * GUARD, wl.FILL_SENTINEL, np.uint16)
        host[GUARD:GUARD + flat.size] = flat
        lo = max(off - GUARD, 0)
        self.t[lo:off + flat.size + GUARD] = to_dev(host[GUARD - (off - lo):])
        self.regions.append((off, flat.size))

    def get(self, off, n):
        return from_dev(self.t[off:off + n])

    def assert_guards(self):
        for off, n in self.regions:
            below = from_dev(self.t[max(off - GUARD, 0):off])
            above = from_dev(self.t[off + n:off + n + GUARD])
            assert np.all(below == wl.FILL_SENTINEL), f"write below the region at {off}"
            assert np.all(above == wl.FILL_SENTINEL), f"write above the region at {off}"


def _slot_layout(logical, layout):
    """[D, L] logical values of one slot -> the bits stored at its base."""
    return logical if layout == "compact" else np.ascontiguousarray(logical.T)


def _slot_logical(bits, D, L, layout):
    return bits.reshape(D, L) if layout == "compact" else bits.reshape(L, D).T


def _state_buffer(state_logical, layout):
    S, D, L = state_logical.shape
    buf = SparseBuffer((S - 1) * SLOT_STRIDE + D * L)
    for k in range(S):
        buf.put(k * SLOT_STRIDE, _slot_layout(state_logical[k], layout))
    view = (buf.t.as_strided((S, D, L), (SLOT_STRIDE, L, 1)) if layout == "compact"
            else buf.t.as_strided((S, D, L), (SLOT_STRIDE, 1, D)))
    return buf, view


def _check_state(buf, ref_state, layout):
    S, D, L = ref_state.shape
    for k in range(S):
        got = _slot_logical(buf.get(k * SLOT_STRIDE, D * L), D, L, layout)
        np.testing.assert_array_equal(got, ref_state[k], err_msg=f"slot {k} not bit-exact")
    buf.assert_guards()


def _x_rows(x_rows):
    """x rows [N, D] placed ROW_STRIDE apart; returns the buffer and an [N, D] view."""
    N, D = x_rows.shape
    buf = SparseBuffer((N - 1) * ROW_STRIDE + D)
    for r in range(N):
        buf.put(r * ROW_STRIDE, x_rows[r])
    return buf, buf.t.as_strided((N, D), (ROW_STRIDE, 1))


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
@pytest.mark.parametrize("L,act", [(3, "silu"), (4, None)])
@pytest.mark.parametrize("D", [1032, 87560])
def test_update_past_4gib(layout, L, act, D):
    # D = 1032: two full 512-channel tiles and a ragged 8-channel tile (three
    # rows of it take the narrow form); D = 87560: 171 full tiles and a ragged
    # one, which three rows take in the 512-channel kernels
    rng = np.random.default_rng(700 + L)
    N, S = 3, 2
    x = _bf(rng, (N, D))
    w = _bf(rng, (D, 4))
    b = _bf(rng, (D,), 0.1)
    state = _bf(rng, (S, D, L))
    ref_state = state.copy()
    ref, ref32 = oracle.update(x, ref_state, w, b, act, conv_state_indices=INDICES, want_f32=True)

    sbuf, sview = _state_buffer(state, layout)
    xbuf, xview = _x_rows(x)
    out = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    dc.causal_conv1d_update_out(xview, sview, to_dev(w), to_dev(b), act, out=out,
                                conv_state_indices=torch.from_numpy(INDICES).cuda(), dev_status=status)
    kernel = dc.dcconv_last_kernel()
    torch.cuda.synchronize()
    assert ("update_narrow" if takes_narrow(N, D) else "_v8") in kernel, kernel
    assert takes_narrow(N, D) == (D == 1032)
    assert int(status.item()) == 0
    assert_outputs_match(from_dev(out), ref, ref32, exact=act is None)
    _check_state(sbuf, ref_state, layout)
    xbuf.assert_guards()
    for r in range(N):
        np.testing.assert_array_equal(xbuf.get(r * ROW_STRIDE, D), x[r], err_msg="x was written")


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
def test_ring_update_past_4gib(layout):
    rng = np.random.default_rng(710)
    N, D, S, L = 3, 1032, 2, 3
    x = _bf(rng, (N, D))
    w = _bf(rng, (D, 4))
    state = _bf(rng, (S, D, L))
    seen = rng.integers(0, 50, size=N).astype(np.int32)
    ref_state = state.copy()
    ref, ref32 = oracle.update_ring(x, N, D, D, ref_state, S, L, (D * L, L, 1), w, None, INDICES, seen, "silu",
                                    want_f32=True)

    sbuf, sview = _state_buffer(state, layout)
    xbuf, xview = _x_rows(x)
    out = torch.empty(N, D, dtype=torch.bfloat16, device="cuda")
    dc.causal_conv1d_update_out(xview, sview, to_dev(w), None, "silu", out=out,
                                conv_state_indices=torch.from_numpy(INDICES).cuda(),
                                cache_seqlens=torch.from_numpy(seen).cuda())
    kernel = dc.dcconv_last_kernel()
    torch.cuda.synchronize()
    if layout == "channel_last":
        assert "_v8" in kernel, kernel
    assert_outputs_match(from_dev(out), ref, ref32)
    _check_state(sbuf, ref_state, layout)
    xbuf.assert_guards()


@pytest.mark.parametrize("layout", ["compact", "channel_last"])
@pytest.mark.parametrize("T", [5, 16])
def test_tokens_past_4gib(layout, T):
    rng = np.random.default_rng(720 + T)
    N, D, S, L = 3, 1032, 2, 4
    xt = _bf(rng, (N, T, D))                      # token-major rows
    w = _bf(rng, (D, 4))
    b = _bf(rng, (D,), 0.1)
    state = _bf(rng, (S, D, L))
    ref_state = state.copy()
    ref, ref32 = oracle.update_tokens(xt, N, D, T, (T * D, 1, D), ref_state, S, L, (D * L, L, 1), w, b, INDICES,
                                      "silu", want_f32=True)

    sbuf, sview = _state_buffer(state, layout)
    xbuf = SparseBuffer((N - 1) * ROW_STRIDE + T * D)
    for r in range(N):
        xbuf.put(r * ROW_STRIDE, xt[r])
    xview = xbuf.t.as_strided((N, D, T), (ROW_STRIDE, 1, D))
    out = dc.causal_conv1d_update_tokens(xview, sview, to_dev(w), to_dev(b), "silu",
                                         conv_state_indices=torch.from_numpy(INDICES).cuda())
    kernel = dc.dcconv_last_kernel()
    torch.cuda.synchronize()
    assert "tokens_v8" in kernel, kernel
    got = from_dev(out.permute(0, 2, 1))        # [N, T, D]
    assert_outputs_match(got, ref, ref32)
    assert np.all(got[1] == 0), "padding row not zero"
    _check_state(sbuf, ref_state, layout)
    xbuf.assert_guards()


@pytest.mark.parametrize("layout,D,T,form", [("channel_last", 1032, 40, "prefill_sweep_v8"),
                                             ("compact", 1032, 40, "prefill_sweep_v8"),
                                             ("channel_last", 8192, 3000, "prefill_v8<")])
def test_prefill_past_4gib(layout, D, T, form):
    rng = np.random.default_rng(730 + T)
    N, S, L = 3, 2, 3
    xt = _bf(rng, (N, T, D))
    w = wl.f32_to_bf16_bits(rng.uniform(-0.5, 0.5, (D, 4)).astype(np.float32))
    state = _bf(rng, (S, D, L))
    has_init = np.array([1, 0, 1], np.uint8)
    ref_state = state.copy()
    ref, ref32 = oracle.prefill(xt, N, D, T, (T * D, 1, D), w, None, "silu", state_buf=ref_state, S=S, L=L,
                                state_strides=(D * L, L, 1), indices=INDICES, has_init=has_init, want_f32=True)

    sbuf, sview = _state_buffer(state, layout)
    xbuf = SparseBuffer((N - 1) * ROW_STRIDE + T * D)
    for r in range(N):
        xbuf.put(r * ROW_STRIDE, xt[r])
    xview = xbuf.t.as_strided((N, D, T), (ROW_STRIDE, 1, D))
    out = dc.causal_conv1d(xview, to_dev(w), None, "silu", conv_state=sview,
                           conv_state_indices=torch.from_numpy(INDICES).cuda(),
                           has_initial_state=torch.from_numpy(has_init).cuda())
    kernel = dc.dcconv_last_kernel()
    torch.cuda.synchronize()
    assert kernel.startswith(form), kernel
    got = from_dev(out.permute(0, 2, 1))
    assert_outputs_match(got, ref, ref32)
    assert np.all(got[1] == 0), "padding sequence not zero"
    _check_state(sbuf, ref_state, layout)
    xbuf.assert_guards()
