"""GPU parity when a launch holds more work units than blocks.

Every kernel is launched with min(units, 2^20) blocks and strides over its units
by 2^20, so a call with more than 2^20 units runs some blocks more than once.
These cases make each kernel family cross that line (millions of narrow rows or
sequences) and compare the whole result with the CPU oracle under the usual
bar: state bit-exact, outputs within 1 BF16 ulp or 1e-2 * max(1, |ref|) of the
FP32 oracle, guard bands intact.

Semantics: cuDNN FE-OSS page "Causal Conv1d Decode Update", sections "Causal
Conv1d Decode Update" (update rule, routing, cache_seqlens) and "Semantic tensor
contract" (layouts, the multi-token form); the prefill is the whole-sequence form
the page names at its top.
"""
import numpy as np
import pytest
import torch

import depthwise_causal_conv1d_amd as dc
from depthwise_causal_conv1d_amd import workloads as wl
from parity import assert_guards_intact, assert_outputs_match, from_dev, guarded_copy, guarded_empty, to_dev
from test_gpu_prefill import PrefillCase
from test_gpu_ring import RingCase, _ring_tokens_reference
from test_gpu_tokens import TokensCase
from test_gpu_update import make_case

pytestmark = pytest.mark.gpu

GRID_CAP = 1 << 20
# Vector kernels: one 512-channel tile at D = 8 and two waves of one or two
# rows per block, so at least 2^20 + 256 block units; the scalar kernels: one
# row per unit at D < 256.
ROWS_V8 = 4 * GRID_CAP + 1024
ROWS_SCALAR = GRID_CAP + 7


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dc._load()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layout,L,N,D,kernel", [("compact", 3, ROWS_V8, 8, "update_compact_v8<L=3,silu,R="),
                                                 ("channel_last", 4, ROWS_V8, 8, "update_channel_last_v8<L=4,silu,R="),
                                                 ("compact", 3, ROWS_SCALAR, 7, "update_scalar<silu>")])
def test_update_more_units_than_blocks(layout, L, N, D, kernel):
    case = make_case(5000 + L, N=N, D=D, L=L, layout=layout, bias=True)
    case.check()
    assert case.kernel.startswith(kernel), case.kernel


@pytest.mark.parametrize("N,D,kernel", [(ROWS_V8, 8, "update_ring_v8<silu,R="),
                                        (ROWS_SCALAR, 7, "update_ring_scalar<silu>")])
def test_ring_more_units_than_blocks(N, D, kernel):
    case = RingCase(5100 + D, N, D, 3, max_seen=1000)
    case.check()
    assert case.kernel.startswith(kernel), case.kernel


@pytest.mark.parametrize("N,D,layout,kernel", [(ROWS_V8, 8, "compact", "tokens_v8<L=3,silu,compact,R=2>"),
                                               (ROWS_SCALAR, 7, "compact", "tokens_scalar<silu>")])
def test_tokens_more_units_than_blocks(N, D, layout, kernel):
    case = TokensCase(5200 + D, N, D, 2, 3, layout=layout, bias=True)
    case.check()
    assert case.kernel == kernel, case.kernel


def test_ring_tokens_more_units_than_blocks():
    rng = np.random.default_rng(5300)
    N, D, T, L = ROWS_V8, 8, 2, 3
    bf = lambda shape: wl.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
    x, w, st = bf((N, T, D)), bf((D, 4)), bf((N, D, L))
    seen = rng.integers(0, 1000, size=N).astype(np.int32)
    ref_state = st.copy()
    ref, ref32 = _ring_tokens_reference(x, ref_state, w, None, None, seen, "silu")
    sb, sd = guarded_copy(np.ascontiguousarray(st.transpose(0, 2, 1)))
    ob, od = guarded_empty((N * T * D,))
    out = torch.as_strided(od, (N, D, T), (T * D, 1, D))
    dc.causal_conv1d_update_tokens(to_dev(x).permute(0, 2, 1), sd.permute(0, 2, 1), to_dev(w), None, "silu",
                                   cache_seqlens=torch.from_numpy(seen).cuda(), out=out)
    kernel = dc.dcconv_last_kernel()
    torch.cuda.synchronize()
    assert kernel == "tokens_ring_v8<silu,R=2>", kernel
    assert_guards_intact(sb)
    assert_guards_intact(ob)
    np.testing.assert_array_equal(from_dev(sd).transpose(0, 2, 1), ref_state, err_msg="ring not bit-exact")
    assert_outputs_match(from_dev(out.permute(0, 2, 1)), ref, ref32)


@pytest.mark.parametrize("N,D,kernel", [(ROWS_V8, 8, "prefill_v8<L=3,silu,compact>"),
                                        (ROWS_SCALAR, 7, "prefill_scalar<silu>")])
def test_prefill_more_units_than_blocks(N, D, kernel):
    # as many sequences as rows above: the edge and chunk roles together hold
    # more than 2^20 blocks, which also keeps the narrow rows off the sweep form
    case = PrefillCase(5400 + D, D, N=N, T=4, L=3, state="compact", has_init="mixed", bias=True)
    case.check()
    assert case.kernel == kernel, case.kernel
