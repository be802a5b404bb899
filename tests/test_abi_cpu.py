"""C-ABI checks that need no GPU: the library loads, exports every function that
include/dcconv.h declares, and refuses every malformed or unserved request on the
host before anything reaches the HIP runtime.

The refusals follow the cuDNN FE-OSS page "Causal Conv1d Decode Update": section
"Semantic tensor contract" (x row-stride rule, L >= W-1) and section "Current
native implementation" (W = 4, 16-byte alignment, cache_seqlens must be None).

The raw-pointer tests pass made-up (never dereferenced) device addresses, so they
only run where no GPU is visible; the GPU suite repeats the refusals on real
tensors.
"""
import ctypes
import os
import re

import pytest
import torch

import depthwise_causal_conv1d_amd as dc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dcconv.h")

no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="made-up pointers are only passed where no GPU exists")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dcconv_\w+)\s*\(", text)))


def _header_constants():
    text = open(HEADER).read()
    consts = dict(re.findall(r"\b(DCCONV_[A-Z_]+)\s*=\s*(\d+)", text))
    consts.update(re.findall(r"#define\s+(DCCONV_[A-Z_]+)\s+(\d+)", text))
    return {k: int(v) for k, v in consts.items()}


@pytest.fixture(scope="module")
def lib():
    return dc._load()


def test_library_exports_every_declared_function(lib):
    declared = _declared()
    assert {"dcconv_update", "dcconv_abi_version", "dcconv_last_error", "dcconv_last_kernel"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in dcconv.h but not exported"


def test_abi_version_and_constants_match_header(lib):
    c = _header_constants()
    assert dc.dcconv_abi_version() == c["DCCONV_ABI_VERSION"]
    for k, v in c.items():
        if k == "DCCONV_ABI_VERSION" or k == "DCCONV_H":
            continue
        assert getattr(dc, k) == v, k


def test_binding_names_match_c_names():
    for name in _declared():
        assert callable(getattr(dc, name)), name


# made-up, 16-byte aligned, far apart device addresses (never dereferenced)
X, ST, WT, BI, IX, OUT, STAT = (0x10000000 * (k + 1) for k in range(7))


def _args(**over):
    a = dict(x=X, n=4, d=64, ld_x=64, conv_state=ST, s=4, l=3, st_s=192, st_d=3, st_l=1,
             weight=WT, w=4, bias=None, conv_state_indices=None, cache_seqlens=None,
             activation=0, out=OUT, dev_status=None, stream=None)
    a.update(over)
    return a


def _call(**over):
    a = _args(**over)
    return dc.dcconv_update(**a)


DECLINES = [
    # (overrides, expected code, message fragment)
    (dict(n=-1), dc.DCCONV_EINVAL, "n (decode rows)"),
    (dict(d=0), dc.DCCONV_EINVAL, "d (channels)"),
    (dict(s=-1), dc.DCCONV_EINVAL, "s (state slots)"),
    (dict(w=0), dc.DCCONV_EINVAL, "filter width"),
    (dict(l=2, st_d=2, st_s=128), dc.DCCONV_EINVAL, "must be >= w-1"),
    (dict(ld_x=63), dc.DCCONV_EINVAL, "smaller than d"),
    (dict(ld_x=70), dc.DCCONV_EINVAL, "ld_x % 8 == 0"),
    (dict(activation=2), dc.DCCONV_EINVAL, "activation"),
    (dict(st_d=-3), dc.DCCONV_EINVAL, "non-negative"),
    (dict(cache_seqlens=IX + 2), dc.DCCONV_EINVAL, "cache_seqlens must be 4-byte aligned"),
    (dict(ld_x=1 << 50), dc.DCCONV_EINVAL, "2^47 bytes"),
    (dict(st_s=1 << 50), dc.DCCONV_EINVAL, "2^47 bytes"),
    (dict(st_s=(1 << 62) + 8), dc.DCCONV_EINVAL, "2^47 bytes"),
    (dict(cache_seqlens=OUT + 64), dc.DCCONV_EINVAL, "overlaps cache_seqlens"),
    (dict(w=3), dc.DCCONV_EUNSUPPORTED, "w=4"),
    (dict(w=5, l=4, st_d=4, st_s=256), dc.DCCONV_EUNSUPPORTED, "w=4"),
    (dict(st_s=192, st_d=1, st_l=2), dc.DCCONV_EUNSUPPORTED, "neither compact"),
    (dict(st_s=100), dc.DCCONV_EUNSUPPORTED, "neither compact"),
    (dict(x=None), dc.DCCONV_EINVAL, "non-NULL"),
    (dict(conv_state=None), dc.DCCONV_EINVAL, "non-NULL"),
    (dict(weight=None), dc.DCCONV_EINVAL, "non-NULL"),
    (dict(out=None), dc.DCCONV_EINVAL, "non-NULL"),
    (dict(s=3), dc.DCCONV_EINVAL, "must be >= n"),
    (dict(x=X + 2), dc.DCCONV_EINVAL, "16-byte aligned"),
    (dict(conv_state=ST + 8), dc.DCCONV_EINVAL, "16-byte aligned"),
    (dict(weight=WT + 4), dc.DCCONV_EINVAL, "16-byte aligned"),
    (dict(out=OUT + 2), dc.DCCONV_EINVAL, "16-byte aligned"),
    (dict(bias=BI + 2), dc.DCCONV_EINVAL, "16-byte aligned"),
    (dict(conv_state_indices=IX + 2), dc.DCCONV_EINVAL, "4-byte aligned"),
    (dict(dev_status=STAT + 1), dc.DCCONV_EINVAL, "4-byte aligned"),
    (dict(out=X + 256), dc.DCCONV_EINVAL, "overlaps"),
    (dict(out=X), dc.DCCONV_EINVAL, "overlaps"),
    (dict(conv_state=X + 128), dc.DCCONV_EINVAL, "overlaps"),
    (dict(out=WT + 64), dc.DCCONV_EINVAL, "overlaps"),
    (dict(conv_state_indices=ST + 16), dc.DCCONV_EINVAL, "overlaps"),
    (dict(dev_status=OUT + 8), dc.DCCONV_EINVAL, "overlaps"),
    (dict(bias=ST + 64), dc.DCCONV_EINVAL, "overlaps"),
]


@no_gpu
@pytest.mark.parametrize("over,code,frag", DECLINES, ids=[str(d[0]) for d in DECLINES])
def test_host_refusals(over, code, frag):
    rc = _call(**over)
    assert rc == code, (rc, dc.dcconv_last_error())
    assert frag in dc.dcconv_last_error()
    assert dc.dcconv_last_kernel() == ""


@no_gpu
def test_zero_rows_enqueue_nothing():
    assert _call(n=0, x=None, out=None, conv_state=None, weight=None) == dc.DCCONV_OK
    assert dc.dcconv_last_error() == "" and dc.dcconv_last_kernel() == ""


@no_gpu
def test_zero_rows_still_checks_metadata():
    assert _call(n=0, w=3) == dc.DCCONV_EUNSUPPORTED
    assert _call(n=0, l=2, st_d=2, st_s=128) == dc.DCCONV_EINVAL


@no_gpu
def test_error_message_is_thread_local():
    import threading
    assert _call(d=0) == dc.DCCONV_EINVAL
    seen = {}

    def other():
        seen["msg"] = dc.dcconv_last_error()

    t = threading.Thread(target=other)
    t.start(); t.join()
    assert seen["msg"] == ""
    assert "d (channels)" in dc.dcconv_last_error()


# ----------------------------------------------------- tensor front-end refusals


def _cpu_args(N=4, D=16, L=3, S=4):
    bf = torch.bfloat16
    return (torch.zeros(N, D, dtype=bf), torch.zeros(S, D, L, dtype=bf), torch.zeros(D, 4, dtype=bf))


def test_frontend_checks_cache_seqlens():
    x, st, w = _cpu_args()
    with pytest.raises(ValueError, match="cache_seqlens"):
        dc.causal_conv1d_update(x, st, w, cache_seqlens=torch.zeros(4, dtype=torch.int64))
    with pytest.raises(ValueError, match="cache_seqlens"):
        dc.causal_conv1d_update(x, st, w, cache_seqlens=torch.zeros(3, dtype=torch.int32))


def test_frontend_refuses_multi_token_x():
    _, st, w = _cpu_args()
    with pytest.raises(NotImplementedError, match="3-D x"):
        dc.causal_conv1d_update(torch.zeros(4, 16, 2, dtype=torch.bfloat16), st, w)


def test_frontend_refuses_autograd_inputs():
    x, st, w = _cpu_args()
    w = w.float().requires_grad_(True)
    with pytest.raises(NotImplementedError, match="inference only"):
        dc.causal_conv1d_update(x, st, w)


@pytest.mark.parametrize("bad", ["dtype_x", "dtype_idx", "act", "shape", "channels", "stride", "device"])
def test_frontend_contract_violations(bad):
    x, st, w = _cpu_args()
    kw = {}
    act = "silu"
    if bad == "dtype_x":
        x = x.float()
    elif bad == "dtype_idx":
        kw["conv_state_indices"] = torch.zeros(4, dtype=torch.int64)
    elif bad == "act":
        act = "gelu"
    elif bad == "shape":
        x = torch.zeros(4, dtype=torch.bfloat16)
    elif bad == "channels":
        w = torch.zeros(8, 4, dtype=torch.bfloat16)
    elif bad == "stride":
        x = torch.zeros(16, 4, dtype=torch.bfloat16).t()
    with pytest.raises(ValueError):
        dc.causal_conv1d_update(x, st, w, None, act, **kw)


# ------------------------------------------------------ multi-token entry point


def _targs(**over):
    a = dict(x=X, n=4, d=64, t=3, xs_n=192, xs_d=1, xs_t=64, conv_state=ST, s=4, l=3, st_s=192, st_d=3, st_l=1,
             weight=WT, w=4, bias=None, conv_state_indices=None, cache_seqlens=None, activation=1,
             out=OUT, os_n=192, os_d=1, os_t=64, dev_status=None, stream=None)
    a.update(over)
    return a


TOKEN_DECLINES = [
    (dict(t=-1), dc.DCCONV_EINVAL, "t (tokens)"),
    (dict(xs_t=-64), dc.DCCONV_EINVAL, "non-negative"),
    (dict(os_d=-1), dc.DCCONV_EINVAL, "non-negative"),
    (dict(xs_t=1 << 61), dc.DCCONV_EINVAL, "2^47 bytes"),
    (dict(os_n=1 << 48), dc.DCCONV_EINVAL, "2^47 bytes"),
    (dict(os_t=32), dc.DCCONV_EINVAL, "same address"),       # tokens overlap channels
    (dict(os_n=64), dc.DCCONV_EINVAL, "same address"),       # rows overlap tokens
    (dict(os_d=0), dc.DCCONV_EINVAL, "same address"),
    (dict(cache_seqlens=IX + 2), dc.DCCONV_EINVAL, "cache_seqlens must be 4-byte aligned"),
    (dict(cache_seqlens=OUT + 64), dc.DCCONV_EINVAL, "overlaps cache_seqlens"),
    (dict(w=3), dc.DCCONV_EUNSUPPORTED, "w=4"),
    (dict(l=2, st_d=2, st_s=128), dc.DCCONV_EINVAL, "must be >= w-1"),
    (dict(x=X + 8), dc.DCCONV_EINVAL, "16-byte aligned"),
    (dict(out=OUT + 2), dc.DCCONV_EINVAL, "16-byte aligned"),
    (dict(out=X + 512), dc.DCCONV_EINVAL, "overlaps"),
    (dict(conv_state=OUT + 256), dc.DCCONV_EINVAL, "overlaps"),
    (dict(s=3), dc.DCCONV_EINVAL, "must be >= n"),
    (dict(st_s=192, st_d=1, st_l=2), dc.DCCONV_EUNSUPPORTED, "neither compact"),
]


@no_gpu
@pytest.mark.parametrize("over,code,frag", TOKEN_DECLINES, ids=[str(d[0]) for d in TOKEN_DECLINES])
def test_tokens_host_refusals(over, code, frag):
    rc = dc.dcconv_update_tokens(**_targs(**over))
    assert rc == code, (rc, dc.dcconv_last_error())
    assert frag in dc.dcconv_last_error()


@no_gpu
def test_tokens_zero_tokens_or_rows_enqueue_nothing():
    assert dc.dcconv_update_tokens(**_targs(t=0, x=None, out=None)) == dc.DCCONV_OK
    assert dc.dcconv_update_tokens(**_targs(n=0, x=None, out=None)) == dc.DCCONV_OK
    assert dc.dcconv_last_kernel() == ""


def test_tokens_frontend_needs_3d_x():
    _, st, w = _cpu_args()
    with pytest.raises(ValueError, match=r"\[N, D, T\]"):
        dc.causal_conv1d_update_tokens(torch.zeros(4, 16, dtype=torch.bfloat16), st, w)


# ----------------------------------------------------------- prefill entry point

SEQ, HI = 0x90000000, 0xA0000000


def _pargs(**over):
    a = dict(x=X, n=4, d=64, t=10, xs_n=640, xs_d=1, xs_t=64, seq_starts=None, conv_state=ST, s=4, l=3, st_s=192,
             st_d=1, st_l=64, conv_state_indices=None, has_initial_state=None, weight=WT, w=4, bias=None,
             activation=1, out=OUT, os_n=640, os_d=1, os_t=64, dev_status=None, stream=None)
    a.update(over)
    return a


PREFILL_DECLINES = [
    (dict(t=-1), dc.DCCONV_EINVAL, "t (tokens)"),
    (dict(xs_t=-64), dc.DCCONV_EINVAL, "non-negative"),
    (dict(xs_t=1 << 60), dc.DCCONV_EINVAL, "2^47 bytes"),
    (dict(os_t=1 << 48), dc.DCCONV_EINVAL, "2^47 bytes"),
    (dict(conv_state=None), dc.DCCONV_EINVAL, "without conv_state"),                 # s = 4 without a state
    (dict(conv_state=None, s=0, conv_state_indices=IX), dc.DCCONV_EINVAL, "without conv_state"),
    (dict(conv_state=None, s=0, has_initial_state=HI), dc.DCCONV_EINVAL, "without conv_state"),
    (dict(w=3), dc.DCCONV_EUNSUPPORTED, "w=4"),
    (dict(l=2, st_l=64, st_s=128), dc.DCCONV_EINVAL, "must be >= w-1"),
    (dict(os_t=32), dc.DCCONV_EINVAL, "same address"),
    (dict(seq_starts=SEQ + 2, n=3, xs_n=0), dc.DCCONV_EINVAL, "4-byte aligned"),
    (dict(out=SEQ - 64, seq_starts=SEQ, n=3), dc.DCCONV_EINVAL, "overlaps seq_starts"),
    (dict(conv_state=HI - 256, has_initial_state=HI), dc.DCCONV_EINVAL, "overlaps has_initial_state"),
    (dict(out=X + 1024), dc.DCCONV_EINVAL, "overlaps"),
    (dict(x=X + 8), dc.DCCONV_EINVAL, "16-byte aligned"),
    (dict(s=3), dc.DCCONV_EINVAL, "must be >= n"),
    (dict(st_d=2, st_l=1, st_s=192), dc.DCCONV_EUNSUPPORTED, "neither compact"),
]


@no_gpu
@pytest.mark.parametrize("over,code,frag", PREFILL_DECLINES, ids=[str(d[0]) for d in PREFILL_DECLINES])
def test_prefill_host_refusals(over, code, frag):
    rc = dc.dcconv_prefill(**_pargs(**over))
    assert rc == code, (rc, dc.dcconv_last_error())
    assert frag in dc.dcconv_last_error()


@no_gpu
def test_prefill_nothing_to_do_enqueues_nothing():
    assert dc.dcconv_prefill(**_pargs(n=0, x=None, out=None)) == dc.DCCONV_OK
    assert dc.dcconv_last_kernel() == ""
    # stateless and no tokens: nothing to read or write
    assert dc.dcconv_prefill(**_pargs(t=0, x=None, out=None, conv_state=None, s=0)) == dc.DCCONV_OK
    assert dc.dcconv_last_kernel() == ""


def test_prefill_frontend_checks():
    x = torch.zeros(2, 16, 5, dtype=torch.bfloat16)
    w = torch.zeros(16, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"\[N, D, T\]"):
        dc.causal_conv1d(x[:, :, 0], w)
    with pytest.raises(ValueError, match="on a GPU"):
        dc.causal_conv1d(x, w)
    with pytest.raises(NotImplementedError, match="inference only"):
        dc.causal_conv1d(x.clone().float().requires_grad_(), w)


def test_stream_copy_refusals_before_any_hip_call():
    # the measurement-control copy validates on the host; fake addresses never
    # reach the device because every case here is refused (or empty)
    a, b = 0x7F0000000000, 0x7F0000100000
    assert dc.dcconv_stream_copy(a, b, 24, None) == dc.DCCONV_EINVAL
    assert "multiple of 16" in dc.dcconv_last_error()
    assert dc.dcconv_stream_copy(a + 8, b, 16, None) == dc.DCCONV_EINVAL
    assert "aligned" in dc.dcconv_last_error()
    assert dc.dcconv_stream_copy(a + 16, a, 32, None) == dc.DCCONV_EINVAL
    assert "overlap" in dc.dcconv_last_error()
    assert dc.dcconv_stream_copy(a, b, -16, None) == dc.DCCONV_EINVAL
    assert dc.dcconv_stream_copy(0, b, 16, None) == dc.DCCONV_EINVAL
    assert dc.dcconv_stream_copy(a, b, 0, None) == dc.DCCONV_OK
    assert dc.dcconv_last_kernel() == ""


def test_busy_spin_refusals_before_any_hip_call():
    # out-of-range spans are refused on the host; 0 enqueues nothing
    for us in (-1.0, float("nan"), float("inf"), 1e6 + 1):
        assert dc.dcconv_busy_spin(us, None) == dc.DCCONV_EINVAL
        assert "microseconds" in dc.dcconv_last_error()
    assert dc.dcconv_busy_spin(0.0, None) == dc.DCCONV_OK
    assert dc.dcconv_last_kernel() == ""
