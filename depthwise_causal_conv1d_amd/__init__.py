"""MI355X-native depthwise causal conv1d decode update.

Python binding over the C ABI of ``libdcconv.so`` (declared in ``include/dcconv.h``).
It only marshals arguments: every step of the update runs in the library's gfx950
HIP kernels.  PyTorch supplies device memory and the current stream.

``dcconv_update`` mirrors the C entry point (raw device pointers as ints).
``causal_conv1d_update`` mirrors the Python signature on the cuDNN FE-OSS page
"Causal Conv1d Decode Update" (section "Python API"): positional ``x, conv_state,
weight, bias, activation``, keyword-only ``cache_seqlens`` and
``conv_state_indices``; ``conv_state`` is updated in place and a newly allocated
output is returned.  ``causal_conv1d_update_out`` writes into a caller buffer and
allocates nothing.  ``causal_conv1d_update_tokens`` applies T tokens per row in one
call (the multi-token form x[N, D, T] the page reserves).  ``causal_conv1d`` is the
full-sequence prefill the page names at its top, returning the final state the
update continues (batch or packed variable-length sequences).

There is no fallback: if the HIP library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = [
    "DCCONV_OK", "DCCONV_EINVAL", "DCCONV_EUNSUPPORTED", "DCCONV_EHIP",
    "DCCONV_ACT_IDENTITY", "DCCONV_ACT_SILU", "DCCONV_DEV_BAD_INDEX", "DCCONV_DEV_DUP_INDEX",
    "dcconv_abi_version", "dcconv_last_error", "dcconv_last_kernel", "dcconv_update",
    "dcconv_update_tokens", "causal_conv1d_update", "causal_conv1d_update_out",
    "causal_conv1d_update_tokens", "dcconv_prefill", "causal_conv1d", "library_path", "DcconvError",
    "DCCONV_DEV_BAD_SEQ", "DCCONV_DEV_BAD_SEQLEN", "dcconv_stream_copy", "stream_copy",
    "dcconv_busy_spin", "busy_spin",
]

DCCONV_OK, DCCONV_EINVAL, DCCONV_EUNSUPPORTED, DCCONV_EHIP = 0, 1, 2, 3
DCCONV_ACT_IDENTITY, DCCONV_ACT_SILU = 0, 1
DCCONV_DEV_BAD_INDEX, DCCONV_DEV_DUP_INDEX, DCCONV_DEV_BAD_SEQ, DCCONV_DEV_BAD_SEQLEN = 1, 2, 4, 8

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libdcconv.so")
_lock = threading.Lock()
_lib = None

_ACTIVATIONS = {None: DCCONV_ACT_IDENTITY, "identity": DCCONV_ACT_IDENTITY,
                "silu": DCCONV_ACT_SILU, "swish": DCCONV_ACT_SILU}


class DcconvError(RuntimeError):
    """The HIP runtime refused a launch (DCCONV_EHIP)."""


def library_path() -> str:
    return _LIB_PATH


def _load() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise ImportError(
                    f"{_LIB_PATH} is not built; run `python -m depthwise_causal_conv1d_amd._build` "
                    "(there is no fallback implementation)")
            lib = ctypes.CDLL(_LIB_PATH)
            i64, vp, i32, cp = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_char_p
            lib.dcconv_abi_version.restype = i32
            lib.dcconv_abi_version.argtypes = []
            lib.dcconv_last_error.restype = cp
            lib.dcconv_last_error.argtypes = []
            lib.dcconv_last_kernel.restype = cp
            lib.dcconv_last_kernel.argtypes = []
            lib.dcconv_update.restype = i32
            lib.dcconv_update.argtypes = [vp, i64, i64, i64,        # x, n, d, ld_x
                                          vp, i64, i64,             # conv_state, s, l
                                          i64, i64, i64,            # st_s, st_d, st_l
                                          vp, i64, vp,              # weight, w, bias
                                          vp, vp, i32,              # indices, cache_seqlens, activation
                                          vp, vp, vp]               # out, dev_status, stream
            lib.dcconv_update_tokens.restype = i32
            lib.dcconv_update_tokens.argtypes = [vp, i64, i64, i64,          # x, n, d, t
                                                 i64, i64, i64,              # xs_n, xs_d, xs_t
                                                 vp, i64, i64,               # conv_state, s, l
                                                 i64, i64, i64,              # st_s, st_d, st_l
                                                 vp, i64, vp,                # weight, w, bias
                                                 vp, vp, i32,                # indices, cache_seqlens, activation
                                                 vp, i64, i64, i64,          # out, os_n, os_d, os_t
                                                 vp, vp]                     # dev_status, stream
            lib.dcconv_prefill.restype = i32
            lib.dcconv_prefill.argtypes = [vp, i64, i64, i64,                # x, n, d, t
                                           i64, i64, i64, vp,                # xs_n, xs_d, xs_t, seq_starts
                                           vp, i64, i64,                     # conv_state, s, l
                                           i64, i64, i64,                    # st_s, st_d, st_l
                                           vp, vp,                           # indices, has_initial_state
                                           vp, i64, vp, i32,                 # weight, w, bias, activation
                                           vp, i64, i64, i64,                # out, os_n, os_d, os_t
                                           vp, vp]                           # dev_status, stream
            lib.dcconv_stream_copy.restype = i32
            lib.dcconv_stream_copy.argtypes = [vp, vp, i64, vp]      # dst, src, bytes, stream
            lib.dcconv_busy_spin.restype = i32
            lib.dcconv_busy_spin.argtypes = [ctypes.c_double, vp]     # microseconds, stream
            _lib = lib
    return _lib


def _raise_for(rc: int) -> None:
    if rc == DCCONV_OK:
        return
    msg = dcconv_last_error()
    if rc == DCCONV_EINVAL:
        raise ValueError(msg)
    if rc == DCCONV_EUNSUPPORTED:
        raise NotImplementedError(msg)
    raise DcconvError(msg or f"dcconv error {rc}")


# ----------------------------------------------------------------- raw C ABI


def dcconv_abi_version() -> int:
    return _load().dcconv_abi_version()


def dcconv_last_error() -> str:
    return _load().dcconv_last_error().decode()


def dcconv_last_kernel() -> str:
    return _load().dcconv_last_kernel().decode()


def dcconv_update(x, n, d, ld_x, conv_state, s, l, st_s, st_d, st_l, weight, w, bias,
                  conv_state_indices, cache_seqlens, activation, out, dev_status, stream) -> int:
    """The C entry point, one to one: pointers are ints (0/None = NULL).  Returns the
    status code; see ``include/dcconv.h`` for the meaning of every argument."""
    return _load().dcconv_update(x, n, d, ld_x, conv_state, s, l, st_s, st_d, st_l, weight, w,
                                 bias, conv_state_indices, cache_seqlens, activation, out,
                                 dev_status, stream)


def dcconv_update_tokens(x, n, d, t, xs_n, xs_d, xs_t, conv_state, s, l, st_s, st_d, st_l, weight, w, bias,
                         conv_state_indices, cache_seqlens, activation, out, os_n, os_d, os_t, dev_status,
                         stream) -> int:
    """The multi-token C entry point, one to one (pointers as ints)."""
    return _load().dcconv_update_tokens(x, n, d, t, xs_n, xs_d, xs_t, conv_state, s, l, st_s, st_d, st_l, weight,
                                        w, bias, conv_state_indices, cache_seqlens, activation, out, os_n, os_d,
                                        os_t, dev_status, stream)


def dcconv_prefill(x, n, d, t, xs_n, xs_d, xs_t, seq_starts, conv_state, s, l, st_s, st_d, st_l,
                   conv_state_indices, has_initial_state, weight, w, bias, activation, out, os_n, os_d, os_t,
                   dev_status, stream) -> int:
    """The prefill C entry point, one to one (pointers as ints)."""
    return _load().dcconv_prefill(x, n, d, t, xs_n, xs_d, xs_t, seq_starts, conv_state, s, l, st_s, st_d, st_l,
                                  conv_state_indices, has_initial_state, weight, w, bias, activation, out, os_n,
                                  os_d, os_t, dev_status, stream)


def dcconv_busy_spin(microseconds, stream) -> int:
    """The busy-spin measurement control, one to one."""
    return _load().dcconv_busy_spin(microseconds, stream)


def dcconv_stream_copy(dst, src, nbytes, stream) -> int:
    """The measurement-control copy, one to one (pointers as ints)."""
    return _load().dcconv_stream_copy(dst, src, nbytes, stream)


# ------------------------------------------------------------ tensor front end


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_tensors(x, conv_state, weight, bias, conv_state_indices, cache_seqlens, activation,
                   x_unit_channel_stride=True):
    import torch

    for name, t in (("x", x), ("conv_state", conv_state), ("weight", weight), ("bias", bias),
                    ("conv_state_indices", conv_state_indices)):
        if t is not None and t.requires_grad:
            raise NotImplementedError(f"inference only: {name} requires grad (training is not served)")
    if x.dim() == 3:
        raise NotImplementedError("a 3-D x (multi-token update) is not served by this call")
    if x.dim() != 2:
        raise ValueError(f"x must be [N, D], got shape {tuple(x.shape)}")
    if conv_state.dim() != 3:
        raise ValueError(f"conv_state must be [S, D, L], got shape {tuple(conv_state.shape)}")
    if weight.dim() != 2:
        raise ValueError(f"weight must be [D, W], got shape {tuple(weight.shape)}")
    for name, t in (("x", x), ("conv_state", conv_state), ("weight", weight), ("bias", bias)):
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if conv_state_indices is not None and conv_state_indices.dtype != torch.int32:
        raise ValueError(f"conv_state_indices must be int32, got {conv_state_indices.dtype}")
    if activation not in _ACTIVATIONS:
        raise ValueError(f"activation must be None, 'identity', 'silu' or 'swish', got {activation!r}")
    N, D = x.shape
    if conv_state.shape[1] != D or weight.shape[0] != D:
        raise ValueError(f"channel counts differ: x {D}, conv_state {conv_state.shape[1]}, weight {weight.shape[0]}")
    if x_unit_channel_stride and x.stride(1) != 1 and D > 1:
        raise ValueError("x must have unit stride along channels (strides (ld, 1))")
    if not weight.is_contiguous():
        raise ValueError("weight must be contiguous [D, W]")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != D or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [D] tensor")
    if conv_state_indices is not None and (conv_state_indices.dim() != 1 or conv_state_indices.shape[0] != N
                                           or not conv_state_indices.is_contiguous()):
        raise ValueError("conv_state_indices must be a contiguous int32 [N] tensor")
    if cache_seqlens is not None and (cache_seqlens.dtype != torch.int32 or cache_seqlens.dim() != 1
                                      or cache_seqlens.shape[0] != N or not cache_seqlens.is_contiguous()):
        raise ValueError("cache_seqlens must be a contiguous int32 [N] tensor (tokens each row's slot has seen)")
    dev = x.device
    for name, t in (("conv_state", conv_state), ("weight", weight), ("bias", bias),
                    ("conv_state_indices", conv_state_indices), ("cache_seqlens", cache_seqlens)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, x on {dev}")
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {dev}")


def causal_conv1d_update_out(x, conv_state, weight, bias=None, activation=None, *, out,
                             cache_seqlens=None, conv_state_indices=None, dev_status=None):
    """Like ``causal_conv1d_update`` but writes ``out`` (bf16 [N, D], contiguous) and
    allocates nothing.  ``dev_status`` (int32 [1] on the device, optional) receives
    DCCONV_DEV_* bits for rejected routing entries."""
    import torch

    _check_tensors(x, conv_state, weight, bias, conv_state_indices, cache_seqlens, activation)
    N, D = x.shape
    if out.shape != (N, D) or out.dtype != torch.bfloat16 or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous bfloat16 [N, D] tensor on x's device")
    if dev_status is not None and (dev_status.dtype != torch.int32 or dev_status.device != x.device):
        raise ValueError("dev_status must be an int32 tensor on x's device")
    S, _, L = conv_state.shape
    st = conv_state.stride()
    ld = x.stride(0) if N > 1 else D
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        rc = dcconv_update(_ptr(x), N, D, ld, _ptr(conv_state), S, L, st[0], st[1], st[2],
                           _ptr(weight), weight.shape[1], _ptr(bias), _ptr(conv_state_indices), _ptr(cache_seqlens),
                           _ACTIVATIONS[activation], _ptr(out), _ptr(dev_status), stream)
    _raise_for(rc)
    return out


def causal_conv1d_update(x, conv_state, weight, bias=None, activation=None, *,
                         cache_seqlens=None, conv_state_indices=None):
    """One decode step: updates ``conv_state`` in place and returns a new bf16 [N, D]
    output (page "Causal Conv1d Decode Update", section "Python API").  With
    ``cache_seqlens`` (int32 [N], tokens each row's slot has seen; not advanced
    here) the state is a circular buffer: token i at position i mod L."""
    import torch

    _check_tensors(x, conv_state, weight, bias, conv_state_indices, cache_seqlens, activation)
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    return causal_conv1d_update_out(x, conv_state, weight, bias, activation, out=out,
                                    cache_seqlens=cache_seqlens, conv_state_indices=conv_state_indices)


def causal_conv1d_update_tokens(x, conv_state, weight, bias=None, activation=None, *, conv_state_indices=None,
                                cache_seqlens=None, out=None, dev_status=None):
    """T successive decode steps in one call: x is [N, D, T] (any strides), the
    multi-token form the page reserves.  ``conv_state`` is updated in place (each
    selected slot read and written once); returns out [N, D, T], by default
    stored token-major (a view of a contiguous [N, T, D] buffer).  With
    ``cache_seqlens`` the state is a circular buffer, token t of row n being the
    (cache_seqlens[n] + t)-th token its slot sees."""
    import torch

    if x.dim() != 3:
        raise ValueError(f"x must be [N, D, T], got shape {tuple(x.shape)}")
    N, D, T = x.shape
    x2 = x[:, :, 0] if T > 0 else x.new_empty(N, D)
    _check_tensors(x2, conv_state, weight, bias, conv_state_indices, cache_seqlens, activation,
                   x_unit_channel_stride=False)
    if x.dtype != torch.bfloat16:
        raise ValueError(f"x must be bfloat16, got {x.dtype}")
    if out is None:
        out = torch.empty(N, T, D, dtype=torch.bfloat16, device=x.device).permute(0, 2, 1)
    elif out.shape != (N, D, T) or out.dtype != torch.bfloat16 or out.device != x.device:
        raise ValueError("out must be a bfloat16 [N, D, T] tensor on x's device")
    if dev_status is not None and (dev_status.dtype != torch.int32 or dev_status.device != x.device):
        raise ValueError("dev_status must be an int32 tensor on x's device")
    S, _, L = conv_state.shape
    st = conv_state.stride()
    xs, os_ = x.stride(), out.stride()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        rc = dcconv_update_tokens(_ptr(x), N, D, T, xs[0], xs[1], xs[2], _ptr(conv_state), S, L, st[0], st[1], st[2],
                                  _ptr(weight), weight.shape[1], _ptr(bias), _ptr(conv_state_indices),
                                  _ptr(cache_seqlens),
                                  _ACTIVATIONS[activation], _ptr(out), os_[0], os_[1], os_[2], _ptr(dev_status),
                                  stream)
    _raise_for(rc)
    return out


def causal_conv1d(x, weight, bias=None, activation=None, *, conv_state=None, conv_state_indices=None,
                  has_initial_state=None, seq_starts=None, return_final_state=False, out=None, dev_status=None):
    """Full-sequence causal convolution (prefill) with its final state.

    x: bf16 [N, D, T] at any strides (token-major storage, i.e. a [N, T, D] buffer
    seen as [N, D, T], is the fast layout).  With ``seq_starts`` (int32 [n+1] on the
    device) x is [1, D, total_T] holding n packed sequences.
    conv_state: optional bf16 [S, D, L], read as the initial state of the sequences
    that ``has_initial_state`` (bool/uint8 [n]) marks and overwritten with every
    live sequence's final state; ``conv_state_indices`` routes sequences to slots
    (-1 = padding) as in the decode update.
    return_final_state: without ``conv_state``, allocate the channel-last
    [n, D, W-1] final state the decode update accepts in place, and return
    ``(out, state)``.  Returns ``out`` [N, D, T] otherwise (by default a view of a
    token-major [N, T, D] buffer).
    """
    import torch

    if x.dim() != 3:
        raise ValueError(f"x must be [N, D, T], got shape {tuple(x.shape)}")
    for name, t in (("x", x), ("weight", weight), ("bias", bias), ("conv_state", conv_state)):
        if t is not None and t.requires_grad:
            raise NotImplementedError(f"inference only: {name} requires grad (training is not served)")
        if t is not None and t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16, got {t.dtype}")
    if activation not in _ACTIVATIONS:
        raise ValueError(f"activation must be None, 'identity', 'silu' or 'swish', got {activation!r}")
    B, D, T = x.shape
    dev = x.device
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, got {dev}")
    if weight.dim() != 2 or weight.shape[0] != D or not weight.is_contiguous():
        raise ValueError("weight must be a contiguous [D, W] tensor")
    if bias is not None and (bias.dim() != 1 or bias.shape[0] != D or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous [D] tensor")
    if seq_starts is not None:
        if B != 1:
            raise ValueError("with seq_starts, x must be [1, D, total_T] (packed sequences)")
        if seq_starts.dtype != torch.int32 or seq_starts.dim() != 1 or not seq_starts.is_contiguous():
            raise ValueError("seq_starts must be a contiguous int32 [n+1] tensor")
        n = seq_starts.shape[0] - 1
        if n < 0:
            raise ValueError("seq_starts must hold at least one entry")
    else:
        n = B
    if has_initial_state is not None:
        if has_initial_state.dtype not in (torch.bool, torch.uint8) or has_initial_state.shape != (n,) \
                or not has_initial_state.is_contiguous():
            raise ValueError("has_initial_state must be a contiguous bool/uint8 [n] tensor")
    if conv_state_indices is not None and (conv_state_indices.dtype != torch.int32 or
                                           conv_state_indices.shape != (n,) or
                                           not conv_state_indices.is_contiguous()):
        raise ValueError("conv_state_indices must be a contiguous int32 [n] tensor")
    for name, t in (("weight", weight), ("bias", bias), ("conv_state", conv_state), ("seq_starts", seq_starts),
                    ("conv_state_indices", conv_state_indices), ("has_initial_state", has_initial_state)):
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, x on {dev}")
    state_out = None
    if conv_state is None and return_final_state:
        if has_initial_state is not None or conv_state_indices is not None:
            raise ValueError("has_initial_state and conv_state_indices need a conv_state")
        W = weight.shape[1]
        conv_state = torch.empty(n, max(W - 1, 1), D, dtype=torch.bfloat16, device=dev).permute(0, 2, 1)
        state_out = conv_state
    if conv_state is not None and (conv_state.dim() != 3 or conv_state.shape[1] != D):
        raise ValueError(f"conv_state must be [S, D, L] with D={D}, got {tuple(conv_state.shape)}")
    if out is None:
        out = torch.empty(B, T, D, dtype=torch.bfloat16, device=dev).permute(0, 2, 1)
    elif out.shape != (B, D, T) or out.dtype != torch.bfloat16 or out.device != dev:
        raise ValueError("out must be a bfloat16 [N, D, T] tensor on x's device")
    if dev_status is not None and (dev_status.dtype != torch.int32 or dev_status.device != dev):
        raise ValueError("dev_status must be an int32 tensor on x's device")
    if conv_state is not None:
        S, _, L = conv_state.shape
        st = conv_state.stride()
    else:
        S, L, st = 0, 0, (0, 0, 0)
    xs, os_ = x.stride(), out.stride()
    hi = None if has_initial_state is None else has_initial_state.view(torch.uint8)
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = dcconv_prefill(_ptr(x), n, D, T, xs[0], xs[1], xs[2], _ptr(seq_starts), _ptr(conv_state), S, L,
                            st[0], st[1], st[2], _ptr(conv_state_indices), _ptr(hi), _ptr(weight), weight.shape[1],
                            _ptr(bias), _ACTIVATIONS[activation], _ptr(out), os_[0], os_[1], os_[2],
                            _ptr(dev_status), stream)
    _raise_for(rc)
    return (out, state_out) if state_out is not None else out


def stream_copy(dst, src) -> None:
    """Copy the bytes of ``src`` into ``dst`` (two contiguous device tensors of the
    same byte size) on the current stream, with the update kernels' access
    pattern: the bandwidth control a benchmark times beside the update."""
    import torch

    if not (dst.is_contiguous() and src.is_contiguous()):
        raise ValueError("stream_copy needs contiguous tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or dst.device != src.device:
        raise ValueError("stream_copy needs two tensors of one size on one device")
    with torch.cuda.device(src.device):
        rc = dcconv_stream_copy(dst.data_ptr(), src.data_ptr(), nbytes,
                                torch.cuda.current_stream(src.device).cuda_stream)
    _raise_for(rc)


def busy_spin(microseconds: float, device=None) -> None:
    """Keep every SIMD of the device busy for about ``microseconds`` on its
    current stream: a benchmark's head ahead of a timed region."""
    import torch

    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        rc = dcconv_busy_spin(float(microseconds), torch.cuda.current_stream(dev).cuda_stream)
    _raise_for(rc)
