"""Oracle for the depthwise causal conv1d decode update -- TEST INFRASTRUCTURE ONLY.

Python access (ctypes, numpy arrays of BF16 bit patterns as ``uint16``) to the
plain-C FP32 oracle in ``dcconv_oracle.c``.  Only ``tests/``, the package smoke
check and the benchmark's CPU-baseline leg may import this module; the GPU
library never calls it and shares no code with it.

Semantics follow the cuDNN FE-OSS page "Causal Conv1d Decode Update",
sections "Causal Conv1d Decode Update" and "Semantic tensor contract"; the
prefill (``prefill``) is the full-sequence convolution that page names at its
top, read as the convolution whose final state the decode update continues.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dcconv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, EARGS, EINDEX, EDUP = 0, 1, 2, 3
ACT = {None: 0, "identity": 0, "silu": 1, "swish": 1}


class OracleError(ValueError):
    """The oracle refused its inputs (the code says why)."""

    def __init__(self, code: int):
        names = {EARGS: "malformed arguments", EINDEX: "slot index out of range",
                 EDUP: "duplicate non-padding slot"}
        super().__init__(f"oracle error {code}: {names.get(code, '?')}")
        self.code = code


_DRIVER = os.path.join(_HERE, "sanitize_driver.c")


def build(force: bool = False) -> str:
    """Compile the oracle with the host C compiler (plain C99, no fast-math).
    With ``force`` also compile the sanitizer driver (plain build here; the CPU
    test suite builds it again with AddressSanitizer and UBSan), so every C
    source of the oracle is known to compile."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
                        "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    if force:
        out_dir = os.path.join(_HERE, "_build")
        os.makedirs(out_dir, exist_ok=True)
        subprocess.run(["gcc", "-std=c99", "-O1", "-ffp-contract=off", "-o", os.path.join(out_dir, "sanitize_driver"),
                        _SRC, _DRIVER, "-lm"], check=True)
    return _LIB


_lock = threading.Lock()
_lib = None


# The test of planted mistakes points this at a deliberately broken build of the
# oracle, to show that the pins catch each mistake; nothing else sets it.
_LIBRARY_ENV = "DCCONV_ORACLE_LIBRARY"


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            other = os.environ.get(_LIBRARY_ENV)
            if not other:
                build()
            L = ctypes.CDLL(other or _LIB)
            i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
            L.oracle_update.restype = i32
            L.oracle_update.argtypes = [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64,
                                        vp, i64, vp, vp, i32, vp, vp]
            L.oracle_update_tokens.restype = i32
            L.oracle_update_tokens.argtypes = [vp, i64, i64, i64, i64, i64, i64,   # x, n, d, t, xs_n, xs_d, xs_t
                                               vp, i64, i64, i64, i64, i64,        # state, s, l, st_s, st_d, st_l
                                               vp, i64, vp, vp, i32,               # weight, w, bias, indices, act
                                               vp, vp, i64, i64, i64]              # out, out_f32, os_n, os_d, os_t
            L.oracle_prefill.restype = i32
            L.oracle_prefill.argtypes = [vp, i64, i64, i64, i64, i64, i64, vp,   # x, n, d, t, xs_n, xs_d, xs_t, starts
                                         vp, i64, i64, i64, i64, i64,            # state, s, l, st_s, st_d, st_l
                                         vp, vp,                                 # indices, has_init
                                         vp, i64, vp, i32,                       # weight, w, bias, act
                                         vp, vp, i64, i64, i64]                  # out, out_f32, os_n, os_d, os_t
            L.oracle_update_ring.restype = i32
            L.oracle_update_ring.argtypes = [vp, i64, i64, i64, vp, i64, i64, i64, i64, i64,
                                             vp, i64, vp, vp, vp, i32, vp, vp]
            L.oracle_bf16_to_f32.restype = ctypes.c_float
            L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
            L.oracle_f32_to_bf16.restype = ctypes.c_uint16
            L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
            L.oracle_bf16_to_f32_bits.restype = ctypes.c_uint32
            L.oracle_bf16_to_f32_bits.argtypes = [ctypes.c_uint16]
            L.oracle_f32_bits_to_bf16.restype = ctypes.c_uint16
            L.oracle_f32_bits_to_bf16.argtypes = [ctypes.c_uint32]
            L.oracle_version.restype = i32
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _need(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype:
        raise TypeError(f"{name} must be a numpy array of {dtype}")
    if not a.flags.c_contiguous:
        raise TypeError(f"{name} must be C-contiguous (strides are passed explicitly)")


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Element-wise oracle BF16 -> FP32 (slow; for pinning the converter).  Bit
    patterns cross the binding, so NaN payloads arrive unchanged."""
    f = lib().oracle_bf16_to_f32_bits
    flat = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([f(int(b)) for b in flat], dtype=np.uint32).view(np.float32).reshape(np.shape(bits))


def f32_to_bf16(vals: np.ndarray) -> np.ndarray:
    """Element-wise oracle FP32 -> BF16 bits, round to nearest even (slow).  Bit
    patterns cross the binding, so a signalling NaN reaches the converter as it is."""
    f = lib().oracle_f32_bits_to_bf16
    flat = np.asarray(vals, dtype=np.float32).ravel().view(np.uint32)
    return np.array([f(int(v)) for v in flat], dtype=np.uint16).reshape(np.shape(vals))


def update(x, conv_state, weight, bias=None, activation=None, *, conv_state_indices=None,
           d=None, ld=None, state_strides=None, want_f32=False):
    """One decode step on host arrays.  ``conv_state`` is updated in place.

    x:          uint16 BF16 bits, shape [N, ld] (first ``d`` columns used) or [N, D]
    conv_state: uint16 BF16 bits buffer; logical [S, D, L] with element strides
                ``state_strides`` (default: compact (D*L, L, 1)); pass the 3-D array
                and, for other layouts, the strides of its logical view.
    weight:     uint16 [D, W];  bias: uint16 [D] or None
    conv_state_indices: int32 [N] or None
    Returns ``out`` (uint16 [N, D]) or ``(out, out_f32)`` when ``want_f32``.
    """
    _need(x, np.uint16, "x"); _need(conv_state, np.uint16, "conv_state")
    _need(weight, np.uint16, "weight")
    if bias is not None:
        _need(bias, np.uint16, "bias")
    if conv_state_indices is not None:
        _need(conv_state_indices, np.int32, "conv_state_indices")
    n = x.shape[0]
    D, W = weight.shape
    d = D if d is None else d
    ld = x.shape[1] if ld is None else ld
    if state_strides is None:
        S, Dd, L = conv_state.shape
        st = (Dd * L, L, 1)
    else:
        S, L, st = state_strides[0], state_strides[1], state_strides[2]
    out = np.zeros((n, d), dtype=np.uint16)
    out_f32 = np.zeros((n, d), dtype=np.float32) if want_f32 else None
    rc = lib().oracle_update(_ptr(x), n, d, ld, _ptr(conv_state), S, L, st[0], st[1], st[2],
                             _ptr(weight), W, _ptr(bias), _ptr(conv_state_indices),
                             ACT[activation], _ptr(out), _ptr(out_f32))
    if rc != OK:
        raise OracleError(rc)
    return (out, out_f32) if want_f32 else out


def update_strided(x, n, d, ld, state_buf, S, L, strides, weight, bias, indices, activation,
                   want_f32=False):
    """``update`` with every layout parameter explicit; ``state_buf`` is the flat
    uint16 buffer that holds the [S, D, L] state at element ``strides``."""
    _need(state_buf, np.uint16, "state_buf")
    W = weight.shape[1]
    out = np.zeros((n, d), dtype=np.uint16)
    out_f32 = np.zeros((n, d), dtype=np.float32) if want_f32 else None
    rc = lib().oracle_update(_ptr(x), n, d, ld, _ptr(state_buf), S, L, strides[0], strides[1],
                             strides[2], _ptr(weight), W, _ptr(bias), _ptr(indices),
                             ACT[activation], _ptr(out), _ptr(out_f32))
    if rc != OK:
        raise OracleError(rc)
    return (out, out_f32) if want_f32 else out


def update_tokens(x_buf, n, d, t, x_strides, state_buf, S, L, state_strides, weight, bias, indices,
                  activation, want_f32=False):
    """T successive decode steps (the multi-token form x[N, D, T]).

    x_buf: flat/any-shape contiguous uint16 buffer holding x at element strides
    ``x_strides`` = (n, channel, token); state_buf likewise at ``state_strides``.
    Returns out as uint16 [N, T, D] (token-major), or (out, out_f32).
    """
    _need(x_buf, np.uint16, "x_buf"); _need(state_buf, np.uint16, "state_buf")
    W = weight.shape[1]
    out = np.zeros((n, t, d), dtype=np.uint16)
    out_f32 = np.zeros((n, t, d), dtype=np.float32) if want_f32 else None
    rc = lib().oracle_update_tokens(_ptr(x_buf), n, d, t, x_strides[0], x_strides[1], x_strides[2],
                                    _ptr(state_buf), S, L, state_strides[0], state_strides[1], state_strides[2],
                                    _ptr(weight), W, _ptr(bias), _ptr(indices), ACT[activation],
                                    _ptr(out), _ptr(out_f32), t * d, 1, d)
    if rc != OK:
        raise OracleError(rc)
    return (out, out_f32) if want_f32 else out


def prefill(x_buf, n, d, t, x_strides, weight, bias=None, activation=None, *, starts=None, state_buf=None, S=0,
            L=0, state_strides=(0, 0, 0), indices=None, has_init=None, want_f32=False):
    """Full-sequence causal convolution (prefill) over n sequences.

    Batch form (``starts`` None): n sequences of t tokens, token j of sequence i
    at x_buf[i*xs_n + c*xs_d + j*xs_t]; out is returned as uint16 [n, t, d].
    Varlen form (``starts`` int32 [n+1]): sequence i is packed tokens
    starts[i]..starts[i+1]-1 at x_buf[c*xs_d + p*xs_t]; out is [t, d] (packed).
    ``state_buf`` (None = stateless) holds [S, D, L] at ``state_strides`` and
    receives the final states in place; ``has_init`` uint8 [n] or None (zeros).
    """
    _need(x_buf, np.uint16, "x_buf"); _need(weight, np.uint16, "weight")
    if state_buf is not None:
        _need(state_buf, np.uint16, "state_buf")
    if starts is not None:
        _need(starts, np.int32, "starts")
    if has_init is not None:
        _need(has_init, np.uint8, "has_init")
    W = weight.shape[1]
    if starts is None:
        shape, os_ = (n, t, d), (t * d, 1, d)
    else:
        shape, os_ = (t, d), (0, 1, d)
    out = np.zeros(shape, dtype=np.uint16)
    out_f32 = np.zeros(shape, dtype=np.float32) if want_f32 else None
    rc = lib().oracle_prefill(_ptr(x_buf), n, d, t, x_strides[0], x_strides[1], x_strides[2], _ptr(starts),
                              _ptr(state_buf), S, L, state_strides[0], state_strides[1], state_strides[2],
                              _ptr(indices), _ptr(has_init), _ptr(weight), W, _ptr(bias), ACT[activation],
                              _ptr(out), _ptr(out_f32), os_[0], os_[1], os_[2])
    if rc != OK:
        raise OracleError(rc)
    return (out, out_f32) if want_f32 else out


def update_ring(x, n, d, ld, state_buf, S, L, strides, weight, bias, indices, cache_seqlens, activation,
                want_f32=False):
    """One decode step on circular-buffer state (``cache_seqlens`` int32 [N]:
    tokens each row's slot has seen).  ``state_buf`` holds [S, D, L] at element
    ``strides`` and is updated in place (one value per channel)."""
    _need(state_buf, np.uint16, "state_buf"); _need(x, np.uint16, "x")
    _need(cache_seqlens, np.int32, "cache_seqlens")
    W = weight.shape[1]
    out = np.zeros((n, d), dtype=np.uint16)
    out_f32 = np.zeros((n, d), dtype=np.float32) if want_f32 else None
    rc = lib().oracle_update_ring(_ptr(x), n, d, ld, _ptr(state_buf), S, L, strides[0], strides[1], strides[2],
                                  _ptr(weight), W, _ptr(bias), _ptr(indices), _ptr(cache_seqlens), ACT[activation],
                                  _ptr(out), _ptr(out_f32))
    if rc != OK:
        raise OracleError(rc)
    return (out, out_f32) if want_f32 else out
