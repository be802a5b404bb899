"""Shared helpers for the GPU parity tests (not a test module).

Moves BF16 bit patterns between numpy and the device, builds guarded device
buffers, runs the CPU oracle beside the HIP library on the same inputs and
compares the results to the accuracy contract:

* state, padding rows, routing and untouched slots: bit-exact;
* outputs: within 1 BF16 ulp of the oracle's BF16 output, or
  |gpu - ref_f32| <= 1e-2 * max(1, |ref_f32|), ref_f32 being the oracle's FP32
  value before its one rounding.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import depthwise_causal_conv1d_amd as dc
from depthwise_causal_conv1d_amd.workloads import FILL_SENTINEL, bf16_bits_to_f32

GUARD = 64  # elements of sentinel on each side of every written device buffer (128 B)


def _narrow_max_waves() -> int:
    import os
    import re

    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "depthwise_causal_conv1d_amd", "csrc", "device_common.h")
    return int(re.search(r"kNarrowMaxWaves\s*=\s*(\d+)", open(path).read()).group(1))


# The one-token update takes the 128-channel (narrow) form when rows x
# 512-channel tiles is at most this; above it, the 512-channel kernels.
NARROW_MAX_WAVES = _narrow_max_waves()


def takes_narrow(n: int, d: int) -> bool:
    return n * ((d + 511) // 512) <= NARROW_MAX_WAVES


def to_dev(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev)
    return t.view(torch.bfloat16)


def from_dev(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def guarded_copy(bits: np.ndarray, dev="cuda"):
    """Device copy of ``bits`` inside a buffer with GUARD sentinel elements on each
    side.  Returns (whole buffer, view of the payload with bits' shape)."""
    flat = np.ascontiguousarray(bits).ravel()
    host = np.full(flat.size + 2 * GUARD, FILL_SENTINEL, dtype=np.uint16)
    host[GUARD:GUARD + flat.size] = flat
    buf = to_dev(host, dev)
    return buf, buf[GUARD:GUARD + flat.size].view(bits.shape)


def guarded_empty(shape, dev="cuda"):
    n = int(np.prod(shape))
    host = np.full(n + 2 * GUARD, FILL_SENTINEL, dtype=np.uint16)
    buf = to_dev(host, dev)
    return buf, buf[GUARD:GUARD + n].view(shape)


def assert_guards_intact(buf: torch.Tensor):
    h = from_dev(buf)
    assert np.all(h[:GUARD] == FILL_SENTINEL), "write below the buffer"
    assert np.all(h[-GUARD:] == FILL_SENTINEL), "write above the buffer"


def _ordered(bits: np.ndarray) -> np.ndarray:
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    return np.abs(_ordered(a) - _ordered(b))


def assert_outputs_match(gpu_bits, ref_bits, ref_f32, exact=False, what="out"):
    g = bf16_bits_to_f32(gpu_bits).astype(np.float64)
    r = bf16_bits_to_f32(ref_bits).astype(np.float64)
    r32 = ref_f32.astype(np.float64)
    both_nan = np.isnan(g) & np.isnan(r32)
    if exact:
        bad = ~((g == r) | both_nan)
    else:
        ulp_ok = bf16_ulp_distance(gpu_bits, ref_bits) <= 1
        abs_ok = np.abs(g - r32) <= 1e-2 * np.maximum(1.0, np.abs(r32))
        bad = ~(ulp_ok | abs_ok | both_nan)
    if np.any(bad):
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} mismatches, first at {tuple(i)}: gpu {g[tuple(i)]} "
                             f"ref {r[tuple(i)]} ref_f32 {r32[tuple(i)]}")


class Case:
    """One decode-update call: host inputs, the oracle's answer, the GPU's answer."""

    def __init__(self, x, D, weight, state, layout="compact", bias=None, indices=None, act=None,
                 status=False, oracle_indices=None):
        # x: uint16 [N, ld]; state: physical uint16 [S, D, L] (compact) or [S, L, D] (channel_last)
        self.x, self.D, self.weight, self.bias, self.indices, self.act = x, D, weight, bias, indices, act
        self.layout, self.status = layout, status
        self.N, self.ld = x.shape
        if layout == "compact":
            self.S, _, self.L = state.shape
            self.strides = (D * self.L, self.L, 1)
        else:
            self.S, self.L, _ = state.shape
            self.strides = (self.L * D, 1, D)
        self.state0 = state.copy()
        # the oracle refuses bad tables; rows the library rejects behave as padding,
        # so the caller may give the table the oracle should see
        self.oracle_indices = indices if oracle_indices is None else oracle_indices

    def reference(self):
        st = self.state0.copy()
        out, out32 = oracle.update_strided(self.x, self.N, self.D, self.ld, st, self.S, self.L, self.strides,
                                           self.weight, self.bias, self.oracle_indices, self.act,
                                           want_f32=True)
        return out, out32, st

    def run_gpu(self, dev="cuda"):
        xb, xd = guarded_copy(self.x, dev)
        xv = xd[:, :self.D]
        sb, sd = guarded_copy(self.state0, dev)
        sv = sd if self.layout == "compact" else sd.permute(0, 2, 1)
        wd = to_dev(self.weight, dev)
        bd = None if self.bias is None else to_dev(self.bias, dev)
        idd = None if self.indices is None else torch.from_numpy(self.indices).to(dev)
        ob, od = guarded_empty((self.N, self.D), dev)
        stat = torch.zeros(1, dtype=torch.int32, device=dev) if self.status else None
        dc.causal_conv1d_update_out(xv, sv, wd, bd, self.act, out=od, conv_state_indices=idd, dev_status=stat)
        self.kernel = dc.dcconv_last_kernel()
        torch.cuda.synchronize()
        assert_guards_intact(sb)
        assert_guards_intact(ob)
        assert np.array_equal(from_dev(xb)[GUARD:GUARD + self.x.size].reshape(self.x.shape), self.x), "x was written"
        return from_dev(od), from_dev(sd), (int(stat.item()) if stat is not None else None)

    def check(self, exact_identity=True):
        ref_out, ref32, ref_state = self.reference()
        out, state, status = self.run_gpu()
        np.testing.assert_array_equal(state, ref_state, err_msg="state not bit-exact")
        assert_outputs_match(out, ref_out, ref32, exact=(exact_identity and self.act in (None, "identity")))
        # padding rows are zero
        if self.oracle_indices is not None:
            pad = self.oracle_indices == -1
            assert np.all(bf16_bits_to_f32(out[pad]) == 0)
        return status
