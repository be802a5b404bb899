"""Planted mistakes in the oracle are caught by its pins (CPU).

Each case below is one plausible slip in ``oracle/dcconv_oracle.c`` -- a tap read
from the wrong end of the history, a dropped bias, a missing shift, truncating
rounding, the wrong sign in SiLU, a padding row that writes, a stride ignored, a
token dropped, a final state or ring position off by one.  The test builds the
oracle with that one change, runs the oracle's pin tests against the broken build
(``test_oracle_pins.py``, ``test_oracle_ring_pins.py``,
``test_oracle_prefill_pins.py``; they compare it with float64 library
convolutions, closed forms, hand-worked examples and routing laws) and requires
them to fail.  The unchanged source, built the same way, must pass them.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "dcconv_oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_pins.py", "test_oracle_ring_pins.py",
                                                  "test_oracle_prefill_pins.py")]

# (name, exact text in the oracle, its replacement): each text occurs once.
MISTAKES = [
    ("tap window one place too old", "hist[l + 1 - w + j]", "hist[l - w + j]"),
    ("taps in reverse order", "acc = acc + hist[l + 1 - w + j] * oracle_bf16_to_f32(weight[c * w + j]);",
     "acc = acc + hist[l + 1 - w + j] * oracle_bf16_to_f32(weight[c * w + (w - 1 - j)]);"),
    ("bias dropped in the update",
     "            if (bias)\n                acc = acc + oracle_bf16_to_f32(bias[c]);\n            float y = act_apply(acc, activation);\n            if (out_f32)\n                out_f32[n * os_n",
     "            if (bias)\n                acc = acc;\n            float y = act_apply(acc, activation);\n            if (out_f32)\n                out_f32[n * os_n"),
    ("state not shifted", "slot[k * st_l] = hist_bits[k + 1];", "slot[k * st_l] = hist_bits[k];"),
    ("rounding truncates", "u += 0x7fffu + keep_lsb;", "u += 0u * keep_lsb;"),
    ("NaN payload lost", "return (uint16_t)((u >> 16) | 0x0040u);", "return (uint16_t)(u >> 16);"),
    ("SiLU with the wrong sign", "acc / (1.0f + expf(-acc))", "acc / (1.0f + expf(acc))"),
    ("padding row writes one", "                out[n * os_n + c * os_d] = 0;",
     "                out[n * os_n + c * os_d] = 0x3f80;"),
    ("x channel stride ignored", "hist_bits[l] = x[n * xs_n + c * xs_d];", "hist_bits[l] = x[n * xs_n + c];"),
    ("duplicate slots accepted", "if (seen[s]) {", "if (0) {"),
    ("every token reads the first token", "update_rows(x + t * xs_t,", "update_rows(x,"),
    ("every token writes the first output", "slot_of_row, activation, out + t * os_t,", "slot_of_row, activation, out,"),
    ("last token dropped", "for (int64_t t = 0; t < t_steps; ++t)", "for (int64_t t = 0; t + 1 < t_steps; ++t)"),
    ("prefill taps in reverse order", "oracle_bf16_to_f32(ext[l + j - (w - 1) + k])",
     "oracle_bf16_to_f32(ext[l + j - (w - 1) + (w - 1 - k)])"),
    ("prefill keeps the initial state", "sc[k * st_l] = ext[len + k];", "sc[k * st_l] = ext[k];"),
    ("prefill ignores has_init", "int from_state = state != NULL && has_init != NULL && has_init[i] != 0;",
     "int from_state = state != NULL;"),
    ("packed prefill ignores the token stride", "const uint16_t *xi = starts ? x + (int64_t)starts[i] * xs_t",
     "const uint16_t *xi = starts ? x + (int64_t)starts[i]"),
    ("ring taps one token too old", "int64_t tok = seen + 1 - w + j;", "int64_t tok = seen - w + j;"),
    ("ring writes the wrong position", "ring[(seen % l) * st_l] = xb;", "ring[((seen + 1) % l) * st_l] = xb;"),
    ("BF16 read from the wrong half", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
]


def _build(source: str, path: str) -> None:
    c_path = path[:-3] + ".c"
    with open(c_path, "w") as f:
        f.write(source)
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
                    "-o", path, c_path, "-lm"], check=True)


def _run_pins(library: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, DCCONV_ORACLE_LIBRARY=library)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                           *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_every_planted_mistake_is_caught(tmp_path):
    source = open(SRC).read()
    builds = [("unchanged", str(tmp_path / "unchanged.so"), source)]
    for k, (name, old, new) in enumerate(MISTAKES):
        assert source.count(old) == 1, f"{name}: the text to change must occur exactly once"
        builds.append((name, str(tmp_path / f"mistake{k}.so"), source.replace(old, new)))
    for _, path, src in builds:
        _build(src, path)
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(lambda b: _run_pins(b[1]), builds))
    control = results[0]
    assert control.returncode == 0, "the unchanged oracle must pass its pins:\n" + control.stdout[-2000:]
    missed = [b[0] for b, r in zip(builds[1:], results[1:]) if r.returncode != 1]
    assert not missed, f"planted mistakes the pins did not catch (or that crashed): {missed}"
