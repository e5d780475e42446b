"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): a sanitized build runs the golden pins, a cross-check against the
Python oracle on random batches, and the K/V scatter and gather, in a child
process with the ASan runtime preloaded.  Any out-of-bounds access or
undefined behaviour aborts the child."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import ctypes, sys
import numpy as np
sys.path.insert(0, {root!r})
from oracle import cbind, step
from tests.oracle_helpers import KEYS, rows_of
from tests.test_oracle_mutations import _pin_suite, _c_runner
import workloads

lib = ctypes.CDLL({so!r})
lib.nano_compile.argtypes = [ctypes.POINTER(cbind._In), ctypes.POINTER(cbind._Out)]
lib.nano_compile.restype = ctypes.c_int
lib.nano_kv_scatter.argtypes = [ctypes.c_void_p] * 4 + [cbind._i32p, ctypes.c_int32, ctypes.c_int64]
lib.nano_kv_scatter.restype = None
lib.nano_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, cbind._i32p, ctypes.c_int32, ctypes.c_void_p]
lib.nano_gather.restype = None
_pin_suite(_c_runner(lib))
cbind._lib = lib

rng = np.random.default_rng(8)
for trial in range(150):
    B = int(rng.choice([1, 2, 3, 4, 7, 16]))
    R = int(rng.integers(1, 7))
    reqs = workloads.random_batch(rng, num_reqs=R, block_size=B, max_model_len=128, num_kv_blocks=400,
                                  max_q=12, max_c=60)
    rows = rows_of(reqs)
    N = sum(r.num_scheduled for r in rows)
    n_pad = N + int(rng.integers(0, 5))
    MR = R + int(rng.integers(0, 3))
    want = step.compile_step(rows, block_size=B, max_num_reqs=MR, max_model_len=128,
                             max_num_batched_tokens=n_pad, num_kv_blocks=400, n_pad=n_pad)
    got = cbind.compile_step(rows, block_size=B, max_num_reqs=MR, n_pad=n_pad)
    for k in KEYS:
        assert [int(x) for x in got[k]] == [int(x) for x in want[k]], (trial, k)

    row = 16 * int(rng.integers(1, 5))
    k_src = rng.integers(0, 256, (n_pad, row), dtype=np.uint8)
    v_src = rng.integers(0, 256, (n_pad, row), dtype=np.uint8)
    slots = np.asarray(want["slot_mapping"], np.int32)
    kc = np.zeros((400 * B, row), np.uint8)
    vc = np.zeros((400 * B, row), np.uint8)
    lib.nano_kv_scatter(k_src.ctypes.data, v_src.ctypes.data, kc.ctypes.data, vc.ctypes.data,
                        slots.ctypes.data_as(cbind._i32p), n_pad, row)
    assert np.array_equal(kc[slots[:N]], k_src[:N]) and np.array_equal(vc[slots[:N]], v_src[:N])
    idx = np.asarray(want["logits_indices"][:R], np.int32)
    out = np.zeros((R, row), np.uint8)
    lib.nano_gather(k_src.ctypes.data, row, idx.ctypes.data_as(cbind._i32p), R, out.ctypes.data)
    assert np.array_equal(out, k_src[idx])
print("sanitized oracle ok")
"""


def _asan_runtime():
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime for gcc here")
    return asan


def _run_sanitized(src_text, tmp_path):
    src = tmp_path / "nano_oracle.c"
    src.write_text(src_text, encoding="utf-8")
    so = tmp_path / "nano_oracle_sanitized.so"
    subprocess.run(["gcc", "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", str(src), "-o", str(so)], check=True)
    preload = ":".join(x for x in (_asan_runtime(), os.environ.get("LD_PRELOAD", "")) if x)   # ASan first
    env = {**os.environ, "LD_PRELOAD": preload, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1"}
    return subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT, so=str(so))], capture_output=True,
                          text=True, timeout=300, env=env)


def _oracle_source():
    with open(os.path.join(ROOT, "oracle", "nano_oracle.c"), encoding="utf-8") as f:
        return f.read()


def test_c_oracle_under_asan_and_ubsan(tmp_path):
    child = _run_sanitized(_oracle_source(), tmp_path)
    assert child.returncode == 0, child.stderr[-3000:]
    assert "sanitized oracle ok" in child.stdout
    assert "AddressSanitizer" not in child.stderr and "runtime error" not in child.stderr


def test_sanitizer_catches_a_planted_overrun(tmp_path):
    """The harness really checks: a copy of the oracle whose gather writes one
    row past its output (planted here, on the CPU) is stopped by ASan."""
    src = _oracle_source()
    old = "for (m = 0; m < count; ++m) {"
    assert src.count(old) == 1
    child = _run_sanitized(src.replace(old, "for (m = 0; m <= count; ++m) {"), tmp_path)
    assert child.returncode != 0
    assert "AddressSanitizer" in child.stderr
