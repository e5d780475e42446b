"""Planted mistakes: copies of each oracle formulation with one plausible error
(a dropped term, a transposed operand, an off-by-one, a wrong comparison) must
fail the golden pins.  The mistakes are planted in oracle copies on the CPU."""
import ctypes
import os
import subprocess
import sys
import types

import numpy as np
import pytest

import oracle.step as step_mod
import oracle.vectorised as vec_mod
from oracle import cbind
from tests.oracle_helpers import Row, golden, labelled_rows

ORACLE_DIR = os.path.dirname(step_mod.__file__)


def _pin_suite(run):
    """``run(rows, B, max_num_reqs, n_pad)`` -> dict of sequences.  Raises on
    the first pin that does not hold."""
    def eq(a, b, what):
        if [int(x) for x in a] != [int(x) for x in b]:
            raise AssertionError(what)

    g = golden("scan_2_5_3.json")
    q = g["num_scheduled"]
    r = run(labelled_rows([0, 0, 0], q, q, 16), 16, 3, 10)
    eq(r["query_start_loc"], g["expect"]["query_start_loc"], "scan qsl")
    eq(r["req_indices"], g["expect"]["req_indices"], "scan req")
    eq(r["logits_indices"], g["expect"]["logits_indices"], "scan logits")

    g = golden("p1_worked_example.json")
    rows = labelled_rows(g["num_computed"], g["num_scheduled"], g["num_prompt"], 4, blocks=g["blocks"])
    r = run(rows, 4, 3, 6)
    for k in ("input_ids", "positions", "seq_lens", "slot_mapping", "logits_indices", "query_start_loc"):
        eq(r[k], g["expect"][k], "p1 " + k)
    if int(r["discard"][1]) != 1:
        raise AssertionError("p1 discard")

    for name in ("p3_layout.json", "p3_verify_step2.json", "p1_min_repro.json"):
        g = golden(name)
        rows = labelled_rows(g["num_computed"], g["num_scheduled"], g["num_prompt"], 16)
        r = run(rows, 16, len(rows), sum(g["num_scheduled"]))
        for k, v in g["expect"].items():
            if k in r and isinstance(v, list):
                eq(r[k], v, name + " " + k)

    g = golden("p3_exercise1.json")
    rows = labelled_rows(g["num_computed"], g["num_scheduled"], g["num_prompt"], 16)
    r = run(rows, 16, 3, 11)
    eq(list(r["sample_indices"])[:2], g["expect"]["sample_indices"], "exercise sample")
    if int(r["sample_indices"][2]) != -1:
        raise AssertionError("exercise sample tail")

    g = golden("p5_slot_ranges.json")
    rows = [Row(1, 37, 38, np.arange(38), np.asarray(g["blocks"]))]
    r = run(rows, 8, 1, 37)
    eq(r["slot_mapping"], [s for a, b in g["expect"]["ranges"] for s in range(a, b)], "p5 ranges")

    rows = labelled_rows([5, 0], [1, 2], [6, 2], 4)
    r = run(rows, 4, 4, 8)
    eq(r["slot_mapping"][3:], [0] * 5, "pad slots")
    eq(r["req_indices"][3:], [-1] * 5, "pad req")
    eq(r["query_start_loc"], [0, 1, 3, 3, 3], "pad qsl")
    eq(r["seq_lens"], [6, 2, 0, 0], "pad seq")


def _py_runner(mod):
    def run(rows, B, R, n_pad):
        return mod.compile_step(rows, block_size=B, max_num_reqs=R, max_model_len=1 << 20,
                                max_num_batched_tokens=1 << 20, num_kv_blocks=1 << 20,
                                n_pad=n_pad, check_unique_slots=False)
    return run


def _np_runner(mod):
    def run(rows, B, R, n_pad):
        tok, blk = cbind.pack_tables(rows)
        return mod.compile_arrays([r.num_computed for r in rows], [r.num_scheduled for r in rows],
                                  [r.num_prompt for r in rows], tok, blk, block_size=B,
                                  max_num_reqs=R, n_pad=n_pad)
    return run


def _mutant_module(path, old, new, name):
    src = open(path, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType(name)
    exec(compile(src.replace(old, new), name, "exec"), mod.__dict__)
    return mod


PY_MUTANTS = [
    ("pos = r.num_computed + (t - qsl[owner])", "pos = t - qsl[owner]"),       # dropped term
    ("block_index, within = divmod(pos, B)", "within, block_index = divmod(pos, B)"),  # transposed
    ("while qsl[owner + 1] <= t:", "while qsl[owner + 1] < t:"),                   # boundary token to the wrong request
    ("logits_indices.append(qsl[i + 1] - 1)", "logits_indices.append(qsl[i + 1])"),     # off by one
    ("1 if r.num_computed + r.num_scheduled < r.num_prompt else 0",
     "1 if r.num_computed + r.num_scheduled <= r.num_prompt else 0"),            # wrong comparison
    ("seq_lens.append(r.num_computed + r.num_scheduled)", "seq_lens.append(r.num_scheduled)"),
    ("input_ids.append(int(r.tokens[pos]))", "input_ids.append(int(r.tokens[t - qsl[owner]]))"),
    ("slot_mapping.append(int(r.blocks[block_index]) * B + within)",
     "slot_mapping.append(int(r.blocks[block_index]) + within * B)"),
    ("qsl.append(qsl[-1] + r.num_scheduled)", "qsl.append(qsl[-1] + r.num_scheduled - 1)"),
    ("slot_mapping.append(null_block * B)", "slot_mapping.append(-1)"),
    ("for _ in range(R, max_num_reqs):\n        qsl.append(N)", "for _ in range(R, max_num_reqs):\n        qsl.append(0)"),
]

NP_MUTANTS = [
    ("starts = cu - q ", "starts = cu "),
    ("positions // block_size)", "positions % block_size)"),
    ("req_indices * M + positions", "req_indices + positions * M"),
    ("logits[:R] = qsl[1:R + 1] - 1", "logits[:R] = qsl[:R]"),
    ("discard[:R] = (c + q < P)", "discard[:R] = (c + q > P)"),
]

C_MUTANTS = [
    ("const int32_t lo = cached > b * B ? cached : b * B;", "const int32_t lo = b * B;"),        # offset in the first block dropped
    ("for (b = cached / B; b * B < total; ++b) {", "for (b = cached / B; (b + 1) * B <= total; ++b) {"),  # partial last block dropped
    ("const int32_t hi = total < (b + 1) * B ? total : (b + 1) * B;", "const int32_t hi = (b + 1) * B;"),  # whole last block
    ("out->slot_mapping[n + (p - cached)] = owned[b] * B + (p - b * B);",
     "out->slot_mapping[n + (p - cached)] = owned[b] * B + (p - cached);"),                          # offset from the wrong origin
    ("out->logits_indices[i] = out->query_start_loc[i + 1] - 1;",
     "out->logits_indices[i] = out->query_start_loc[i];"),
    ("out->positions[n + k] = cached + k;", "out->positions[n + k] = k;"),
]


def test_unmutated_oracles_pass_the_pins():
    _pin_suite(_py_runner(step_mod))
    _pin_suite(_np_runner(vec_mod))
    _pin_suite(_c_runner(cbind.lib()))


@pytest.mark.parametrize("old,new", PY_MUTANTS)
def test_python_mutant_is_caught(old, new):
    mod = _mutant_module(step_mod.__file__, old, new, "step_mutant")
    with pytest.raises(Exception):
        _pin_suite(_py_runner(mod))


@pytest.mark.parametrize("old,new", NP_MUTANTS)
def test_numpy_mutant_is_caught(old, new):
    mod = _mutant_module(vec_mod.__file__, old, new, "vec_mutant")
    with pytest.raises(Exception):
        _pin_suite(_np_runner(mod))


def _c_runner(lib):
    def run(rows, B, R, n_pad):
        saved = cbind._lib
        try:
            cbind._lib = lib
            return cbind.compile_step(rows, block_size=B, max_num_reqs=R, n_pad=n_pad)
        finally:
            cbind._lib = saved
    return run


_C_CHILD = """
import ctypes, sys
sys.path.insert(0, {root!r})
from oracle import cbind
from tests.test_oracle_mutations import _pin_suite, _c_runner
lib = ctypes.CDLL({so!r})
lib.nano_compile.argtypes = [ctypes.POINTER(cbind._In), ctypes.POINTER(cbind._Out)]
lib.nano_compile.restype = ctypes.c_int
_pin_suite(_c_runner(lib))
"""


@pytest.mark.parametrize("old,new", C_MUTANTS)
def test_c_mutant_is_caught(old, new, tmp_path):
    """Each C mutant runs the pins in a child process: a failed pin or a crash
    (a mutant may write past its output arrays) both count as caught."""
    src = open(os.path.join(ORACLE_DIR, "nano_oracle.c"), encoding="utf-8").read()
    assert src.count(old) == 1
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new), encoding="utf-8")
    so = tmp_path / "mutant.so"
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", str(path), "-o", str(so)])
    root = os.path.dirname(ORACLE_DIR)
    child = subprocess.run([sys.executable, "-c", _C_CHILD.format(root=root, so=str(so))],
                           capture_output=True, timeout=120)
    assert child.returncode != 0


def test_c_child_script_passes_unmutated():
    """The child script itself works: with the real oracle library it exits 0,
    so a mutant's non-zero exit comes from the mutation."""
    from oracle import build
    root = os.path.dirname(ORACLE_DIR)
    child = subprocess.run([sys.executable, "-c", _C_CHILD.format(root=root, so=build.LIB)],
                           capture_output=True, timeout=120)
    assert child.returncode == 0, child.stderr.decode()[-2000:]
