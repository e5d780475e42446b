"""The C-ABI library on the CPU: it loads, exports every entry point the
header declares, and its host-only helpers (padded size, condense plan, step
check) agree with the oracle.  No device work is issued here."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import workloads
from oracle import batch as ref_batch, step as ref_step
from tests.oracle_helpers import golden, rows_of

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ric.h")


def _declared():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ric_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def ric():
    from ragged_input_compilation_amd import _ric
    return _ric


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("ric_create", "ric_schedule", "ric_compile", "ric_reshape_and_cache", "ric_gather_rows",
              "ric_condense", "ric_padded_size"):
        assert n in names


def test_library_exports_every_declared_symbol(ric):
    out = subprocess.run(["nm", "-D", "--defined-only", ric.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (ric_\w+)", out))
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    for n in _declared():
        assert hasattr(ric.lib(), n)
        assert hasattr(ric, n), f"binding lacks {n}"


def test_library_is_gfx950_code(ric):
    """The shared object carries a gfx950 code object (offload bundle)."""
    blob = open(ric.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_padded_size_pins(ric):
    g = golden("p2_padding.json")
    for n, padded, _ in g["cases"]:
        assert ric.ric_padded_size(g["capture_sizes"], n) == padded
        assert ric.ric_padded_size(list(reversed(g["capture_sizes"])), n) == padded
    assert ric.ric_padded_size(g["capture_sizes"], 1000) == 1000
    assert ric.ric_padded_size([], 7) == 7
    rng = np.random.default_rng(0)
    for _ in range(200):
        sizes = sorted(set(rng.integers(1, 600, size=int(rng.integers(1, 20))).tolist()))
        n = int(rng.integers(0, 700))
        assert ric.ric_padded_size(sizes, n) == ref_step.padded_size(sizes, n)
    with pytest.raises(ric.RicError):
        ric.ric_padded_size([1, 2], -1)


def test_condense_plan_matches_oracle(ric):
    g = golden("p1_condense.json")
    # A B C D with B removed: D moves into row 1
    assert ric.ric_condense_plan([1, 0, 1, 1]) == [(1, 3)]
    rng = np.random.default_rng(1)
    for _ in range(300):
        n = int(rng.integers(0, 40))
        live = rng.random(n) < rng.random()
        b = ref_batch.RefBatch(max(n, 1), 4, 1, 10)
        for i in range(n):
            b.add_request(i, [0], 1, 0, [1])
        for i in range(n):
            if not live[i]:
                b.remove_request(i)
        assert ric.ric_condense_plan(live.astype(np.uint8)) == b.condense_pairs()
    assert g["expect"]["rows"] == ["A", "D", "C"]


def _cfg(ric, w):
    return ric.make_config(max_num_reqs=w.max_num_reqs, max_model_len=w.max_model_len,
                           block_size=w.block_size, max_blocks_per_req=w.max_blocks_per_req,
                           max_num_batched_tokens=w.max_num_batched_tokens,
                           num_kv_blocks=w.num_kv_blocks, null_block=0, staging_bytes=0)


@pytest.mark.parametrize("name", ["worked_example", "decode_heavy", "mixed", "long_context"])
def test_check_step_scalars_match_oracle(ric, name):
    w = workloads.get(name)
    reqs = w.live_requests()
    rows = rows_of(reqs)
    n = sum(r.num_scheduled for r in rows)
    n_pad = ref_step.padded_size(w.capture_sizes, n)
    ref = ref_step.compile_step(rows, block_size=w.block_size, max_num_reqs=w.max_num_reqs,
                                max_model_len=w.max_model_len, max_num_batched_tokens=w.max_num_batched_tokens,
                                num_kv_blocks=w.num_kv_blocks, n_pad=n_pad)
    s = ric.ric_check_step(_cfg(ric, w), [r.num_computed for r in reqs], [r.num_scheduled for r in reqs],
                           [r.num_prompt for r in reqs], [r.num_tokens for r in reqs],
                           [len(r.blocks) for r in reqs], n_pad)
    assert (s.num_reqs, s.num_actual_tokens, s.num_tokens_padded, s.max_query_len, s.max_seq_len,
            s.num_sampled) == (len(reqs), ref["num_actual_tokens"], n_pad, ref["max_query_len"],
                               ref["max_seq_len"], ref["num_sampled"])


def test_check_step_rejects_what_the_oracle_rejects(ric):
    cfg = ric.make_config(max_num_reqs=4, max_model_len=16, block_size=4, max_blocks_per_req=4,
                          max_num_batched_tokens=8, num_kv_blocks=10, null_block=0, staging_bytes=0)
    ok = dict(num_computed=[0], num_scheduled=[2], num_prompt=[2], num_tokens=[2], num_blocks=[1])
    ric.ric_check_step(cfg, *ok.values(), 4)
    bad = [
        dict(ok, num_scheduled=[0]),                       # nothing scheduled
        dict(ok, num_computed=[1]),                        # c + q beyond the history
        dict(ok, num_scheduled=[5], num_tokens=[5], num_prompt=[5]),  # too few blocks
        dict(ok, num_computed=[-1]),
    ]
    for b in bad:
        with pytest.raises(ric.RicError) as e:
            ric.ric_check_step(cfg, *b.values(), 4)
        assert e.value.code == ric.RIC_EINVAL
    with pytest.raises(ric.RicError):
        ric.ric_check_step(cfg, *ok.values(), 1)           # N_pad < N
    with pytest.raises(ric.RicError):
        ric.ric_check_step(cfg, *ok.values(), 9)           # N_pad > budget
    many = dict(num_computed=[0, 0], num_scheduled=[5, 4], num_prompt=[5, 4], num_tokens=[5, 4],
                num_blocks=[2, 1])
    with pytest.raises(ric.RicError):
        ric.ric_check_step(cfg, *many.values(), 8)         # 9 tokens > budget 8


def test_config_validation(ric):
    base = dict(max_num_reqs=4, max_model_len=16, block_size=4, max_blocks_per_req=4,
                max_num_batched_tokens=8, num_kv_blocks=10, null_block=0, staging_bytes=0)
    assert ric.ric_workspace_bytes(ric.make_config(**base)) > 0
    for bad in (dict(max_num_reqs=0), dict(max_num_reqs=9000), dict(block_size=0),
                dict(null_block=10), dict(num_kv_blocks=1 << 28, block_size=16), dict(staging_bytes=-1)):
        assert ric.ric_workspace_bytes(ric.make_config(**{**base, **bad})) == 0


def test_group_config_validation(ric):
    good = dict(max_num_reqs=4, max_model_len=64, block_size=16, max_blocks_per_req=4, max_num_batched_tokens=8,
                num_kv_blocks=10, null_block=0, staging_bytes=0, num_kv_groups=2, group_block_size=[0, 8],
                group_num_kv_blocks=[0, 0], group_slot_mode=[0, 0])
    one = ric.ric_workspace_bytes(ric.make_config(**{**good, "num_kv_groups": 1}))
    two = ric.ric_workspace_bytes(ric.make_config(**good))
    # a second group adds a [4][8] block table and a slot output of 8 entries
    assert two > one > 0
    assert ric.ric_workspace_bytes(ric.make_config(**{**good, "group_slot_mode": [0, 1]})) < two
    for bad in (dict(num_kv_groups=5), dict(num_kv_groups=-1), dict(group_block_size=[0, 0]),
                dict(group_slot_mode=[0, 7]), dict(group_num_kv_blocks=[0, -1]),
                dict(group_block_size=[0, 1 << 20], group_num_kv_blocks=[0, 1 << 12])):
        assert ric.ric_workspace_bytes(ric.make_config(**{**good, **bad})) == 0


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_workspace_fits(ric, name):
    w = workloads.get(name)
    nbytes = ric.ric_workspace_bytes(_cfg(ric, w))
    table = w.max_num_reqs * (w.max_model_len + w.max_blocks_per_req) * 4
    assert table <= nbytes < table + (64 << 20)


def build_c_step(out_path, ric):
    """Compile the plain-C step program against the library and ric.h."""
    src = os.path.join(ROOT, "tests", "c_abi_step.c")
    libdir = os.path.dirname(ric.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", src, "-o", str(out_path),
                    "-L", libdir, "-l:" + os.path.basename(ric.LIB_PATH), "-L", "/opt/rocm/lib", "-lamdhip64",
                    f"-Wl,-rpath,{libdir}"],
                   check=True, capture_output=True, text=True)
    return str(out_path)


def test_header_is_plain_c_and_links_from_c(ric, tmp_path):
    """ric.h compiles as C99 and a C program links against libric.so with
    no C++ runtime of its own (the GPU test runs it)."""
    exe = build_c_step(tmp_path / "c_abi_step", ric)
    assert os.path.getsize(exe) > 0


def test_launch_size_limits_are_checked_before_any_device_work(ric):
    """Per-call row limits (2^24: the grid's work-item count stays within 32
    bits) and non-zero reserved flags are rejected by validation alone, so
    these calls are safe without a GPU."""
    big = (1 << 24) + 1
    with pytest.raises(ric.RicError) as e:
        ric.ric_reshape_and_cache([16], [16], [16], [16], 16, big, 64, 1024)
    assert e.value.code == ric.RIC_EINVAL
    with pytest.raises(ric.RicError) as e:
        ric.ric_reshape_and_cache([16], [16], [16], [16], 16, 4, 64, 1024, flags=1)
    assert e.value.code == ric.RIC_EINVAL
    with pytest.raises(ric.RicError) as e:
        ric.ric_gather_rows(16, 64, 4, 16, 0, big, 64, 16)
    assert e.value.code == ric.RIC_EINVAL
    ric.ric_reshape_and_cache([16], [16], [16], [16], 16, 0, 64, 1024)    # nothing to do: no launch
    ric.ric_gather_rows(16, 64, 4, 16, 0, 0, 64, 16)


def test_binding_fails_loudly_without_the_library(tmp_path):
    """A copy of the package without libric.so cannot be imported: there is
    no fallback implementation to fall back to."""
    import shutil
    pkg = os.path.join(ROOT, "ragged_input_compilation_amd")
    dst = tmp_path / "ragged_input_compilation_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    code = "import ragged_input_compilation_amd._ric"
    r = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), capture_output=True, text=True,
                       timeout=120, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "is not built" in r.stderr


def test_struct_layouts_match_the_header(ric, tmp_path):
    """Every field of the header's structs sits at the same offset, with the
    same size, in the C compiler's layout and in the ctypes mirrors."""
    structs = {"ric_config": ric.ric_config, "ric_sampling": ric.ric_sampling, "ric_step": ric.ric_step,
               "ric_columns": ric.ric_columns, "ric_spec_decode": ric.ric_spec_decode}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "ric.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'    printf("{name} sizeof %zu\\n", sizeof({name}));')
        for field, _ in cls._fields_:
            lines.append(f'    printf("{name} {field} %zu %zu\\n", offsetof({name}, {field}), '
                         f'sizeof((({name}*)0)->{field}));')
    lines += ["    return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    for line in filter(None, out):
        parts = line.split()
        cls = structs[parts[0]]
        if parts[1] == "sizeof":
            assert int(parts[2]) == ctypes.sizeof(cls), line
        else:
            desc = getattr(cls, parts[1])
            assert (desc.offset, desc.size) == (int(parts[2]), int(parts[3])), line
