"""Host-side pieces of bench.py, on the CPU: the algorithmic byte count of a
step, the counter-file lookup and its code digest, and the refusal of more
than one GPU."""
import os
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_step_bytes_long_context():
    """4 x 8192 tokens of 2 KiB K and V rows, one layer: read 2*N*row + 4N,
    write 2*N*row."""
    sb = bench.step_bytes(workloads.get("long_context"))
    N, row = 32768, 2048
    assert (sb["R"], sb["N"]) == (4, N)
    assert sb["kv"] == 2 * N * row + 4 * N + 2 * N * row == 268566528


def test_step_bytes_decode_heavy():
    sb = bench.step_bytes(workloads.get("decode_heavy"))
    assert sb["kv"] == 32 * (4 * 256 * 2048 + 4 * 256) == 67141632
    assert sb["gather_rows"] == 256


def test_code_digest_ignores_comments_only():
    code = "int f(int x) {\n  return x + 1;  // one more\n}\n/* block\n comment */\n"
    same = "// header\nint f(int x) {   return x + 1;\n}\n"
    other = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench.code_digest(code) == bench.code_digest(same)
    assert bench.code_digest(code) != bench.code_digest(other)


def test_kernel_digest_covers_the_kv_code_only():
    """Edits to other kernels keep a kernel's counters valid; an edit to its
    own code (or to code it calls) voids them; a source without the region is
    an error."""
    with open(os.path.join(os.path.dirname(bench.__file__), "ragged_input_compilation_amd", "csrc",
                           "ric_kernels.hip"), encoding="utf-8") as f:
        text = f.read()
    base = bench.kernel_source_digest(text)
    assert base == bench.kernel_source_digest()
    other = text.replace("__global__ __launch_bounds__(kCompileThreads) void compile_kernel(CompileParams p) {",
                         "__global__ __launch_bounds__(kCompileThreads) void compile_kernel(CompileParams p) { int z = 0;")
    assert other != text and bench.kernel_source_digest(other) == base
    kv = text.replace("const int C = p.row_bytes >> 4;", "const int C = (p.row_bytes >> 4) + 0;", 1)
    assert kv != text and bench.kernel_source_digest(kv) != base
    with pytest.raises(ValueError):
        bench.kernel_source_digest(text.replace("u32x4 load16(", "u32x4 load_16("))
    # the single compile + K/V kernel depends on the compile's code and the K/V
    # helpers too; the compile kernel's own counters only on the compile's code
    fused = bench.kernel_source_digest(text, "compile_kv")
    comp = bench.kernel_source_digest(text, "compile")
    edit_scan = text.replace("const int per = (R + kCompileThreads - 1) / kCompileThreads;",
                             "const int per = (R + kCompileThreads - 1) / kCompileThreads + 0;", 1)
    assert edit_scan != text
    assert bench.kernel_source_digest(edit_scan, "compile_kv") != fused
    assert bench.kernel_source_digest(edit_scan, "compile") != comp
    assert bench.kernel_source_digest(edit_scan, "kv") == base
    assert bench.kernel_source_digest(kv, "compile") == comp
    assert bench.kernel_source_digest(kv, "compile_kv") != fused


def test_load_traffic_needs_matching_code(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "kv_chunk_kernel_x_pmc.md").write_text(
        "traffic_bytes_per_launch: 123\nkernel_code_sha256: " + "0" * 64 + "\n")
    (prof / "kv_chunk_kernel_y_pmc.md").write_text(
        "traffic_bytes_per_launch: 456\nkernel_code_sha256: " + bench.kernel_source_digest() + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda region="kv": bench.code_digest("x"))
    assert bench.load_traffic("kv_chunk_kernel", "x") is None
    assert bench.load_traffic("kv_chunk_kernel", "missing") is None
    (prof / "kv_chunk_kernel_z_pmc.md").write_text(
        "traffic_bytes_per_launch: 789\nkernel_code_sha256: " + bench.code_digest("x") + "\n")
    assert bench.load_traffic("kv_chunk_kernel", "z") == 789


@pytest.mark.parametrize("gpus", [2, 8])
def test_more_than_one_gpu_is_refused(gpus):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(gpus)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_library_path_rule():
    """The bench's mirror of the library's choice: one kernel for rows of
    128, 256 and 512 B, and for rows of 1, 2, 3, 4, 6 and 8 KiB unless the
    step averages 1024 or more tokens per request; other row sizes take two
    kernels."""
    import dataclasses
    for name in ("churn", "mixed", "decode_heavy", "worked_example"):     # the last: 256 B rows
        assert bench.fused_path(workloads.get(name)), name
    lc = workloads.get("long_context")
    assert not bench.fused_path(lc)
    assert bench.fused_path(dataclasses.replace(lc, kv_heads=1))        # 256 B rows: long runs too
    assert bench.fused_path(dataclasses.replace(lc, kv_heads=2))
    assert bench.fused_path(dataclasses.replace(workloads.get("mixed"), kv_heads=12))       # 3 KiB rows
    assert not bench.fused_path(dataclasses.replace(lc, kv_heads=32))                       # 8 KiB long runs
    assert not bench.fused_path(dataclasses.replace(workloads.get("mixed"), kv_heads=6))    # 1.5 KiB rows
    assert bench.fused_path(dataclasses.replace(workloads.get("worked_example"), kv_heads=1))       # 128 B
    assert not bench.fused_path(dataclasses.replace(workloads.get("worked_example"), kv_heads=1, head_dim=32))
    assert bench.dominant_kernel(workloads.get("churn"), 16384) == "compile_kv_kernel"
    assert bench.dominant_kernel(lc, 32768) == "kv_chunk_kernel"
    assert bench.dominant_kernel(workloads.get("worked_example"), 32) == "compile_kv_kernel"


def test_cpu_baseline_parallel_equals_single(tmp_path):
    """The all-cores CPU step (request ranges compiled on threads, K/V rows
    split by tokens over every thread, then the running totals, compaction and
    padding) gives the single-thread oracle's outputs; cpu_baseline itself
    asserts this before timing."""
    pool = len(os.sched_getaffinity(0))
    w = workloads.get("worked_example")
    res = bench.cpu_baseline(w, 0.2)
    assert res["kind"] == "oracle" and res["cores"] == 1 and res["value"] > 0
    assert 1 <= res["all_cores"]["compile_threads"] <= min(3, pool)
    assert 1 <= res["all_cores"]["cores"] <= pool
    res = bench.cpu_baseline(workloads.get("mixed"), 0.5)
    assert 1 <= res["all_cores"]["compile_threads"] <= min(124, pool)
    assert res["all_cores"]["cores"] >= res["all_cores"]["compile_threads"]
    assert res["all_cores"]["value"] > 0
