"""ric_compile_and_cache (the compile and the K/V write of up to 32 layers in
one kernel for rows of 128 B to 8 KiB) against the CPU oracle: every compile
output bit-exact, every byte of every cache (real rows at the oracle's slots,
the sentinel everywhere else outside the null block), on the full-size
configurations, on random batches across block sizes, row sizes and padded
sizes, past 32 layers, and on rows the fused kernel does not take."""
import numpy as np
import pytest
import torch

import workloads
from oracle import vectorised
from tests.gpu_helpers import assert_step_equal, check_cache_exact, expected_step, replay_history

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_input_compilation_amd import _ric, runner
    return _ric, runner


def _prepare(rt, w):
    ric, runner = rt
    b = runner.Batch(runner.config_of(w))
    b.load_history(w)
    ref, order = replay_history(w)
    assert b.row_order() == order
    b.schedule_from(w, order)
    exp = expected_step(w, ref, use_python=(w.name == "worked_example"))
    return b, exp


def _expected_path(w, exp, flags):
    """The path ric_compile_and_cache reports (ric_step.kv_path) by its rule:
    1 (one kernel) for rows of 128, 256 or 512 B or 1, 2, 3, 4, 6 or 8 KiB,
    unless flags force two kernels or the rows are 1 KiB or more and the step
    averages 1024 or more tokens per request (without RIC_FUSE_ALWAYS); else
    2 (the compile kernel, then the K/V kernel)."""
    supported = w.row_bytes in (128, 256, 512, 1024, 2048, 3072, 4096, 6144, 8192)
    long_runs = exp["num_actual_tokens"] >= 1024 * max(exp["num_reqs"], 1)
    if not supported or flags == NEVER or exp["n_pad"] == 0:
        return 2
    if flags == ALWAYS:
        return 1
    return 2 if (long_runs and w.row_bytes >= 1024) else 1


def _fused_step(rt, w, b, exp, sentinel, host_sources=False, layers=None, flags=0):
    ric, runner = rt
    L = w.num_layers if layers is None else layers
    kc, vc = runner.alloc_caches(w, L, fill=sentinel)
    k, v = runner.alloc_sources(w, exp["n_pad"], seed=w.seed + 29, num_layers=L, host=host_sources)
    kv = runner.KVSet(k, v, kc, vc, w.row_bytes, w.num_kv_blocks * w.block_size)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = runner.compile_and_cache(b, exp["n_pad"], kv, dev_status=status.data_ptr(), flags=flags)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert (s.num_reqs, s.num_actual_tokens, s.num_tokens_padded) == (exp["num_reqs"], exp["num_actual_tokens"],
                                                                      exp["n_pad"])
    assert s.kv_path == _expected_path(w, exp, flags), (w.name, w.row_bytes, flags, s.kv_path)
    return s, kv


def _check_all(w, exp, kv, sentinel, label):
    B = w.block_size
    nslots = w.num_kv_blocks * B
    null = (w.null_block * B, w.null_block * B + B)
    for l in range(len(kv.k)):
        for nm, src, cache in (("K", kv.k[l], kv.kc[l]), ("V", kv.v[l], kv.vc[l])):
            check_cache_exact(cache, src, exp["slot_mapping"], exp["num_actual_tokens"], sentinel, nslots, null,
                              f"{label} layer {l} {nm}")


ALWAYS, NEVER = 1, 2
CASES = [(n, 0) for n in ("worked_example", "decode_heavy", "mixed", "churn", "long_context", "long_context_forced")] + \
    [("long_context", ALWAYS), ("long_context_forced", ALWAYS), ("mixed", NEVER), ("churn", NEVER),
     ("decode_heavy", NEVER)]


@pytest.mark.parametrize("name,flags", CASES, ids=[f"{n}-{f}" for n, f in CASES])
def test_fused_step_matches_oracle(rt, name, flags):
    """Each configuration through the library's own choice of path, the
    long-context steps forced onto the single kernel (its long-run tile
    shape), the others forced onto the compile kernel followed by the K/V
    kernel."""
    w = workloads.get(name)
    b, exp = _prepare(rt, w)
    sentinel = 0x2C3D
    s, kv = _fused_step(rt, w, b, exp, sentinel, flags=flags)
    assert_step_equal(b.step_outputs(s), exp, name)
    _check_all(w, exp, kv, sentinel, name)
    del kv
    torch.cuda.empty_cache()
    b.close()


NARROW = [("long_context", 1), ("churn", 2), ("decode_heavy", 1), ("mixed", 2)]


@pytest.mark.parametrize("name,heads", NARROW, ids=[f"{n}-{h * 256}B" for n, h in NARROW])
def test_fused_full_size_narrow_rows(rt, name, heads):
    """The configurations at full size with a tensor-parallel rank's rows
    (one or two heads of 128: 256 B or 512 B) through the library's own
    choice, which is the single kernel for these rows, long runs included:
    every compile output, and every row of every K/V cache against the
    oracle (real rows against their sources, all others still the
    sentinel)."""
    import dataclasses
    w = dataclasses.replace(workloads.get(name), kv_heads=heads)
    b, exp = _prepare(rt, w)
    sentinel = 0x4B4B
    s, kv = _fused_step(rt, w, b, exp, sentinel, flags=0)
    assert_step_equal(b.step_outputs(s), exp, f"{name} {w.row_bytes} B")
    _check_all(w, exp, kv, sentinel, f"{name} {w.row_bytes} B")
    del kv
    torch.cuda.empty_cache()
    b.close()


VARIANTS = [(n, v) for n in ("churn", "mixed", "decode_heavy", "long_context") for v in (1, 2)]


@pytest.mark.parametrize("name,variant", VARIANTS, ids=[f"{n}-{v}" for n, v in VARIANTS])
def test_fused_other_seeded_instances(rt, name, variant):
    """Independently seeded instances of the full-size configurations (the
    ones the benchmark rotates over) through the library's own choice of
    path: every compile output and every row of every K/V cache against the
    oracle."""
    w = workloads.get(name, variant=variant)
    b, exp = _prepare(rt, w)
    sentinel = 0x3A3A
    s, kv = _fused_step(rt, w, b, exp, sentinel, flags=0)
    assert_step_equal(b.step_outputs(s), exp, f"{name} instance {variant}")
    _check_all(w, exp, kv, sentinel, f"{name} instance {variant}")
    del kv
    torch.cuda.empty_cache()
    b.close()


def _random_workload(rng, trial, head_choices):
    B = int(rng.choice([1, 2, 3, 4, 8, 16, 32, 64]))
    R = int(rng.integers(1, 300))
    max_q = int(rng.choice([1, 5, 40, 300]))
    M = 2048
    pool = R * -(-(1200 + max_q) // B) + 10
    reqs = workloads.random_batch(rng, num_reqs=R, block_size=B, max_model_len=M, num_kv_blocks=pool,
                                  max_q=max_q, max_c=1200)
    N = sum(r.num_scheduled for r in reqs)
    n_pad = N + int(rng.integers(0, 70))
    heads, dim = head_choices[trial % len(head_choices)]
    return workloads.Workload("fused_random", block_size=B, max_num_reqs=R + int(rng.integers(0, 20)),
                              max_model_len=M, max_blocks_per_req=-(-M // B), max_num_batched_tokens=n_pad,
                              num_kv_blocks=pool, kv_heads=heads, head_dim=dim, kv_dtype="bf16",
                              num_layers=int(rng.integers(1, 4)), hidden_size=64, gather="all", initial=reqs,
                              capture_sizes=[n_pad], seed=int(rng.integers(1 << 30)))


def test_fused_random_batches(rt):
    """Eighty seeded batches: block sizes 1 to 64 (shift and division
    paths), decode-only to 300-token chunks, up to 300 requests, padded tails
    of up to 69 tokens, 1-3 layers, rows of 128 B, 256 B, 512 B, 1, 2, 3, 4
    and 8 KiB (fused) and 64 B and 1.5 KiB (compile, then the separate K/V
    kernel)."""
    rng = np.random.default_rng(4321)
    heads = [(4, 128), (8, 128), (16, 128), (1, 128), (12, 128), (2, 128), (1, 64), (1, 32), (32, 128), (6, 128)]
    for trial in range(80):
        w = _random_workload(rng, trial, heads)
        label = f"trial {trial}: B={w.block_size} R={len(w.initial)} row={w.row_bytes} L={w.num_layers}"
        b, exp = _prepare(rt, w)
        sentinel = 0x1357
        s, kv = _fused_step(rt, w, b, exp, sentinel, flags=(0, ALWAYS, NEVER)[trial % 3])
        assert_step_equal(b.step_outputs(s), exp, label)
        _check_all(w, exp, kv, sentinel, label)
        b.close()


def test_fused_past_one_launch_of_layers(rt):
    """40 layers of 2 KiB rows: the fused launch writes the first 32, the K/V
    kernel the rest; every cache byte is checked."""
    rng = np.random.default_rng(99)
    reqs = workloads.random_batch(rng, num_reqs=7, block_size=16, max_model_len=512, num_kv_blocks=300,
                                  max_q=80, max_c=300)
    N = sum(r.num_scheduled for r in reqs)
    w = workloads.Workload("fused_layers", block_size=16, max_num_reqs=8, max_model_len=512,
                           max_blocks_per_req=32, max_num_batched_tokens=N + 5, num_kv_blocks=300, kv_heads=8,
                           head_dim=128, kv_dtype="bf16", num_layers=40, hidden_size=64, gather="all",
                           initial=reqs, capture_sizes=[N + 5], seed=7)
    b, exp = _prepare(rt, w)
    s, kv = _fused_step(rt, w, b, exp, 0x0F0F, flags=ALWAYS)
    assert_step_equal(b.step_outputs(s), exp, "40 layers")
    _check_all(w, exp, kv, 0x0F0F, "40 layers")
    b.close()


def test_fused_equals_separate_calls(rt):
    """The single kernel and ric_compile + ric_reshape_and_cache leave
    identical caches (mixed has no padded tokens, so the whole cache is
    deterministic)."""
    ric, runner = rt
    w = workloads.get("mixed")
    caches = []
    for fused in (True, False):
        b, exp = _prepare(rt, w)
        n_pad = exp["n_pad"]
        kc, vc = runner.alloc_caches(w, fill=0x4444)
        k, v = runner.alloc_sources(w, n_pad, seed=w.seed + 3)
        kv = runner.KVSet(k, v, kc, vc, w.row_bytes, w.num_kv_blocks * w.block_size)
        if fused:
            runner.compile_and_cache(b, n_pad, kv, flags=ALWAYS)
        else:
            s = b.compile(n_pad)
            runner.reshape_and_cache(kv, s.slot_mapping, n_pad)
        torch.cuda.synchronize()
        caches.append((kc[0], vc[0]))
        b.close()
    assert torch.equal(caches[0][0], caches[1][0]) and torch.equal(caches[0][1], caches[1][1])


def test_fused_argument_errors_enqueue_nothing(rt):
    ric, runner = rt
    w = workloads.get("worked_example")
    b, exp = _prepare(rt, w)
    kc, vc = runner.alloc_caches(w, fill=0)
    k, v = runner.alloc_sources(w, exp["n_pad"], seed=1)
    ptrs = [[t.data_ptr() for t in lst] for lst in (k, v, kc, vc)]
    nslots = w.num_kv_blocks * w.block_size
    for kw, code in ((dict(row_bytes=24, num_slots=nslots), ric.RIC_EINVAL),
                     (dict(row_bytes=w.row_bytes, num_slots=0), ric.RIC_EINVAL),
                     (dict(row_bytes=w.row_bytes, num_slots=nslots, flags=4), ric.RIC_EINVAL),
                     (dict(row_bytes=w.row_bytes, num_slots=nslots, flags=3), ric.RIC_EINVAL),
                     (dict(row_bytes=w.row_bytes, num_slots=nslots, src_row_stride=8), ric.RIC_EINVAL)):
        with pytest.raises(ric.RicError) as e:
            ric.ric_compile_and_cache(b.h, exp["n_pad"], *ptrs, **kw)
        assert e.value.code == code
    with pytest.raises(ric.RicError) as e:
        ric.ric_compile_and_cache(b.h, exp["n_pad"] + 1000, *ptrs, row_bytes=w.row_bytes, num_slots=nslots)
    assert e.value.code == ric.RIC_EINVAL
    s = ric.ric_compile_and_cache(b.h, exp["n_pad"], *ptrs, row_bytes=w.row_bytes, num_slots=nslots)
    torch.cuda.synchronize()
    assert_step_equal(b.step_outputs(s), exp, "after rejected calls")
    b.close()


def test_fused_empty_batch_is_all_padding(rt):
    """No live request: the single kernel writes every padded row to the null
    block and nothing else; the compile outputs are the padding reading."""
    ric, runner = rt
    cfg = ric.make_config(max_num_reqs=4, max_model_len=16, block_size=4, max_blocks_per_req=4,
                          max_num_batched_tokens=8, num_kv_blocks=10, null_block=3, staging_bytes=0)
    b = runner.Batch(cfg)
    ric.ric_schedule(b.h, [], [])
    row = 1024
    nslots = 40
    k = torch.randn((8, row // 2), device="cuda").to(torch.float16)
    v = torch.randn((8, row // 2), device="cuda").to(torch.float16)
    kc = torch.full((nslots, row // 2), 77, dtype=torch.int16, device="cuda")
    vc = torch.full((nslots, row // 2), 77, dtype=torch.int16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = ric.ric_compile_and_cache(b.h, 8, [k.data_ptr()], [v.data_ptr()], [kc.data_ptr()], [vc.data_ptr()], row,
                                  nslots, dev_status=status.data_ptr(), flags=ric.RIC_FUSE_ALWAYS)
    torch.cuda.synchronize()
    got = b.step_outputs(s)
    assert list(got["slot_mapping"]) == [12] * 8 and list(got["req_indices"]) == [-1] * 8
    assert list(got["query_start_loc"]) == [0] * 5 and list(got["sample_indices"]) == [-1] * 4
    assert int(status.item()) == 0
    others = [i for i in range(nslots) if i != 12]
    assert bool((kc[others] == 77).all()) and bool((vc[others] == 77).all())
    # the null slot holds one of the padded rows (which one is not defined)
    assert any(torch.equal(kc[12], k[t].view(torch.int16)) for t in range(8))
    b.close()


@pytest.mark.parametrize("R,heads", [(255, 8), (256, 8), (257, 8), (512, 8), (256, 1), (257, 1), (512, 2),
                                     (300, 0)])
def test_fused_around_the_counters_first_limit(rt, R, heads):
    """With at most 256 requests each thread of a token workgroup loads its
    own request's counters before the K/V rows; above that the counters are
    loaded in a loop after them (and rows narrower than 1 KiB take four rows
    per wave instead of two).  Batches of 255-512 requests (decodes and short
    prefills, spare rows past R) through the single kernel, rows of 2 KiB,
    128 B (heads 0: one head of 64), 256 B and 512 B: every output and cache
    byte against the oracle."""
    rng = np.random.default_rng(7000 + R)
    B, M = 16, 256
    pool = R * -(-M // B) + 1
    reqs = workloads.random_batch(rng, num_reqs=R, block_size=B, max_model_len=M, num_kv_blocks=pool,
                                  max_q=6, max_c=200)
    N = sum(r.num_scheduled for r in reqs)
    w = workloads.Workload("fused_counters", block_size=B, max_num_reqs=R + 7, max_model_len=M,
                           max_blocks_per_req=-(-M // B), max_num_batched_tokens=N + 5, num_kv_blocks=pool,
                           kv_heads=max(heads, 1), head_dim=128 if heads else 64, kv_dtype="bf16", num_layers=2,
                           hidden_size=64,
                           gather="all", initial=reqs, capture_sizes=[N + 5], seed=R)
    b, exp = _prepare(rt, w)
    s, kv = _fused_step(rt, w, b, exp, 0x5A5A, flags=ALWAYS)
    assert_step_equal(b.step_outputs(s), exp, f"{R} requests, {w.row_bytes} B rows")
    _check_all(w, exp, kv, 0x5A5A, f"{R} requests, {w.row_bytes} B rows")
    b.close()


@pytest.mark.parametrize("heads", [1, 4, 8])
def test_fused_strided_sources(rt, heads):
    """K and V as views into one fused [N_pad, 3, H, D] projection output (row
    stride three rows), rows of 256 B, 1 KiB and 2 KiB, through the single
    kernel: every output and cache byte against the oracle."""
    ric, runner = rt
    rng = np.random.default_rng(3 + heads)
    reqs = workloads.random_batch(rng, num_reqs=40, block_size=16, max_model_len=512, num_kv_blocks=40 * 33 + 1,
                                  max_q=40, max_c=400)
    N = sum(r.num_scheduled for r in reqs)
    w = workloads.Workload("fused_strided", block_size=16, max_num_reqs=48, max_model_len=512,
                           max_blocks_per_req=32, max_num_batched_tokens=N + 9, num_kv_blocks=40 * 33 + 1,
                           kv_heads=heads, head_dim=128, kv_dtype="bf16", num_layers=2, hidden_size=64, gather="all",
                           initial=reqs, capture_sizes=[N + 9], seed=heads)
    b, exp = _prepare(rt, w)
    n_pad = exp["n_pad"]
    sentinel = 0x6E6E
    kc, vc = runner.alloc_caches(w, fill=sentinel)
    qkv = [torch.randn((n_pad, 3, heads, 128), device="cuda").to(torch.bfloat16) for _ in range(2)]
    k = [t[:, 1] for t in qkv]
    v = [t[:, 2] for t in qkv]
    assert k[0].stride(0) == 3 * heads * 128
    kv = runner.KVSet(k, v, kc, vc, w.row_bytes, w.num_kv_blocks * w.block_size)
    s = runner.compile_and_cache(b, n_pad, kv, flags=ALWAYS)
    torch.cuda.synchronize()
    assert_step_equal(b.step_outputs(s), exp, f"strided {w.row_bytes} B")
    _check_all(w, exp, runner.KVSet([t.contiguous() for t in k], [t.contiguous() for t in v], kc, vc, w.row_bytes,
                                    kv.num_slots), sentinel, f"strided {w.row_bytes} B")
    b.close()


def test_fused_at_the_row_limit(rt):
    """8000 requests (the row limit: the largest prefix sum a workgroup keeps
    in LDS) through the single kernel, decodes and short prefills mixed."""
    rng = np.random.default_rng(8000)
    reqs = workloads.random_batch(rng, num_reqs=8000, block_size=16, max_model_len=64,
                                  num_kv_blocks=8000 * 4 + 1, max_q=3, max_c=40)
    N = sum(r.num_scheduled for r in reqs)
    w = workloads.Workload("fused_rows", block_size=16, max_num_reqs=8000, max_model_len=64, max_blocks_per_req=4,
                           max_num_batched_tokens=N + 3, num_kv_blocks=8000 * 4 + 1, kv_heads=4, head_dim=128,
                           kv_dtype="bf16", num_layers=1, hidden_size=64, gather="all", initial=reqs,
                           capture_sizes=[N + 3], seed=11)
    b, exp = _prepare(rt, w)
    s, kv = _fused_step(rt, w, b, exp, 0x7171, flags=ALWAYS)
    assert_step_equal(b.step_outputs(s), exp, "8000 rows")
    _check_all(w, exp, kv, 0x7171, "8000 rows")
    b.close()


def test_fused_long_runs(rt):
    """Steps of long per-request runs (1024 or more scheduled tokens per
    request on average), alternately forced onto the single kernel and
    through the library's own choice (two kernels for rows of 1 KiB or more),
    24 seeded
    batches: 1-8 requests, chunks of 1024-4096 tokens on cached prefixes up to
    4000, block sizes 1, 16, 64 and 100, rows of 256 B, 512 B, 1, 2 and 4
    KiB (the narrow ones take the single kernel by the library's own choice
    too), 1-3 layers, padded tails; every output and cache byte against the
    oracle."""
    rng = np.random.default_rng(1024)
    for trial in range(24):
        B = int(rng.choice([1, 16, 64, 100]))
        R = int(rng.integers(1, 9))
        M = 8192
        pool = R * -(-M // B) + 10
        reqs = workloads.random_batch(rng, num_reqs=R, block_size=B, max_model_len=M, num_kv_blocks=pool,
                                      max_q=4096, max_c=4000)
        N = sum(r.num_scheduled for r in reqs)
        if N < 1024 * R:                    # not a long-run step: drawn again in the next trial
            continue
        heads = (4, 8, 16, 1, 2)[trial % 5]
        n_pad = N + int(rng.integers(0, 40))
        w = workloads.Workload("long_runs", block_size=B, max_num_reqs=R + 2, max_model_len=M,
                               max_blocks_per_req=-(-M // B), max_num_batched_tokens=n_pad, num_kv_blocks=pool,
                               kv_heads=heads, head_dim=128, kv_dtype="bf16", num_layers=1 + trial % 3,
                               hidden_size=64, gather="all", initial=reqs, capture_sizes=[n_pad],
                               seed=int(rng.integers(1 << 30)))
        label = f"trial {trial}: B={B} R={R} N={N} row={w.row_bytes} L={w.num_layers}"
        b, exp = _prepare(rt, w)
        s, kv = _fused_step(rt, w, b, exp, 0x5A5A, flags=(ALWAYS, 0)[trial % 2])
        assert_step_equal(b.step_outputs(s), exp, label)
        _check_all(w, exp, kv, 0x5A5A, label)
        b.close()


def test_two_handles_on_two_streams(rt):
    """Two handles, each on its own stream, their calls interleaved with no
    synchronisation between them (mixed through the single kernel, the
    worked example through the single kernel with 256 B rows, then each
    scheduled and compiled again): per-handle state is separate, so both
    steps equal the oracle's."""
    ric, runner = rt
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    made = []
    for name, st in (("mixed", s1), ("worked_example", s2)):
        w = workloads.get(name)
        with torch.cuda.stream(st):
            b = runner.Batch(runner.config_of(w), stream=runner.current_stream())
            for r in w.initial:
                b.add(r)
            for rid in w.finished:
                ric.ric_remove_request(b.h, rid)
            if w.finished:
                ric.ric_condense(b.h)
            for r in w.refill:
                b.add(r)
        ref, order = replay_history(w)
        exp = expected_step(w, ref, use_python=(name == "worked_example"))
        kc, vc = runner.alloc_caches(w, fill=0x1111)
        k, v = runner.alloc_sources(w, exp["n_pad"], seed=w.seed + 77)
        made.append((name, w, st, b, order, exp, runner.KVSet(k, v, kc, vc, w.row_bytes,
                                                               w.num_kv_blocks * w.block_size)))
    torch.cuda.synchronize()
    for rep in range(3):
        steps = []
        for name, w, st, b, order, exp, kv in made:     # enqueue both, then wait once
            with torch.cuda.stream(st):
                b.schedule_from(w, order)
                steps.append(runner.compile_and_cache(b, exp["n_pad"], kv))
        torch.cuda.synchronize()
        for (name, w, st, b, order, exp, kv), s in zip(made, steps):
            assert s.kv_path == 1, (name, s.kv_path)
            assert_step_equal(b.step_outputs(s), exp, f"{name} round {rep}")
            _check_all(w, exp, kv, 0x1111, f"{name} round {rep}")
    for m in made:
        m[3].close()
