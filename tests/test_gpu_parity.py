"""GPU parity: libric on an MI355X against the CPU oracle, element by element.

Compile outputs and the column store must be bit-exact; K/V cache rows and
gathered hidden rows byte-exact.  Every K/V check covers the whole cache:
small cases on the host against the oracle's assignment, the full-size
configurations on the device (every real row against its source at the
oracle's slot, every other row outside the null block against the sentinel)."""
import numpy as np
import pytest
import torch

import workloads
from oracle import batch as ref_batch, cbind, step as ref_step, vectorised
from tests.gpu_helpers import assert_step_equal, check_cache_exact, expected_step, read_rows_i32, replay_history
from workloads import payload_numpy
from tests.oracle_helpers import golden

pytestmark = pytest.mark.gpu

CONFIGS = ["worked_example", "decode_heavy", "mixed", "churn", "long_context", "long_context_forced"]


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_input_compilation_amd import _ric, runner
    return _ric, runner


def _compile(rt, w):
    ric, runner = rt
    b = runner.Batch(runner.config_of(w))
    moved = b.load_history(w)
    ref, order = replay_history(w)
    assert b.row_order() == order, "row order differs from the reference batch"
    b.schedule_from(w, order)
    exp = expected_step(w, ref, use_python=(w.name == "worked_example"))
    n_pad = ric.ric_padded_size(w.capture_sizes, exp["num_actual_tokens"])
    assert n_pad == exp["n_pad"]
    s = b.compile(n_pad)
    assert (s.num_reqs, s.num_actual_tokens, s.num_tokens_padded, s.max_query_len, s.max_seq_len,
            s.num_sampled, s.kv_path) == (exp["num_reqs"], exp["num_actual_tokens"], n_pad, exp["max_query_len"],
                                          exp["max_seq_len"], exp["num_sampled"], 0)
    return b, s, ref, order, exp, moved


@pytest.mark.parametrize("name", CONFIGS)
def test_compile_matches_oracle(rt, name):
    w = workloads.get(name)
    b, s, ref, order, exp, moved = _compile(rt, w)
    got = b.step_outputs(s)
    torch.cuda.synchronize()
    assert_step_equal(got, exp, name)
    b.close()


def test_worked_example_printed_values(rt):
    """The configuration built from the third page's example gives its printed
    query_start_loc, seq_lens and logits indices on the GPU."""
    w = workloads.get("worked_example")
    b, s, *_ = _compile(rt, w)
    got = b.step_outputs(s)
    assert list(got["query_start_loc"][:4]) == [0, 7, 8, 20]
    assert list(got["seq_lens"][:3]) == [7, 6, 22]
    assert list(got["logits_indices"][:3]) == [6, 7, 19]
    assert list(got["positions"][:20]) == list(range(7)) + [5] + list(range(10, 22))
    assert s.num_tokens_padded == 32
    b.close()


@pytest.mark.parametrize("name", ["churn", "mixed", "worked_example"])
def test_column_store_matches_reference_batch(rt, name):
    """After the history (adds, removals, condense, refills) every live row's
    columns equal the reference batch's: token history, block row, counters
    and sampling values moved together."""
    ric, runner = rt
    w = workloads.get(name)
    b, s, ref, order, exp, moved = _compile(rt, w)
    if name == "churn":
        assert moved > 0
    cols = ric.ric_get_columns(b.h)
    R = len(order)
    T = b.device_i32(cols.num_tokens, R)
    P = b.device_i32(cols.num_prompt, R)
    C = b.device_i32(cols.num_computed, R)
    Q = b.device_i32(cols.num_scheduled, R)
    NB = b.device_i32(cols.num_blocks, R)
    K = b.device_i32(cols.top_k, R)
    temp = b.device_u8(cols.temperature, 4 * R).view(np.float32)
    top_p = b.device_u8(cols.top_p, 4 * R).view(np.float32)
    rep = b.device_u8(cols.repetition_penalty, 4 * R).view(np.float32)
    for i in range(R):
        r = ref.rows[i]
        assert (T[i], P[i], C[i], Q[i], NB[i]) == (len(r.tokens), r.num_prompt, r.num_computed,
                                                   r.num_scheduled, len(r.blocks)), f"row {i}"
        t_, p_, rp_, k_ = r.sampling
        assert (temp[i], top_p[i], rep[i], K[i]) == (np.float32(t_), np.float32(p_), np.float32(rp_), k_)
    for i in range(R):
        r = ref.rows[i]
        toks = read_rows_i32(b.workspace, cols.tokens, cols.token_stride, [i], len(r.tokens))[0]
        assert np.array_equal(toks, np.asarray(r.tokens, np.int32)), f"token row {i}"
        blks = read_rows_i32(b.workspace, cols.blocks, cols.block_stride, [i], len(r.blocks))[0]
        assert np.array_equal(blks, np.asarray(r.blocks, np.int32)), f"block row {i}"
    b.close()


def _full_kv_check(rt, w, b, s, exp, layers=None):
    """Every cache byte: real slots equal their source rows, everything outside
    the real slots and the null block keeps its sentinel."""
    ric, runner = rt
    L = w.num_layers if layers is None else layers
    n_pad = exp["n_pad"]
    kc, vc = runner.alloc_caches(w, L, fill=0x3A5C)
    k, v = runner.alloc_sources(w, n_pad, seed=w.seed + 11, num_layers=L, host=True)
    kv = runner.KVSet(k, v, kc, vc, w.row_bytes, w.num_kv_blocks * w.block_size)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    runner.reshape_and_cache(kv, s.slot_mapping, n_pad, dev_status=status.data_ptr())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    rows = w.num_kv_blocks * w.block_size
    B = w.block_size
    slots = exp["slot_mapping"]
    for l in range(L):
        for src, cache in ((k[l], kc[l]), (v[l], vc[l])):
            want = np.full((rows, w.row_bytes // 2), 0x3A5C, np.int16)
            vectorised.reshape_and_cache(src.view(torch.int16).reshape(n_pad, -1).cpu().numpy(),
                                         src.view(torch.int16).reshape(n_pad, -1).cpu().numpy(),
                                         want, want.copy(), slots)
            got = cache.view(torch.int16).reshape(rows, -1).cpu().numpy()
            assert np.array_equal(got[B:], want[B:]), f"layer {l}: cache differs outside the null block"


def test_kv_write_worked_example_full(rt):
    w = workloads.get("worked_example")
    b, s, ref, order, exp, _ = _compile(rt, w)
    _full_kv_check(rt, w, b, s, exp)
    b.close()


@pytest.mark.parametrize("name", ["decode_heavy", "mixed", "churn", "long_context", "long_context_forced"])
def test_kv_write_full_size(rt, name):
    """Full-size caches, every layer of the configuration, one launch, every
    byte: each real token's K and V rows equal their source rows at the
    oracle's slot, and every cache row outside the step's real slots and the
    null block still holds the sentinel (the rows holding anything else are
    exactly the oracle's slot set), checked on the device.  Decode-heavy and
    mixed take the wave-per-row shape, churn and long-context chunk tiles."""
    ric, runner = rt
    w = workloads.get(name)
    b, s, ref, order, exp, _ = _compile(rt, w)
    n_pad, N = exp["n_pad"], exp["num_actual_tokens"]
    sentinel = 0x1F2E
    kc, vc = runner.alloc_caches(w, fill=sentinel)
    k, v = runner.alloc_sources(w, n_pad, seed=w.seed + 17)
    kv = runner.KVSet(k, v, kc, vc, w.row_bytes, w.num_kv_blocks * w.block_size)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    runner.reshape_and_cache(kv, s.slot_mapping, n_pad, dev_status=status.data_ptr())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    B = w.block_size
    nslots = w.num_kv_blocks * B
    null = (w.null_block * B, w.null_block * B + B)
    for l in range(w.num_layers):
        for nm, src, cache in (("K", k[l], kc[l]), ("V", v[l], vc[l])):
            check_cache_exact(cache, src, exp["slot_mapping"], N, sentinel, nslots, null, f"{name} layer {l} {nm}")
    del kc, vc, k, v, kv
    torch.cuda.empty_cache()
    b.close()


# Row sizes and token counts that select each K/V launch shape: wave rows for
# 1, 2 and 4 KiB rows up to 8192 tokens; chunk tiles otherwise (several rows
# per workgroup below 4 KiB, one row per workgroup above, in one or several
# passes; a chunk count per row that is not a power of two takes a division).
KV_SHAPES = [
    ("wave 1 KiB", 1024, 3000, 0),
    ("wave 2 KiB", 2048, 777, 0),
    ("wave 4 KiB", 4096, 5000, 0),
    ("wave 4 KiB strided source", 4096, 1500, 4096 + 256),
    ("wave 1 KiB at the token limit", 1024, 8192, 0),
    ("chunk 1 KiB above the wave limit", 1024, 8193, 0),
    ("chunk 4 KiB above the wave limit", 4096, 9000, 0),
    ("chunk 8 KiB, two passes per row", 8192, 1200, 0),
    ("chunk 12 KiB, three passes per row", 12288, 300, 0),
    ("chunk 3 KiB, 192 chunks per row", 3072, 2000, 0),
    ("chunk 48 B, division per chunk", 48, 4000, 64),
    ("chunk 16 B", 16, 2500, 0),
    ("chunk 256 B", 256, 3333, 0),
]


@pytest.mark.parametrize("label,row_bytes,n_tok,stride", KV_SHAPES, ids=[x[0] for x in KV_SHAPES])
def test_kv_write_every_launch_shape(rt, label, row_bytes, n_tok, stride):
    """Each K/V launch shape the library can pick, two layers in one launch,
    distinct random slots in a cache of about twice the step: the whole cache
    (every byte of every row) equals the oracle's fancy-index assignment into
    a sentinel-filled copy."""
    ric, runner = rt
    rng = np.random.default_rng(row_bytes * 7919 + n_tok)
    L = 2
    num_slots = 2 * n_tok + 37
    elems = row_bytes // 2
    stride = stride or row_bytes
    slots = rng.permutation(num_slots)[:n_tok].astype(np.int32)
    sentinel = 0x6A6B
    ks, vs, kcs, vcs, srcs = [], [], [], [], []
    for l in range(L):
        pair = []
        for j in range(2):
            base = payload_numpy(np.random.default_rng(1000 * l + j + row_bytes), (n_tok, stride // 2), "bf16")
            pair.append(base)
            t = torch.from_numpy(base.view(np.int16)).cuda()
            (ks if j == 0 else vs).append(t)
        srcs.append(pair)
        for lst in (kcs, vcs):
            lst.append(torch.full((num_slots, elems), sentinel, dtype=torch.int16, device="cuda"))
    slot_t = torch.from_numpy(slots).cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ric.ric_reshape_and_cache([t.data_ptr() for t in ks], [t.data_ptr() for t in vs],
                              [t.data_ptr() for t in kcs], [t.data_ptr() for t in vcs],
                              slot_t.data_ptr(), n_tok, row_bytes, num_slots, src_row_stride=stride,
                              dev_status=status.data_ptr(), stream=runner.current_stream())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    for l in range(L):
        k_np = srcs[l][0].view(np.int16)[:, :elems]
        v_np = srcs[l][1].view(np.int16)[:, :elems]
        want_k = np.full((num_slots, elems), sentinel, np.int16)
        want_v = want_k.copy()
        vectorised.reshape_and_cache(k_np, v_np, want_k, want_v, slots)
        assert np.array_equal(kcs[l].cpu().numpy(), want_k), f"{label}: layer {l} K cache differs"
        assert np.array_equal(vcs[l].cpu().numpy(), want_v), f"{label}: layer {l} V cache differs"


@pytest.mark.parametrize("name", CONFIGS)
def test_gather_matches_oracle(rt, name):
    """Hidden rows gathered at logits_indices (one per request) and at the
    compacted sample_indices with the device count."""
    ric, runner = rt
    w = workloads.get(name)
    b, s, ref, order, exp, _ = _compile(rt, w)
    n_pad, R, MR = exp["n_pad"], exp["num_reqs"], w.max_num_reqs
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 23)
    hidden = torch.randn((n_pad, w.hidden_size), generator=g, device="cuda").to(torch.bfloat16)
    out = torch.full((MR, w.hidden_size), 7.0, dtype=torch.bfloat16, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    runner.gather(hidden, s.logits_indices, 0, R, out, dev_status=status.data_ptr())
    out2 = torch.full((MR, w.hidden_size), 7.0, dtype=torch.bfloat16, device="cuda")
    runner.gather(hidden, s.sample_indices, s.dev_scalars + 20, MR, out2, dev_status=status.data_ptr())
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    li = torch.from_numpy(exp["logits_indices"][:R]).cuda()
    assert torch.equal(out[:R].view(torch.int16), hidden[li].view(torch.int16))
    assert bool((out[R:] == 7.0).all())
    ns = exp["num_sampled"]
    si = torch.from_numpy(exp["sample_indices"][:ns]).cuda()
    assert torch.equal(out2[:ns].view(torch.int16), hidden[si].view(torch.int16))
    assert bool((out2[ns:] == 7.0).all())
    b.close()


def _tiny_workload(rng, B, R, max_q=6, max_c=20, extra_pad=3):
    reqs = workloads.random_batch(rng, num_reqs=R, block_size=B, max_model_len=64, num_kv_blocks=200,
                                  max_q=max_q, max_c=max_c)
    N = sum(r.num_scheduled for r in reqs)
    w = workloads.Workload("tiny", block_size=B, max_num_reqs=R + int(rng.integers(0, 3)), max_model_len=64,
                           max_blocks_per_req=64, max_num_batched_tokens=N + extra_pad, num_kv_blocks=200,
                           kv_heads=1, head_dim=8 * int(rng.integers(1, 5)), kv_dtype="f16", num_layers=2,
                           hidden_size=64, gather="all", initial=reqs,
                           capture_sizes=[N + int(rng.integers(0, extra_pad + 1))], seed=int(rng.integers(1 << 30)))
    return w


def test_bruteforce_tiny_batches(rt):
    """Many tiny random batches, block sizes 1, 2, 3, 4, 8 and 16, padded
    sizes above N: every compile output and every cache byte (outside the null
    block) equals the oracle."""
    ric, runner = rt
    rng = np.random.default_rng(77)
    for trial in range(120):
        B = int(rng.choice([1, 2, 3, 4, 8, 16]))
        R = int(rng.integers(1, 6))
        w = _tiny_workload(rng, B, R)
        b, s, ref, order, exp, _ = _compile(rt, w)
        assert_step_equal(b.step_outputs(s), exp, f"trial {trial}")
        if trial % 4 == 0:
            _full_kv_check(rt, w, b, s, exp)
        b.close()


def test_random_medium_batches(rt):
    """A hundred seeded batches between the tiny cases and the named workloads:
    up to 400 requests, decode-only to 600-token chunks, cached prefixes up to
    3000, block sizes from 1 to 128 (powers of two and not), padded sizes up to
    256 above N, and table payloads that overflow the default staging log.
    Every compile output equals the C oracle's; every fifth batch also checks
    every cache byte outside the null block."""
    ric, runner = rt
    rng = np.random.default_rng(1234)
    for trial in range(100):
        B = int(rng.choice([1, 3, 5, 7, 16, 32, 64, 100, 128]))
        R = int(rng.integers(1, 401))
        max_q = int(rng.choice([1, 8, 64, 600]))
        M = 4096
        pool = R * -(-(3000 + max_q) // B) + 10
        reqs = workloads.random_batch(rng, num_reqs=R, block_size=B, max_model_len=M, num_kv_blocks=pool,
                                      max_q=max_q, max_c=3000)
        N = sum(r.num_scheduled for r in reqs)
        n_pad = N + int(rng.integers(0, 257))
        w = workloads.Workload("medium", block_size=B, max_num_reqs=R + int(rng.integers(0, 50)), max_model_len=M,
                               max_blocks_per_req=-(-M // B), max_num_batched_tokens=n_pad, num_kv_blocks=pool,
                               kv_heads=1, head_dim=8, kv_dtype="f16", num_layers=1, hidden_size=64, gather="all",
                               initial=reqs, capture_sizes=[n_pad], seed=int(rng.integers(1 << 30)))
        label = f"trial {trial}: B={B} R={R} max_q={max_q} N={N} n_pad={n_pad}"
        b, s, ref, order, exp, _ = _compile(rt, w)
        assert_step_equal(b.step_outputs(s), exp, label)
        if trial % 5 == 0:
            _full_kv_check(rt, w, b, s, exp)
        b.close()


def test_empty_batch_is_all_padding(rt):
    ric, runner = rt
    cfg = ric.make_config(max_num_reqs=4, max_model_len=16, block_size=4, max_blocks_per_req=4,
                          max_num_batched_tokens=8, num_kv_blocks=10, null_block=3, staging_bytes=0)
    b = runner.Batch(cfg)
    ric.ric_schedule(b.h, [], [])
    s = b.compile(8)
    got = b.step_outputs(s)
    assert list(got["slot_mapping"]) == [12] * 8 and list(got["req_indices"]) == [-1] * 8
    assert list(got["query_start_loc"]) == [0] * 5 and list(got["seq_lens"]) == [0] * 4
    assert list(got["sample_indices"]) == [-1] * 4 and got["num_sampled"] == 0
    b.close()


def test_serving_loop_deltas(rt):
    """Several steps of a simulated serving loop on one handle: requests
    arrive, decode (one appended token per step, a new block when the last one
    fills), get preempted and resume with replaced blocks, finish, get aborted
    and resubmitted under the same id; the batch is condensed.  Every step's
    compile equals the oracle's compile of the reference batch."""
    ric, runner = rt
    rng = np.random.default_rng(99)
    B, MR, M = 4, 12, 96
    cfg = ric.make_config(max_num_reqs=MR, max_model_len=M, block_size=B, max_blocks_per_req=M // B,
                          max_num_batched_tokens=128, num_kv_blocks=4096, null_block=0, staging_bytes=0)
    b = runner.Batch(cfg)
    ref = ref_batch.RefBatch(MR, M, M // B, 4096)
    free_blocks = list(rng.permutation(np.arange(1, 4096)))
    state = {}   # req_id -> dict(T, c)
    next_id = 0

    def new_blocks(n):
        return [int(free_blocks.pop()) for _ in range(n)]

    for step_no in range(40):
        # finish / abort-resubmit / preempt some requests
        for rid in list(state):
            x = rng.random()
            if x < 0.12:
                ric.ric_remove_request(b.h, rid); ref.remove_request(rid); del state[rid]
            elif x < 0.16:   # abort and resubmit under the same id: a new request
                ric.ric_remove_request(b.h, rid); ref.remove_request(rid)
                T = int(rng.integers(1, 30))
                toks = rng.integers(0, 1000, T)
                blks = new_blocks(-(-T // B))
                ric.ric_add_request(b.h, rid, toks, T, 0, blks); ref.add_request(rid, toks, T, 0, blks)
                state[rid] = dict(T=T, c=0)
            elif x < 0.20 and state[rid]["c"] > 0:   # preempted and resumed: blocks replaced
                st = state[rid]
                blks = new_blocks(min(-(-st["T"] // B) + 1, M // B))
                ric.ric_replace_blocks(b.h, rid, blks); ref.replace_blocks(rid, blks)
        # arrivals
        while len(state) < MR and rng.random() < 0.6:
            T = int(rng.integers(1, 40))
            toks = rng.integers(0, 1000, T)
            c0 = int(rng.integers(0, T))     # prefix-cache hit
            blks = new_blocks(-(-T // B))
            ric.ric_add_request(b.h, next_id, toks, T, c0, blks); ref.add_request(next_id, toks, T, c0, blks)
            state[next_id] = dict(T=T, c=c0)
            next_id += 1
        ric.ric_condense(b.h)
        ref.condense()
        order = [rid for rid in ref.req_ids_by_row() if rid is not None]
        assert b.row_order() == order
        if not order:
            continue
        cs, qs = [], []
        for rid in order:
            st = state[rid]
            if st["c"] >= st["T"]:           # decode: one new token appended
                tok = [int(rng.integers(0, 1000))]
                ric.ric_append_tokens(b.h, rid, tok); ref.append_tokens(rid, tok)
                st["T"] += 1
                nb = len(ref.rows[ref.row_of[rid]].blocks)
                if nb * B < st["T"]:
                    blk = new_blocks(1)
                    ric.ric_append_blocks(b.h, rid, blk); ref.append_blocks(rid, blk)
            q = min(st["T"] - st["c"], int(rng.integers(1, 9)))
            cs.append(st["c"]); qs.append(q)
        ric.ric_schedule(b.h, cs, qs)
        ref.schedule(cs, qs)
        rows = ref.step_rows()
        N = sum(qs)
        n_pad = N + int(rng.integers(0, 4))
        want = ref_step.compile_step(rows, block_size=B, max_num_reqs=MR, max_model_len=M,
                                     max_num_batched_tokens=128, num_kv_blocks=4096, n_pad=n_pad)
        s = b.compile(n_pad)
        got = b.step_outputs(s)
        for k in ("input_ids", "positions", "req_indices", "slot_mapping", "query_start_loc", "seq_lens",
                  "logits_indices", "discard", "sample_indices"):
            assert np.array_equal(np.asarray(got[k], np.int64), np.asarray(want[k], np.int64)), \
                f"step {step_no} {k}"
        for rid, q in zip(order, qs):
            state[rid]["c"] += q
    b.close()


def test_error_paths_leave_state_unchanged(rt):
    ric, runner = rt
    cfg = ric.make_config(max_num_reqs=2, max_model_len=16, block_size=4, max_blocks_per_req=4,
                          max_num_batched_tokens=8, num_kv_blocks=10, null_block=0, staging_bytes=0)
    b = runner.Batch(cfg)
    h = b.h
    ric.ric_add_request(h, 1, [5, 6, 7], 3, 0, [2])

    def code(fn, *a):
        with pytest.raises(ric.RicError) as e:
            fn(*a)
        return e.value.code

    assert code(ric.ric_add_request, h, 1, [1], 1, 0, [3]) == ric.RIC_EEXIST
    assert code(ric.ric_add_request, h, 2, [1] * 17, 1, 0, [3]) == ric.RIC_ERANGE
    assert code(ric.ric_add_request, h, 2, [1], 1, 0, [0]) == ric.RIC_ERANGE       # null block
    assert code(ric.ric_add_request, h, 2, [1], 1, 0, [10]) == ric.RIC_ERANGE      # beyond the pool
    assert code(ric.ric_remove_request, h, 9) == ric.RIC_ENOENT
    assert code(ric.ric_append_tokens, h, 1, [0] * 14) == ric.RIC_EFULL
    assert code(ric.ric_append_blocks, h, 1, [1, 2, 3, 4]) == ric.RIC_EFULL
    assert code(ric.ric_schedule, h, [0], [0]) == ric.RIC_EINVAL                   # q = 0
    assert code(ric.ric_schedule, h, [1], [3]) == ric.RIC_EINVAL                   # past the history
    assert code(ric.ric_schedule, h, [0, 0], [1, 1]) == ric.RIC_EINVAL             # R != live
    assert code(ric.ric_compile, h, 8) == ric.RIC_ESTATE                           # not scheduled
    ric.ric_add_request(h, 2, [1, 2, 3, 4, 5], 5, 0, [3])
    assert code(ric.ric_add_request, h, 3, [1], 1, 0, [4]) == ric.RIC_EFULL       # no free row
    assert code(ric.ric_schedule, h, [0, 0], [3, 5]) == ric.RIC_EINVAL             # too few blocks
    ric.ric_remove_request(h, 1)
    assert code(ric.ric_schedule, h, [0], [1]) == ric.RIC_ESTATE                   # hole at row 0
    assert ric.ric_condense(h) == 1
    ric.ric_schedule(h, [0], [4])
    assert code(ric.ric_compile, h, 3) == ric.RIC_EINVAL                           # N_pad < N
    assert code(ric.ric_compile, h, 9) == ric.RIC_EINVAL                           # above the budget
    s = b.compile(4)
    got = b.step_outputs(s)
    assert list(got["input_ids"]) == [1, 2, 3, 4]
    assert list(got["slot_mapping"]) == [12, 13, 14, 15]
    assert ric.ric_num_reqs(h) == 1 and ric.ric_row_of(h, 2) == 0 and ric.ric_req_at(h, 1) is None
    b.close()


def test_out_of_range_indices_are_reported_not_written(rt):
    """The copy kernels' own bounds checks: a slot outside the cache or an
    index past the source rows is skipped (zero row for the gather) and counted
    in the status word; in-range rows are still written."""
    ric, runner = rt
    row_bytes = 64
    nslots = 32
    k = torch.arange(4 * 32, dtype=torch.int16, device="cuda").reshape(4, 32)
    v = k + 1000
    kc = torch.full((nslots, 32), -1, dtype=torch.int16, device="cuda")
    vc = torch.full((nslots, 32), -1, dtype=torch.int16, device="cuda")
    slot = torch.tensor([3, nslots, -5, 7], dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    ric.ric_reshape_and_cache([k.data_ptr()], [v.data_ptr()], [kc.data_ptr()], [vc.data_ptr()],
                              slot.data_ptr(), 4, row_bytes, nslots, dev_status=status.data_ptr(),
                              stream=runner.current_stream())
    torch.cuda.synchronize()
    assert int(status.item()) == 4        # two bad tokens, K and V rows each
    assert torch.equal(kc[3], k[0]) and torch.equal(vc[7], v[3])
    others = [i for i in range(nslots) if i not in (3, 7)]
    assert bool((kc[others] == -1).all()) and bool((vc[others] == -1).all())
    # the same on the few-token launch shape (1 KiB rows, wave-per-row kernel)
    k1 = torch.arange(4 * 512, dtype=torch.int16, device="cuda").reshape(4, 512)
    v1 = k1 + 7
    kc1 = torch.full((nslots, 512), -1, dtype=torch.int16, device="cuda")
    vc1 = torch.full((nslots, 512), -1, dtype=torch.int16, device="cuda")
    status.zero_()
    ric.ric_reshape_and_cache([k1.data_ptr()], [v1.data_ptr()], [kc1.data_ptr()], [vc1.data_ptr()],
                              slot.data_ptr(), 4, 1024, nslots, dev_status=status.data_ptr(),
                              stream=runner.current_stream())
    torch.cuda.synchronize()
    assert int(status.item()) == 4
    assert torch.equal(kc1[3], k1[0]) and torch.equal(vc1[7], v1[3])
    assert bool((kc1[others] == -1).all()) and bool((vc1[others] == -1).all())
    # the reserved flags must be 0: anything else is rejected before a launch
    with pytest.raises(ric.RicError) as e:
        ric.ric_reshape_and_cache([k.data_ptr()], [v.data_ptr()], [kc.data_ptr()], [vc.data_ptr()],
                                  slot.data_ptr(), 4, row_bytes, nslots, flags=2, stream=runner.current_stream())
    assert e.value.code == ric.RIC_EINVAL
    src = torch.arange(5 * 16, dtype=torch.int32, device="cuda").reshape(5, 16)
    idx = torch.tensor([4, 5, -1, 0], dtype=torch.int32, device="cuda")
    out = torch.full((4, 16), 9, dtype=torch.int32, device="cuda")
    status.zero_()
    ric.ric_gather_rows(src.data_ptr(), 64, 5, idx.data_ptr(), 0, 4, 64, out.data_ptr(), 64,
                        status.data_ptr(), runner.current_stream())
    torch.cuda.synchronize()
    assert int(status.item()) == 1
    assert torch.equal(out[0], src[4]) and torch.equal(out[3], src[0])
    assert bool((out[1] == 0).all()) and bool((out[2] == 0).all())


def _simple_rows_workload(reqs, B, max_num_reqs, max_model_len, num_kv_blocks, row_heads=8, head_dim=128,
                          layers=1, name="custom", staging=0):
    N = sum(r.num_scheduled for r in reqs)
    return workloads.Workload(name, block_size=B, max_num_reqs=max_num_reqs, max_model_len=max_model_len,
                              max_blocks_per_req=-(-max_model_len // B), max_num_batched_tokens=N,
                              num_kv_blocks=num_kv_blocks, kv_heads=row_heads, head_dim=head_dim,
                              kv_dtype="bf16", num_layers=layers, hidden_size=256, gather="all",
                              initial=reqs, capture_sizes=[N], seed=4242)


def test_library_allocated_workspace_and_stream_switch(rt):
    """ric_create without a caller workspace (the library allocates), then a
    switch to another stream; the compile still equals the oracle."""
    ric, runner = rt
    w = workloads.get("mixed")
    ref, order = replay_history(w)
    exp = expected_step(w, ref)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        h = ric.ric_create(runner.config_of(w), runner.current_stream())
        for r in w.initial:
            ric.ric_add_request(h, r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks)
        other = torch.cuda.Stream()
        ric.ric_set_stream(h, int(other.cuda_stream))
        by_id = w.by_id()
        ric.ric_schedule(h, [by_id[i].num_computed for i in order], [by_id[i].num_scheduled for i in order])
        s = ric.ric_compile(h, exp["n_pad"])
        ric.ric_sync(h)
        got = {k: _copy_out(getattr(s, k), n)
               for k, n in (("input_ids", exp["n_pad"]), ("slot_mapping", exp["n_pad"]),
                            ("positions", exp["n_pad"]), ("query_start_loc", w.max_num_reqs + 1))}
        ric.ric_destroy(h)
    for k in got:
        assert np.array_equal(got[k].astype(np.int64), exp[k]), k


def _copy_out(ptr, n):
    """Read n int32 values at a device address the caller does not own as a tensor."""
    from ragged_input_compilation_amd import _ric
    return _ric.ric_read_device(ptr, 4 * n, np.int32)


def test_minimum_staging_forces_chunked_uploads(rt):
    """A staging buffer at its minimum size and a 300k-token request: the
    payload crosses many flushes; the compiled chunk near the end still reads
    the right token ids and block entries."""
    ric, runner = rt
    rng = np.random.default_rng(11)
    B, M = 16, 1 << 19
    T = 300_000
    c0, q = T - 4096, 4096
    tokens = rng.integers(0, 1 << 20, size=T).astype(np.int32)
    blocks = (rng.permutation(40000)[: -(-T // B)] + 1).astype(np.int32)
    req = workloads.Req(0, tokens, T, c0, q, blocks)
    w = _simple_rows_workload([req], B, 2, M, 40001)
    cfg = runner.config_of(w)
    cfg.staging_bytes = 96 * cfg.max_num_reqs + (64 << 10)     # the documented minimum
    b = runner.Batch(cfg)
    b.load_history(w)
    ref, order = replay_history(w)
    b.schedule_from(w, order)
    exp = expected_step(w, ref)
    s = b.compile(exp["n_pad"])
    assert_step_equal(b.step_outputs(s), exp, "min staging")
    cols = ric.ric_get_columns(b.h)
    whole = read_rows_i32(b.workspace, cols.tokens, cols.token_stride, [0], T)[0]
    assert np.array_equal(whole, tokens)
    b.close()
    bad = runner.config_of(w)
    bad.staging_bytes = 1024
    with pytest.raises(ric.RicError):
        runner.Batch(bad)


def test_more_layers_than_one_launch_holds(rt):
    """40 layers: the library splits them over launches of at most 32; every
    layer's cache gets its rows."""
    ric, runner = rt
    rng = np.random.default_rng(12)
    reqs = workloads.random_batch(rng, num_reqs=6, block_size=16, max_model_len=512, num_kv_blocks=256,
                                  max_q=64, max_c=300)
    w = _simple_rows_workload(reqs, 16, 8, 512, 256, row_heads=2, head_dim=64, layers=40)
    b, s, ref, order, exp, _ = _compile(rt, w)
    _full_kv_check(rt, w, b, s, exp)
    b.close()


def test_max_rows_batch(rt):
    """8000 rows (the row limit): every thread of the compile owns 32
    requests; decodes and short prefills mixed."""
    ric, runner = rt
    rng = np.random.default_rng(13)
    reqs = workloads.random_batch(rng, num_reqs=8000, block_size=16, max_model_len=64,
                                  num_kv_blocks=8000 * 4 + 1, max_q=3, max_c=40)
    w = _simple_rows_workload(reqs, 16, 8000, 64, 8000 * 4 + 1)
    b, s, ref, order, exp, _ = _compile(rt, w)
    assert_step_equal(b.step_outputs(s), exp, "8000 rows")
    b.close()


def test_non_power_of_two_block_size_at_scale(rt):
    """Block size 48 (a division, not a shift) over long chunks."""
    ric, runner = rt
    rng = np.random.default_rng(14)
    reqs = []
    pool = rng.permutation(np.arange(1, 5000)).astype(np.int32)
    nxt = 0
    for i, (c, q) in enumerate([(1000, 3000), (0, 2500), (4095, 1), (77, 1234)]):
        T = c + q + int(rng.integers(0, 50))
        nb = -(-(c + q) // 48)
        reqs.append(workloads.Req(i, rng.integers(0, 1 << 20, size=T).astype(np.int32), T, c, q,
                                  pool[nxt:nxt + nb]))
        nxt += nb
    w = _simple_rows_workload(reqs, 48, 4, 8192, 5000)
    b, s, ref, order, exp, _ = _compile(rt, w)
    assert_step_equal(b.step_outputs(s), exp, "B=48")
    b.close()


def test_two_million_token_step(rt):
    """2^21 scheduled tokens in one compile launch (eight 262144-token chunks
    at random cached offsets of 524288-token prompts, block size 64: 8192
    token tiles plus the per-request workgroup), compared in full with the
    oracle; the histories (16 MiB) reach the device in several staged
    uploads."""
    ric, runner = rt
    rng = np.random.default_rng(15)
    M, B, Q = 1 << 19, 64, 1 << 18
    pool = rng.permutation(np.arange(1, 70001)).astype(np.int32)
    reqs, nxt = [], 0
    for i in range(8):
        c = int(rng.integers(0, M - Q + 1))
        T = M if i % 2 == 0 else c + Q
        nb = -(-T // B)
        reqs.append(workloads.Req(i, rng.integers(0, 1 << 20, size=T).astype(np.int32), T, c, Q,
                                  pool[nxt:nxt + nb]))
        nxt += nb
    w = _simple_rows_workload(reqs, B, 8, M, 70001)
    b, s, ref, order, exp, _ = _compile(rt, w)
    assert s.num_actual_tokens == 1 << 21
    assert_step_equal(b.step_outputs(s), exp, "2^21 tokens")
    b.close()


def test_strided_sources_from_a_fused_qkv_tensor(rt):
    """K and V passed as strided views of one [N, Hq+2Hkv, D] projection
    output (row stride larger than the K/V row)."""
    ric, runner = rt
    w = workloads.get("mixed")
    b, s, ref, order, exp, _ = _compile(rt, w)
    n = exp["n_pad"]
    H, D = w.kv_heads, w.head_dim
    qkv = torch.randn((n, 32 + 2 * H, D), device="cuda").to(torch.bfloat16)
    k = qkv[:, 32:32 + H, :]
    v = qkv[:, 32 + H:, :]
    kc, vc = runner.alloc_caches(w, fill=0x0101)
    kv = runner.KVSet([k], [v], kc, vc, w.row_bytes, w.num_kv_blocks * w.block_size)
    runner.reshape_and_cache(kv, s.slot_mapping, n)
    torch.cuda.synchronize()
    slots = torch.from_numpy(exp["slot_mapping"][: exp["num_actual_tokens"]]).cuda()
    flat_k = kc[0].view(torch.int16).reshape(-1, H * D)
    flat_v = vc[0].view(torch.int16).reshape(-1, H * D)
    N = exp["num_actual_tokens"]
    assert torch.equal(flat_k[slots], k[:N].reshape(N, -1).view(torch.int16))
    assert torch.equal(flat_v[slots], v[:N].reshape(N, -1).view(torch.int16))
    b.close()


def test_c_program_through_the_abi(rt, tmp_path):
    """A plain-C program (tests/c_abi_step.c) runs the first page's worked
    example through ric.h: its printed outputs equal the page's values, and
    its K/V rows land at the printed slots, through the separate calls and
    through ric_compile_and_cache."""
    import json
    import subprocess
    from tests.test_abi import build_c_step
    ric, runner = rt
    exe = build_c_step(tmp_path / "c_abi_step", ric)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr[-2000:]
    got = json.loads(run.stdout)
    g = golden("p1_worked_example.json")["expect"]
    N = 6
    assert (got["num_reqs"], got["num_actual_tokens"], got["num_tokens_padded"]) == (3, N, 8)
    for k in ("query_start_loc", "seq_lens", "logits_indices"):
        assert got[k] == g[k], k
    for k in ("req_indices", "positions", "input_ids", "slot_mapping"):
        assert got[k][:N] == g[k], k
    assert got["req_indices"][N:] == [-1, -1] and got["slot_mapping"][N:] == [0, 0]
    assert got["cu_seqlens_k"] == [0, 6, 9, 19]
    assert got["sample_indices"] == [0, 5, -1]          # B's chunk is discarded
    # both writes: the separate calls (64-byte rows) and ric_compile_and_cache
    # (128-byte rows, one kernel), whose compile equals the first
    assert got["fused_slot_mapping"] == got["slot_mapping"]
    for name in ("k_cache_first_byte", "fused_v_cache_first_byte"):
        first = got[name]
        for t, s in enumerate(g["slot_mapping"]):
            assert first[s] == t + 1, name
        assert all(first[i] == 0 for i in range(4, len(first)) if i not in g["slot_mapping"]), name


def test_debug_dump_prints_the_step(rt, capsys):
    """RIC_DEBUG's dump shows the small per-step arrays of the worked example."""
    w = workloads.get("worked_example")
    b, s, ref, order, exp, _ = _compile(rt, w)
    b.debug_dump(s)
    out = capsys.readouterr().out
    assert "[ric] R=3 N=20 N_pad=32" in out
    assert "[ric] qsl        0 7 8 20\n" in out
    assert "[ric] seq_lens   7 6 22\n" in out
    assert "[ric] logits     6 7 19\n" in out
    assert "[ric] positions  0 1 2 3 4 5 6 5 10 11" in out
    assert "[ric] slot collisions 0, out-of-range slots 0" in out
    b.close()


def test_debug_check_finds_a_planted_collision(rt):
    """The debug check counts a slot shared by two real tokens: the worked
    example's slot list with token 5 redirected to token 4's slot."""
    ric, runner = rt
    w = workloads.get("worked_example")
    b, s, ref, order, exp, _ = _compile(rt, w)
    assert b.slot_collisions(s) == (0, 0)
    slots = torch.from_numpy(np.asarray(exp["slot_mapping"], np.int32)).cuda()
    slots[5] = slots[4]
    fake = ric.ric_step()
    fake.slot_mapping = slots.data_ptr()
    fake.num_tokens_padded = exp["n_pad"]
    fake.dev_scalars = s.dev_scalars
    assert b.slot_collisions(fake) == (1, 0)
    b.close()
