"""GPU parity for the rows after the core path: dense padded block tables,
the device-side append of sampled tokens (async-scheduling input path),
speculative-decoding indices, and the device-side correction of optimistic
computed counts (asynchronous speculative decoding).  cu_seqlens_k is compared
with every compile in test_gpu_parity.py."""
import numpy as np
import pytest
import torch

import workloads
from oracle import batch as ref_batch, step as ref_step
from tests.gpu_helpers import expected_step, replay_history

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_input_compilation_amd import _ric, runner
    return _ric, runner


@pytest.mark.parametrize("name", ["mixed", "churn", "worked_example"])
def test_padded_block_table(rt, name):
    ric, runner = rt
    w = workloads.get(name)
    b = runner.Batch(runner.config_of(w))
    b.load_history(w)
    ref, order = replay_history(w)
    b.schedule_from(w, order)
    rows = ref.step_rows()
    width = min(max(len(r.blocks) for r in rows) + 3, w.max_blocks_per_req)
    want = np.asarray(ref_step.padded_block_table(rows, width), np.int32)
    dst = torch.full((len(rows), width), 12345, dtype=torch.int32, device="cuda")
    ric.ric_block_table_padded(b.h, width, -1, dst.data_ptr())
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy(), want)
    narrow = max(1, width // 3)
    dst2 = torch.zeros((len(rows), narrow), dtype=torch.int32, device="cuda")
    ric.ric_block_table_padded(b.h, narrow, 0, dst2.data_ptr())
    torch.cuda.synchronize()
    assert np.array_equal(dst2.cpu().numpy(), np.asarray(ref_step.padded_block_table(rows, narrow, 0), np.int32))
    b.close()


def test_padded_block_table_needs_a_schedule(rt):
    ric, runner = rt
    w = workloads.get("worked_example")
    b = runner.Batch(runner.config_of(w))
    b.load_history(w)
    with pytest.raises(ric.RicError) as e:
        ric.ric_block_table_padded(b.h, 4, -1, 0)
    assert e.value.code == ric.RIC_ESTATE
    b.schedule_from(w)
    dst = torch.zeros((3, 4), dtype=torch.int32, device="cuda")
    for kw in (dict(group=1), dict(group=-1), dict(kernel_blocks_per_block=0),
               dict(kernel_blocks_per_block=1 << 30)):          # expanded ids would overflow int32
        with pytest.raises(ric.RicError) as e:
            ric.ric_block_table_padded(b.h, 4, -1, dst.data_ptr(), **kw)
        assert e.value.code == ric.RIC_EINVAL, kw
    with pytest.raises(ric.RicError):
        ric.ric_block_table_padded(b.h, w.max_blocks_per_req + 1, -1, dst.data_ptr())   # wider than the table
    b.close()


def test_append_sampled_decode_loop(rt):
    """Twelve decode steps where last step's sampled ids (a device array in
    sample order) are appended through a row -> sample-position map, with a
    request finishing and the batch condensed midway.  Every step's compile
    equals the oracle's, whose histories got the same ids on the host."""
    ric, runner = rt
    rng = np.random.default_rng(21)
    B, MR, M = 16, 16, 256
    cfg = ric.make_config(max_num_reqs=MR, max_model_len=M, block_size=B, max_blocks_per_req=M // B,
                          max_num_batched_tokens=64, num_kv_blocks=2048, null_block=0, staging_bytes=0)
    b = runner.Batch(cfg)
    ref = ref_batch.RefBatch(MR, M, M // B, 2048)
    free = list(rng.permutation(np.arange(1, 2048)))
    for rid in range(10):
        T = int(rng.integers(3, 60))
        toks = rng.integers(0, 50000, T)
        blks = [int(free.pop()) for _ in range(-(-(T + 20) // B))]
        ric.ric_add_request(b.h, rid, toks, T, T - 1, blks)
        ref.add_request(rid, toks, T, T - 1, blks)
    prev_sample_pos = None      # request id -> position in last step's sampled array
    sampled_host = None
    sampled_dev = None
    for step_no in range(12):
        if step_no == 5:
            for rid in (2, 7):
                ric.ric_remove_request(b.h, rid)
                ref.remove_request(rid)
            ric.ric_condense(b.h)
            ref.condense()
        order = [rid for rid in ref.req_ids_by_row() if rid is not None]
        assert b.row_order() == order
        if sampled_dev is not None:
            rows = [i for i, rid in enumerate(order) if rid in prev_sample_pos]
            src = [prev_sample_pos[order[i]] for i in rows]
            ric.ric_append_sampled(b.h, rows, sampled_dev.data_ptr(), sampled_dev.numel(), src)
            for i, j in zip(rows, src):
                ref.append_tokens(order[i], [int(sampled_host[j])])
        c = [len(ref.rows[i].tokens) - 1 for i in range(len(order))]
        ric.ric_schedule(b.h, c, [1] * len(order))
        ref.schedule(c, [1] * len(order))
        want = ref_step.compile_step(ref.step_rows(), block_size=B, max_num_reqs=MR, max_model_len=M,
                                     max_num_batched_tokens=64, num_kv_blocks=2048, n_pad=len(order))
        s = b.compile(len(order))
        got = b.step_outputs(s)
        for k in ("input_ids", "positions", "slot_mapping", "seq_lens", "cu_seqlens_k", "query_start_loc"):
            assert np.array_equal(np.asarray(got[k], np.int64), np.asarray(want[k], np.int64)), (step_no, k)
        assert int(got["dev_scalars"][7]) == 0
        # "sample": one new id per request; request order[i]'s id sits at
        # position perm[i] of the device array (a sampler's own order)
        perm = rng.permutation(len(order))
        sampled_host = rng.integers(0, 50000, len(order)).astype(np.int32)
        sampled_dev = torch.from_numpy(sampled_host).cuda()
        prev_sample_pos = {order[i]: int(perm[i]) for i in range(len(order))}
    with pytest.raises(ric.RicError):
        ric.ric_append_sampled(b.h, [0, 0], sampled_dev.data_ptr(), sampled_dev.numel(), [0, 1])
    with pytest.raises(ric.RicError):
        ric.ric_append_sampled(b.h, [0], sampled_dev.data_ptr(), sampled_dev.numel(), [99])
    b.close()


@pytest.mark.parametrize("name", ["mixed", "churn", "decode_heavy", "worked_example"])
def test_spec_decode_metadata(rt, name):
    """Random draft counts (0..7, at most q-1 per row): every index array
    equals the oracle's, computed from the oracle's own compile."""
    ric, runner = rt
    w = workloads.get(name)
    b = runner.Batch(runner.config_of(w))
    b.load_history(w)
    ref, order = replay_history(w)
    b.schedule_from(w, order)
    exp = expected_step(w, ref)
    with pytest.raises(ric.RicError) as e:
        ric.ric_spec_decode_metadata(b.h, [0] * len(order))
    assert e.value.code == ric.RIC_ESTATE
    b.compile(exp["n_pad"])
    rng = np.random.default_rng(41)
    rows = ref.step_rows()
    for trial in range(3):
        d = [0] * len(rows) if trial == 0 else \
            [int(rng.integers(0, min(r.num_scheduled - 1, 7) + 1)) for r in rows]
        want = ref_step.spec_decode_metadata(exp["query_start_loc"], exp["input_ids"], d)
        out = ric.ric_spec_decode_metadata(b.h, d)
        assert (out.num_logits, out.num_draft_tokens) == (len(want["logits_indices"]), sum(d))
        for key, n in (("logits_indices", out.num_logits), ("cu_num_logits", len(rows) + 1),
                       ("target_logits_indices", out.num_draft_tokens),
                       ("bonus_logits_indices", len(rows)), ("draft_token_ids", out.num_draft_tokens)):
            got = ric.ric_read_device(getattr(out, key), 4 * n, np.int32) if n else np.zeros(0, np.int32)
            assert np.array_equal(got.astype(np.int64), np.asarray(want[key], np.int64)), (trial, key)
        if trial == 0:
            assert np.array_equal(np.asarray(want["logits_indices"]), exp["logits_indices"][:len(rows)])
    if any(r.num_scheduled == 1 for r in rows):
        bad = [r.num_scheduled for r in rows]       # d = q: one too many
        with pytest.raises(ric.RicError):
            ric.ric_spec_decode_metadata(b.h, bad)
    b.close()


def test_async_spec_decode_correction_loop(rt):
    """Eight rounds of speculative decoding over ten requests.  Each round has
    a synchronous step (fresh drafts appended, counts known) and then an
    asynchronous one: the host schedules every row as if all its drafts had
    been accepted, and ric_correct_computed lowers the counts on the device
    from an accepted-count array in the sampler's own order, writing the last
    kept token into the history.  Afterwards the host learns what was kept and
    drops the rejected drafts (ric_truncate_tokens), and the step's new token
    is appended from the device (ric_append_sampled).  Two requests finish and the batch is condensed midway.  Every
    compile, the device's computed counts and histories equal the oracle's."""
    ric, runner = rt
    rng = np.random.default_rng(33)
    B, MR, M = 16, 16, 512
    NB = 4096
    cfg = ric.make_config(max_num_reqs=MR, max_model_len=M, block_size=B, max_blocks_per_req=M // B,
                          max_num_batched_tokens=128, num_kv_blocks=NB, null_block=0, staging_bytes=0)
    b = runner.Batch(cfg)
    ref = ref_batch.RefBatch(MR, M, M // B, NB)
    free = list(rng.permutation(np.arange(1, NB)))
    count = {}                          # request id -> tokens with valid K/V (the last token is the next input)
    for rid in range(10):
        T = int(rng.integers(5, 80))
        toks = rng.integers(0, 50000, T)
        blks = [int(free.pop()) for _ in range(M // B)]
        ric.ric_add_request(b.h, rid, toks, T, T - 1, blks)
        ref.add_request(rid, toks, T, T - 1, blks)
        count[rid] = T - 1
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def compile_and_compare(tag):
        order = [rid for rid in ref.req_ids_by_row() if rid is not None]
        n = sum(ref.rows[i].num_scheduled for i in range(len(order)))
        want = ref_step.compile_step(ref.step_rows(), block_size=B, max_num_reqs=MR, max_model_len=M,
                                     max_num_batched_tokens=128, num_kv_blocks=NB, n_pad=n)
        got = b.step_outputs(b.compile(n))
        for k in ("input_ids", "positions", "slot_mapping", "seq_lens", "cu_seqlens_k", "query_start_loc",
                  "logits_indices", "req_indices"):
            assert np.array_equal(np.asarray(got[k], np.int64), np.asarray(want[k], np.int64)), (tag, k)
        assert np.array_equal(np.asarray(got["discard"], np.int64), np.asarray(want["discard"], np.int64)), tag
        assert int(got["dev_scalars"][4]) == max(want["seq_lens"]), tag      # exact max after correction
        cols = ric.ric_get_columns(b.h)
        R = len(order)
        dev_c = ric.ric_read_device(cols.num_computed, 4 * R, np.int32)
        assert list(dev_c) == [ref.rows[i].num_computed for i in range(R)], tag
        for i in range(R):
            T = len(ref.rows[i].tokens)
            row = ric.ric_read_device(cols.tokens + 4 * i * cols.token_stride, 4 * T, np.int32)
            assert list(row) == ref.rows[i].tokens, (tag, i)

    for rnd in range(8):
        if rnd == 4:
            for rid in (3, 6):
                ric.ric_remove_request(b.h, rid)
                ref.remove_request(rid)
                del count[rid]
            ric.ric_condense(b.h)
            ref.condense()
        order = [rid for rid in ref.req_ids_by_row() if rid is not None]
        assert b.row_order() == order
        R = len(order)
        # synchronous step: the last token plus d fresh drafts
        d = [int(rng.integers(0, 5)) for _ in range(R)]
        for i, rid in enumerate(order):
            drafts = rng.integers(60000, 70000, d[i])
            ric.ric_append_tokens(b.h, rid, drafts)
            ref.append_tokens(rid, drafts)
        c = [count[rid] for rid in order]
        q = [di + 1 for di in d]
        ric.ric_schedule(b.h, c, q)
        ref.schedule(c, q)
        compile_and_compare((rnd, "sync"))
        # the sampler keeps v = accepted drafts + 1 tokens per row, reported in its own order
        pos_of = [int(x) for x in rng.permutation(R)]
        width = max(d) + 1
        v = [int(rng.integers(1, di + 2)) for di in d]
        kept = np.full((R, width), -1, np.int32)
        acc = np.zeros(R, np.int32)
        for i, rid in enumerate(order):
            toks = ref.rows[i].tokens
            row_kept = toks[c[i] + 1:c[i] + v[i]] + [int(rng.integers(80000, 90000))]
            kept[pos_of[i], :v[i]] = row_kept
            acc[pos_of[i]] = v[i]
        kept_dev = torch.from_numpy(kept).cuda()
        acc_dev = torch.from_numpy(acc).cuda()
        # asynchronous step: counts advanced as if every draft was accepted,
        # one placeholder for the next input, then the device correction
        for i, rid in enumerate(order):
            ric.ric_append_tokens(b.h, rid, [-5])
            ref.append_tokens(rid, [-5])
        c_opt = [c[i] + d[i] + 1 for i in range(R)]
        ric.ric_schedule(b.h, c_opt, [1] * R)
        ref.schedule(c_opt, [1] * R)
        rows = [int(x) for x in rng.permutation(R)]
        ric.ric_correct_computed(b.h, rows, [pos_of[i] for i in rows], [d[i] for i in rows], acc_dev.data_ptr(),
                                 R, kept_dev.data_ptr(), width, status.data_ptr())
        cc = [ref.rows[i].num_computed for i in range(R)]
        bad = ref_step.correct_computed(cc, [ref.rows[i].tokens for i in range(R)], rows,
                                        [pos_of[i] for i in rows], [d[i] for i in rows], acc, kept.tolist())
        assert bad == 0
        for i in range(R):
            ref.rows[i].num_computed = cc[i]
            assert cc[i] == c[i] + v[i]
        compile_and_compare((rnd, "async"))
        # the host learns what was kept: rejected drafts leave the history,
        # and the async step's own sampled token (still on the device, in the
        # sampler's order) follows the kept ones
        for i, rid in enumerate(order):
            keep = c[i] + v[i] + 1
            ric.ric_truncate_tokens(b.h, rid, keep)
            ref.truncate_tokens(rid, keep)
            count[rid] = keep
        y = rng.integers(0, 50000, R).astype(np.int32)
        y_dev = torch.from_numpy(y).cuda()
        y_pos = [int(x) for x in rng.permutation(R)]          # row i's token at y[y_pos[i]]
        ric.ric_append_sampled(b.h, list(range(R)), y_dev.data_ptr(), R, y_pos)
        for i, rid in enumerate(order):
            ref.append_tokens(rid, [int(y[y_pos[i]])])
    assert int(status.item()) == 0

    # out-of-range kept counts leave their rows alone and are counted
    order = [rid for rid in ref.req_ids_by_row() if rid is not None]
    R = len(order)
    c = [count[rid] for rid in order]
    ric.ric_schedule(b.h, c, [1] * R)
    ref.schedule(c, [1] * R)
    acc_bad = torch.tensor([0, 3, 1] + [1] * (R - 3), dtype=torch.int32, device="cuda")
    ric.ric_correct_computed(b.h, [0, 1, 2], [0, 1, 2], [1, 1, 0], acc_bad.data_ptr(), R, 0, 0, status.data_ptr())
    compile_and_compare("bad counts")               # rows 0 and 1 unchanged, row 2 (d = 0, v = 1) unchanged
    assert int(status.item()) == 2
    with pytest.raises(ric.RicError) as e:          # after the compile
        ric.ric_correct_computed(b.h, [0], [0], [0], acc_bad.data_ptr(), R)
    assert e.value.code == ric.RIC_ESTATE
    ric.ric_schedule(b.h, c, [1] * R)
    for args in (([0, 0], [0, 1], [0, 0]),           # row twice
                 ([0], [R], [0]),                    # position past prev_len
                 ([0], [0], [c[0] + 1]),             # more drafts than the count holds
                 ([R], [0], [0])):                   # row not scheduled
        with pytest.raises(ric.RicError) as e:
            ric.ric_correct_computed(b.h, *args, acc_bad.data_ptr(), R)
        assert e.value.code == ric.RIC_EINVAL, args
    with pytest.raises(ric.RicError) as e:           # stride cannot hold d + 1 tokens
        ric.ric_correct_computed(b.h, [0], [0], [2], acc_bad.data_ptr(), R, acc_bad.data_ptr(), 2)
    assert e.value.code == ric.RIC_EINVAL
    with pytest.raises(ric.RicError) as e:           # into the prompt
        ric.ric_truncate_tokens(b.h, order[0], ref.rows[0].num_prompt - 1)
    assert e.value.code == ric.RIC_ERANGE
    b.close()
