"""GPU parity for several KV-cache groups: per-group block tables and slot
mappings, a group without per-token slots, manager-to-kernel block expansion
of the exported table, condense moving every group's row, and every
group's slots following counts corrected on the device."""
import numpy as np
import pytest
import torch

import workloads
from oracle import batch as ref_batch, step as ref_step
from tests.gpu_helpers import read_rows_i32

pytestmark = pytest.mark.gpu

B0, B1, B2 = 16, 32, 8          # group block sizes: full attention, a second table, recurrent state
POOL0, POOL1, POOL2 = 40000, 20000, 3000
M = 2048


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_input_compilation_amd import _ric, runner
    return _ric, runner


def _cfg(ric, MR, budget):
    return ric.make_config(max_num_reqs=MR, max_model_len=M, block_size=B0, max_blocks_per_req=M // B0,
                           max_num_batched_tokens=budget, num_kv_blocks=POOL0, null_block=0, staging_bytes=0,
                           num_kv_groups=3, group_block_size=[0, B1, B2], group_num_kv_blocks=[0, POOL1, POOL2],
                           group_slot_mode=[0, ric.RIC_SLOTS_PER_TOKEN, ric.RIC_SLOTS_NONE])


def test_groups_compile_tables_and_condense(rt):
    ric, runner = rt
    rng = np.random.default_rng(61)
    MR = 48
    reqs = workloads.random_batch(rng, num_reqs=40, block_size=B0, max_model_len=M, num_kv_blocks=POOL0,
                                  max_q=100, max_c=900)
    p1 = list(rng.permutation(np.arange(1, POOL1)))
    p2 = list(rng.permutation(np.arange(1, POOL2)))
    budget = sum(r.num_scheduled for r in reqs) + 16
    b = runner.Batch(_cfg(ric, MR, budget))
    ref = ref_batch.RefBatch(MR, M, M // B0, POOL0)
    g1, g2 = {}, {}
    for r in reqs:
        b.add(r)
        ref.add_request(r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks)
        g1[r.req_id] = [int(p1.pop()) for _ in range(-(-(r.num_computed + r.num_scheduled) // B1))]
        g2[r.req_id] = [int(p2.pop())]
        half = len(g1[r.req_id]) // 2           # two appends, to exercise both paths
        ric.ric_append_blocks_group(b.h, r.req_id, 1, g1[r.req_id][:half])
        ric.ric_append_blocks_group(b.h, r.req_id, 1, g1[r.req_id][half:])
        ric.ric_replace_blocks_group(b.h, r.req_id, 2, g2[r.req_id])
        ref.append_blocks_group(r.req_id, 1, g1[r.req_id])
        ref.replace_blocks_group(r.req_id, 2, g2[r.req_id])
    for rid in (3, 11, 12, 30):
        ric.ric_remove_request(b.h, rid)
        ref.remove_request(rid)
    assert ric.ric_condense(b.h) == len(ref.condense())
    order = [rid for rid in ref.req_ids_by_row() if rid is not None]
    assert b.row_order() == order
    by_id = {r.req_id: r for r in reqs}
    c = [by_id[i].num_computed for i in order]
    q = [by_id[i].num_scheduled for i in order]
    ric.ric_schedule(b.h, c, q)
    ref.schedule(c, q)
    rows = ref.step_rows()
    n_pad = sum(q) + 5
    want = ref_step.compile_step(rows, block_size=B0, max_num_reqs=MR, max_model_len=M,
                                 max_num_batched_tokens=budget, num_kv_blocks=POOL0, n_pad=n_pad)
    s = b.compile(n_pad)
    got = b.step_outputs(s)
    for k in ("input_ids", "positions", "slot_mapping", "query_start_loc", "seq_lens", "cu_seqlens_k"):
        assert np.array_equal(np.asarray(got[k], np.int64), np.asarray(want[k], np.int64)), k
    group1_rows = [ref.rows[i].group_blocks[1] for i in range(len(order))]
    want1 = ref_step.group_slot_mapping(want["positions"], want["req_indices"], group1_rows, B1)
    assert s.group_slot_mapping[0] == s.slot_mapping
    assert s.group_slot_mapping[2] is None and s.group_slot_mapping[3] is None
    got1 = ric.ric_read_device(s.group_slot_mapping[1], 4 * n_pad, np.int32)
    assert np.array_equal(got1.astype(np.int64), np.asarray(want1, np.int64))
    assert int(got["dev_scalars"][6]) == 0

    # exported tables: group 1 as stored and expanded to 16-token kernel blocks; group 2
    for group, ratio, cap in ((1, 1, M // B1), (1, 2, 2 * (M // B1)), (2, 1, M // B2)):
        width = min(cap, max(len(r.group_blocks[group]) for r in ref.rows[:len(order)]) * ratio + 2)
        dst = torch.full((len(order), width), 7, dtype=torch.int32, device="cuda")
        ric.ric_block_table_padded(b.h, width, -1, dst.data_ptr(), group=group, kernel_blocks_per_block=ratio)
        torch.cuda.synchronize()
        exp = ref_step.padded_block_table(rows, width, -1, ratio, blocks_of=lambda i, r: ref.rows[i].group_blocks[group])
        assert np.array_equal(dst.cpu().numpy(), np.asarray(exp, np.int32)), (group, ratio)

    # the persistent per-group tables through the column views
    cols = ric.ric_get_columns(b.h)
    assert cols.group_blocks[0] == cols.blocks and cols.group_block_stride[0] == cols.block_stride
    assert cols.group_blocks[3] is None and cols.group_block_stride[3] == 0
    for group in (1, 2):
        counts = ric.ric_read_device(cols.group_num_blocks[group], 4 * len(order), np.int32)
        for i in range(len(order)):
            want_ids = ref.rows[i].group_blocks[group]
            assert counts[i] == len(want_ids), (group, i)
            got_ids = read_rows_i32(b.workspace, cols.group_blocks[group], cols.group_block_stride[group], [i],
                                    len(want_ids))[0]
            assert list(got_ids) == list(want_ids), (group, i)

    # a row whose second table does not cover its positions is rejected
    rid0 = order[0]
    ric.ric_replace_blocks_group(b.h, rid0, 1, [])
    with pytest.raises(ric.RicError):
        ric.ric_schedule(b.h, c, q)
    with pytest.raises(ric.RicError):
        ric.ric_append_blocks_group(b.h, rid0, 3, [1])          # no such group
    with pytest.raises(ric.RicError):
        ric.ric_append_blocks_group(b.h, rid0, 2, [POOL2])      # outside group 2's pool
    b.close()


def test_group_slots_follow_corrected_counts(rt):
    """Counts corrected on the device (asynchronous speculative decoding) move
    every group's slots with them: group 0's compile and group 1's slot
    mapping equal the oracle's on the corrected positions."""
    ric, runner = rt
    rng = np.random.default_rng(62)
    MR, R = 16, 12
    b = runner.Batch(_cfg(ric, MR, 64))
    ref = ref_batch.RefBatch(MR, M, M // B0, POOL0)
    p0 = list(rng.permutation(np.arange(1, POOL0)))
    p1 = list(rng.permutation(np.arange(1, POOL1)))
    c_opt, d = [], []
    for rid in range(R):
        T = int(rng.integers(8, 400))
        toks = rng.integers(0, 50000, T)
        b0 = [int(p0.pop()) for _ in range(-(-T // B0))]
        b1 = [int(p1.pop()) for _ in range(-(-T // B1))]
        ric.ric_add_request(b.h, rid, toks, T, T - 1, b0)
        ref.add_request(rid, toks, T, T - 1, b0)
        ric.ric_append_blocks_group(b.h, rid, 1, b1)
        ref.append_blocks_group(rid, 1, b1)
        d.append(int(rng.integers(0, 4)))
        c_opt.append(T - 1)
    ric.ric_schedule(b.h, c_opt, [1] * R)
    ref.schedule(c_opt, [1] * R)
    pos_of = [int(x) for x in rng.permutation(R)]
    acc = np.zeros(R, np.int32)
    kept = np.full((R, 4), -1, np.int32)
    for i in range(R):
        v = int(rng.integers(1, d[i] + 2))
        acc[pos_of[i]] = v
        kept[pos_of[i], :v] = rng.integers(90000, 99999, v)
    acc_dev, kept_dev = torch.from_numpy(acc).cuda(), torch.from_numpy(kept).cuda()
    rows = list(range(R))
    ric.ric_correct_computed(b.h, rows, pos_of, d, acc_dev.data_ptr(), R, kept_dev.data_ptr(), 4)
    cc = [ref.rows[i].num_computed for i in range(R)]
    assert ref_step.correct_computed(cc, [ref.rows[i].tokens for i in range(R)], rows, pos_of, d, acc,
                                     kept.tolist()) == 0
    for i in range(R):
        ref.rows[i].num_computed = cc[i]
    want = ref_step.compile_step(ref.step_rows(), block_size=B0, max_num_reqs=MR, max_model_len=M,
                                 max_num_batched_tokens=64, num_kv_blocks=POOL0, n_pad=R)
    s = b.compile(R)
    got = b.step_outputs(s)
    for k in ("input_ids", "positions", "slot_mapping", "seq_lens", "cu_seqlens_k"):
        assert np.array_equal(np.asarray(got[k], np.int64), np.asarray(want[k], np.int64)), k
    want1 = ref_step.group_slot_mapping(want["positions"], want["req_indices"],
                                        [ref.rows[i].group_blocks[1] for i in range(R)], B1)
    got1 = ric.ric_read_device(s.group_slot_mapping[1], 4 * R, np.int32)
    assert np.array_equal(got1.astype(np.int64), np.asarray(want1, np.int64))
    assert any(cc[i] != c_opt[i] for i in range(R))          # some counts really moved
    b.close()
