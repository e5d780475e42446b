"""A long seeded serving loop on one handle, every operation mixed: arrivals
(with prefix-cache hits), finishes, abort-and-resubmit, preemption with
replaced block rows, condense, decode appends, prefill chunks, a second
KV-cache group with its own block size, device-side appends of sampled
tokens, history truncation, device-side corrections of computed counts (some
with out-of-range accepted counts), and K/V writes, some of them through the
single compile + K/V kernel (ric_compile_and_cache, rows of 1 KiB and 256 B).  Every step's compile
(group 1's slots included), every corrected count and every written cache row
equals the oracle's."""
import numpy as np
import pytest
import torch

from oracle import batch as ref_batch, step as ref_step

pytestmark = pytest.mark.gpu

B0, B1 = 8, 16
MR, M = 24, 256
POOL = 20000
BUDGET = 192
ROW = 64
ROWF = (1024, 256)   # rows the single compile + K/V kernel takes (a wide and a narrow size)


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_input_compilation_amd import _ric, runner
    return _ric, runner


def test_serving_loop_soak(rt):
    ric, runner = rt
    rng = np.random.default_rng(2024)
    cfg = ric.make_config(max_num_reqs=MR, max_model_len=M, block_size=B0, max_blocks_per_req=M // B0,
                          max_num_batched_tokens=BUDGET, num_kv_blocks=POOL, null_block=0, staging_bytes=0,
                          num_kv_groups=2, group_block_size=[0, B1], group_num_kv_blocks=[0, POOL],
                          group_slot_mode=[0, ric.RIC_SLOTS_PER_TOKEN])
    b = runner.Batch(cfg)
    ref = ref_batch.RefBatch(MR, M, M // B0, POOL)
    free0 = list(rng.permutation(np.arange(1, POOL)))
    free1 = list(rng.permutation(np.arange(1, POOL)))
    done = {}                      # request id -> tokens whose K/V is valid
    next_id = 0
    cache = torch.zeros((POOL * B0, ROW), dtype=torch.uint8, device="cuda")
    cache_ref = np.zeros((POOL * B0, ROW), np.uint8)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    kf = [torch.zeros((POOL * B0, r), dtype=torch.uint8, device="cuda") for r in ROWF]
    vf = [torch.zeros((POOL * B0, r), dtype=torch.uint8, device="cuda") for r in ROWF]
    kf_ref = [np.zeros((POOL * B0, r), np.uint8) for r in ROWF]
    vf_ref = [np.zeros((POOL * B0, r), np.uint8) for r in ROWF]
    counts = dict(corrections=0, bad_counts=0, kv_writes=0, sampled=0, truncations=0, fused=0)

    def row(rid):
        return ref.rows[ref.row_of[rid]]

    def cover(rid):
        """Give both groups enough blocks for the row's whole history."""
        r = row(rid)
        T = len(r.tokens)
        need0 = -(-T // B0) - len(r.blocks)
        if need0 > 0:
            ids = [int(free0.pop()) for _ in range(need0)]
            ric.ric_append_blocks(b.h, rid, ids)
            ref.append_blocks(rid, ids)
        need1 = -(-T // B1) - len(r.group_blocks.get(1, []))
        if need1 > 0:
            ids = [int(free1.pop()) for _ in range(need1)]
            ric.ric_append_blocks_group(b.h, rid, 1, ids)
            ref.append_blocks_group(rid, 1, ids)

    def arrive(rid):
        T = int(rng.integers(2, 60))
        toks = rng.integers(0, 1 << 20, T)
        c0 = int(rng.integers(0, T))
        ric.ric_add_request(b.h, rid, toks, T, c0, [])
        ref.add_request(rid, toks, T, c0, [])
        cover(rid)
        done[rid] = c0

    for step_no in range(600):
        for rid in list(done):
            x = rng.random()
            if x < 0.06:                                           # finished
                ric.ric_remove_request(b.h, rid)
                ref.remove_request(rid)
                del done[rid]
            elif x < 0.08:                                         # aborted, resubmitted under the same id
                ric.ric_remove_request(b.h, rid)
                ref.remove_request(rid)
                arrive(rid)
            elif x < 0.11:                                         # preempted and resumed: new block rows
                r = row(rid)
                ids0 = [int(free0.pop()) for _ in range(len(r.blocks))]
                ids1 = [int(free1.pop()) for _ in range(len(r.group_blocks.get(1, [])))]
                ric.ric_replace_blocks(b.h, rid, ids0)
                ref.replace_blocks(rid, ids0)
                ric.ric_replace_blocks_group(b.h, rid, 1, ids1)
                ref.replace_blocks_group(rid, 1, ids1)
        while len(done) < MR and rng.random() < 0.45:
            arrive(next_id)
            next_id += 1
        assert ric.ric_condense(b.h) == len(ref.condense())
        order = [rid for rid in ref.req_ids_by_row() if rid is not None]
        assert b.row_order() == order, step_no
        if not order:
            continue

        # decoding rows get a token; occasionally a history is cut back first
        for rid in order:
            r = row(rid)
            if rng.random() < 0.05 and len(r.tokens) > max(done[rid], r.num_prompt) + 1:
                keep = int(rng.integers(max(done[rid], r.num_prompt) + 1, len(r.tokens) + 1))
                ric.ric_truncate_tokens(b.h, rid, keep)
                ref.truncate_tokens(rid, keep)
                counts["truncations"] += 1
            if done[rid] >= len(r.tokens) and len(r.tokens) < M:
                tok = [int(rng.integers(0, 1 << 20))]
                ric.ric_append_tokens(b.h, rid, tok)
                ref.append_tokens(rid, tok)
                cover(rid)
        c, q = [], []
        for rid in order:
            T = len(row(rid).tokens)
            ci = min(done[rid], T - 1)
            c.append(ci)
            q.append(int(min(T - ci, rng.integers(1, 12))))
        while sum(q) > BUDGET:
            q[int(np.argmax(q))] -= 1
        ric.ric_schedule(b.h, c, q)
        ref.schedule(c, q)
        R = len(order)

        if rng.random() < 0.3:                                     # optimistic counts corrected on the device
            n = int(rng.integers(1, R + 1))
            rows = [int(x) for x in rng.choice(R, size=n, replace=False)]
            d = [int(rng.integers(0, min(c[i], 3) + 1)) for i in rows]
            prev_len = R + 3
            pos = [int(x) for x in rng.choice(prev_len, size=n, replace=False)]
            acc = rng.integers(0, 6, prev_len).astype(np.int32)   # some outside [1, d + 1]
            kept = rng.integers(0, 1 << 20, (prev_len, 4)).astype(np.int32)
            status.zero_()
            acc_dev, kept_dev = torch.from_numpy(acc).cuda(), torch.from_numpy(kept).cuda()
            ric.ric_correct_computed(b.h, rows, pos, d, acc_dev.data_ptr(), prev_len, kept_dev.data_ptr(), 4,
                                     status.data_ptr())
            cc = [ref.rows[i].num_computed for i in range(R)]
            bad = ref_step.correct_computed(cc, [ref.rows[i].tokens for i in range(R)], rows, pos, d, acc,
                                            kept.tolist())
            for i in range(R):
                ref.rows[i].num_computed = cc[i]
            torch.cuda.synchronize()
            assert int(status.item()) == bad, step_no
            counts["corrections"] += 1
            counts["bad_counts"] += bad

        N = sum(q)
        n_pad = min(BUDGET, N + int(rng.integers(0, 5)))
        step_rows = ref.step_rows()
        want = ref_step.compile_step(step_rows, block_size=B0, max_num_reqs=MR, max_model_len=M,
                                     max_num_batched_tokens=BUDGET, num_kv_blocks=POOL, n_pad=n_pad)
        fused = rng.random() < 0.25
        fi = step_no % 2                                           # which of the two row sizes
        if fused:                                                  # compile + K/V in one kernel
            rowf = ROWF[fi]
            # always 1 KiB drawn (the seeded trajectory does not depend on fi);
            # narrow steps use the first rowf bytes of each row
            srck = np.ascontiguousarray(rng.integers(0, 256, (n_pad, ROWF[0]), dtype=np.uint8)[:, :rowf])
            srcv = np.ascontiguousarray(rng.integers(0, 256, (n_pad, ROWF[0]), dtype=np.uint8)[:, :rowf])
            k_dev, v_dev = torch.from_numpy(srck).cuda(), torch.from_numpy(srcv).cuda()
            status.zero_()
            s = ric.ric_compile_and_cache(b.h, n_pad, [k_dev.data_ptr()], [v_dev.data_ptr()], [kf[fi].data_ptr()],
                                          [vf[fi].data_ptr()], rowf, POOL * B0, dev_status=status.data_ptr(),
                                          flags=ric.RIC_FUSE_ALWAYS)
        else:
            s = b.compile(n_pad)
        got = b.step_outputs(s)
        for k in ("input_ids", "positions", "req_indices", "slot_mapping", "query_start_loc", "seq_lens",
                  "cu_seqlens_k", "logits_indices", "discard", "sample_indices"):
            assert np.array_equal(np.asarray(got[k], np.int64), np.asarray(want[k], np.int64)), (step_no, k)
        assert int(got["dev_scalars"][6]) == 0
        want1 = ref_step.group_slot_mapping(want["positions"], want["req_indices"],
                                            [ref.rows[i].group_blocks[1] for i in range(R)], B1)
        got1 = ric.ric_read_device(s.group_slot_mapping[1], 4 * n_pad, np.int32)
        assert np.array_equal(got1.astype(np.int64), np.asarray(want1, np.int64)), step_no

        if fused:
            assert int(status.item()) == 0, step_no
            slots = np.asarray(want["slot_mapping"][:N], np.int64)
            kf_ref[fi][slots] = srck[:N]
            vf_ref[fi][slots] = srcv[:N]
            touched = torch.from_numpy(np.unique(slots)).cuda()
            assert np.array_equal(kf[fi][touched].cpu().numpy(), kf_ref[fi][touched.cpu().numpy()]), step_no
            assert np.array_equal(vf[fi][touched].cpu().numpy(), vf_ref[fi][touched.cpu().numpy()]), step_no
            counts["fused"] += 1

        if rng.random() < 0.2:                                     # this step's K/V rows
            src = rng.integers(0, 256, (n_pad, ROW), dtype=np.uint8)
            src_dev = torch.from_numpy(src).cuda()
            ric.ric_reshape_and_cache([src_dev.data_ptr()], [src_dev.data_ptr()], [cache.data_ptr()],
                                      [cache.data_ptr()], s.slot_mapping, n_pad, ROW, POOL * B0,
                                      stream=runner.current_stream())
            slots = np.asarray(want["slot_mapping"][:N], np.int64)
            cache_ref[slots] = src[:N]
            touched = np.unique(slots)
            assert np.array_equal(cache[torch.from_numpy(touched).cuda()].cpu().numpy(), cache_ref[touched])
            counts["kv_writes"] += 1

        for i, rid in enumerate(order):
            done[rid] = ref.rows[i].num_computed + q[i]

        if rng.random() < 0.25:                                    # sampled tokens appended on the device
            rows = [i for i in range(R) if len(ref.rows[i].tokens) < M and rng.random() < 0.7]
            if rows:
                y = rng.integers(0, 1 << 20, len(rows)).astype(np.int32)
                src_index = [int(x) for x in rng.permutation(len(rows))]
                y_dev = torch.from_numpy(y).cuda()
                ric.ric_append_sampled(b.h, rows, y_dev.data_ptr(), len(rows), src_index)
                for k, i in enumerate(rows):
                    ref.append_tokens(order[i], [int(y[src_index[k]])])
                    cover(order[i])
                counts["sampled"] += 1

    assert all(v > 5 for v in counts.values()), counts
    b.close()
