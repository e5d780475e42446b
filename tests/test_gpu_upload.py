"""Delta uploads on both sides of the in-place limit.

A flush's log is read by the scatter kernel straight from pinned host memory
when it is at most 64 KiB and no op exceeds 2048 words; otherwise it is copied
into device staging first.  These flushes straddle both limits (one request of
2044-2052 tokens per flush; groups of 17-21 requests of 800 tokens per flush),
then a step is scheduled and compiled: every row of the column store and every
compile output must equal the oracle's."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import assert_step_equal, expected_step, read_rows_i32, replay_history

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_input_compilation_amd import _ric, runner
    return _ric, runner


def _workload(groups, B, max_model_len, num_kv_blocks):
    reqs = [r for g in groups for r in g]
    N = sum(r.num_scheduled for r in reqs)
    mr = 1 << max(0, (len(reqs) - 1).bit_length())
    return workloads.Workload("uploads", block_size=B, max_num_reqs=mr, max_model_len=max_model_len,
                              max_blocks_per_req=-(-max_model_len // B), max_num_batched_tokens=N,
                              num_kv_blocks=num_kv_blocks, kv_heads=8, head_dim=128, kv_dtype="bf16",
                              num_layers=1, hidden_size=256, gather="all", initial=reqs, capture_sizes=[N],
                              seed=4243)


def test_uploads_around_the_in_place_limits(rt):
    ric, runner = rt
    rng = np.random.default_rng(29)
    B = 16
    pool = rng.permutation(np.arange(1, 16384, dtype=np.int32))
    used = 0
    groups, rid = [], 0
    # one request per flush: its token history is one op of T words
    sizes = [[T] for T in range(2044, 2053)]
    # several requests per flush: ops of 800 words, logs of about 60-75 KiB
    sizes += [[800] * k for k in range(17, 22)]
    for g in sizes:
        reqs = []
        for T in g:
            q = int(rng.integers(1, 9))
            nb = -(-T // B)
            blocks = pool[used:used + nb]
            used += nb
            tokens = rng.integers(0, 1 << 20, size=T).astype(np.int32)
            reqs.append(workloads.Req(rid, tokens, T, T - q, q, blocks,
                                      temperature=float(rng.uniform(0.1, 2.0)), top_p=0.9,
                                      rep_penalty=1.1, top_k=int(rng.integers(0, 50))))
            rid += 1
        groups.append(reqs)
    w = _workload(groups, B, 2176, 16384)
    b = runner.Batch(runner.config_of(w))
    for g in groups:
        for r in g:
            b.add(r)
        ric.ric_flush(b.h)
    torch.cuda.synchronize()
    ref, order = replay_history(w)
    assert b.row_order() == order
    cols = ric.ric_get_columns(b.h)
    R = len(order)
    T_dev = b.device_i32(cols.num_tokens, R)
    NB_dev = b.device_i32(cols.num_blocks, R)
    K_dev = b.device_i32(cols.top_k, R)
    temp = b.device_u8(cols.temperature, 4 * R).view(np.float32)
    for i in range(R):
        r = ref.rows[i]
        assert (T_dev[i], NB_dev[i], K_dev[i]) == (len(r.tokens), len(r.blocks), r.sampling[3]), f"row {i}"
        assert temp[i] == np.float32(r.sampling[0]), f"row {i} temperature"
        toks = read_rows_i32(b.workspace, cols.tokens, cols.token_stride, [i], len(r.tokens))[0]
        assert np.array_equal(toks, np.asarray(r.tokens, np.int32)), f"token row {i} ({len(r.tokens)} tokens)"
        blks = read_rows_i32(b.workspace, cols.blocks, cols.block_stride, [i], len(r.blocks))[0]
        assert np.array_equal(blks, np.asarray(r.blocks, np.int32)), f"block row {i}"
    b.schedule_from(w, order)
    exp = expected_step(w, ref)
    s = b.compile(exp["n_pad"])
    assert_step_equal(b.step_outputs(s), exp, "after the uploads")
    b.close()
