"""Persistent-batch oracle (add / remove / append / replace / condense) and the
K/V-write and gather oracles."""
import numpy as np
import pytest

import workloads
from oracle import batch, cbind, step, vectorised
from tests.oracle_helpers import golden, labelled_rows, rows_of, run_all


def _mk(max_reqs=8):
    return batch.RefBatch(max_num_reqs=max_reqs, max_model_len=64, max_blocks_per_req=8,
                          num_kv_blocks=100)


def test_condense_several_holes():
    b = _mk()
    for k in range(6):
        b.add_request(k, [k] * 3, 3, 0, [k + 1])
    for k in (1, 2):
        b.remove_request(k)
    pairs = b.condense()
    assert pairs == [(1, 5), (2, 4)]
    assert b.req_ids_by_row()[:4] == [0, 5, 4, 3]
    # maps are inverses (first invariant of the first page)
    for row, rid in enumerate(b.req_ids_by_row()):
        if rid is not None:
            assert b.row_of[rid] == row
    # every column moved with its row
    assert b.rows[1].tokens == [5] * 3 and b.rows[1].blocks == [6]


def test_condense_no_move_when_holes_at_tail():
    b = _mk()
    for k in range(4):
        b.add_request(k, [k], 1, 0, [k + 1])
    b.remove_request(3)
    b.remove_request(2)
    assert b.condense() == []
    assert b.num_used_rows() == 2


def test_condense_hole_below_every_row():
    b = _mk()
    for k in range(5):
        b.add_request(k, [k], 1, 0, [k + 1])
    for k in (0, 1, 2, 3):
        b.remove_request(k)
    assert b.condense() == [(0, 4)]
    assert b.req_ids_by_row()[:1] == [4] and b.num_used_rows() == 1


def test_add_takes_lowest_free_row_and_abort_resubmit():
    b = _mk()
    for k in range(3):
        b.add_request(k, [1, 2], 2, 0, [k + 1])
    with pytest.raises(batch.BatchError):
        b.add_request(1, [9], 1, 0, [9])           # id still live
    b.remove_request(1)                              # abort ...
    row = b.add_request(1, [7, 7, 7], 3, 1, [20])   # ... and resubmit: a new request
    assert row == 1 and b.rows[1].tokens == [7, 7, 7] and b.rows[1].num_computed == 1


def test_preempt_resume_replaces_blocks():
    b = _mk()
    b.add_request(0, list(range(10)), 10, 0, [1, 2])
    b.append_blocks(0, [3])
    assert b.rows[0].blocks == [1, 2, 3]
    b.replace_blocks(0, [7, 8])
    assert b.rows[0].blocks == [7, 8]
    with pytest.raises(batch.BatchError):
        b.append_blocks(0, [0])                      # the null block is never owned


def test_schedule_requires_condensed_rows():
    b = _mk()
    for k in range(3):
        b.add_request(k, [1, 2], 2, 0, [k + 1])
    b.remove_request(0)
    with pytest.raises(batch.BatchError):
        b.schedule([0, 0], [1, 1])
    b.condense()
    b.schedule([0, 0], [1, 1])


def test_churn_history():
    """The churn configuration: 1024 rows, 102 finish, condense, 102 refills.
    After the history the rows are exactly [0, 1024) and every moved row
    carries its own columns."""
    w = workloads.get("churn")
    b = batch.RefBatch(w.max_num_reqs, w.max_model_len, w.max_blocks_per_req, w.num_kv_blocks)
    for r in w.initial:
        b.add_request(r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks)
    for rid in w.finished:
        b.remove_request(rid)
    pairs = b.condense()
    assert len(pairs) <= len(w.finished)
    assert b.num_used_rows() == b.num_live() == w.max_num_reqs - len(w.finished)
    for r in w.refill:
        b.add_request(r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks)
    assert b.num_used_rows() == w.max_num_reqs
    by_id = w.by_id()
    for row, rid in enumerate(b.req_ids_by_row()):
        assert b.rows[row].tokens[:5] == [int(t) for t in by_id[rid].tokens[:5]]
        assert b.rows[row].blocks == [int(x) for x in by_id[rid].blocks]
    order = b.req_ids_by_row()
    b.schedule([by_id[r].num_computed for r in order], [by_id[r].num_scheduled for r in order])
    rows = b.step_rows()
    assert sum(r.num_scheduled for r in rows) == 16384
    res = run_all(rows, block_size=w.block_size, max_num_reqs=w.max_num_reqs, n_pad=16384,
                  max_model_len=w.max_model_len, num_kv_blocks=w.num_kv_blocks)
    for other in res[1:]:
        for k in ("input_ids", "slot_mapping", "positions", "query_start_loc"):
            assert np.array_equal(res[0][k], other[k])


def _kv_case(rng, n_tokens, n_slots, row_bytes):
    k = rng.integers(0, 256, size=(n_tokens, row_bytes), dtype=np.uint8)
    v = rng.integers(0, 256, size=(n_tokens, row_bytes), dtype=np.uint8)
    return k, v


def test_kv_write_worked_example():
    """First page worked example: six new K/V rows land in slots
    9, 20, 21, 22, 16, 17 (block size 4)."""
    g = golden("p1_worked_example.json")
    rows = labelled_rows(g["num_computed"], g["num_scheduled"], g["num_prompt"], 4, blocks=g["blocks"])
    slots = run_all(rows, block_size=4)[0]["slot_mapping"]
    rng = np.random.default_rng(1)
    k, v = _kv_case(rng, 6, 40, 8)
    kc = np.zeros((40, 8), np.uint8)
    vc = np.zeros((40, 8), np.uint8)
    step.reshape_and_cache(k, v, kc, vc, slots)
    for t, s in enumerate(g["expect"]["slot_mapping"]):
        assert np.array_equal(kc[s], k[t]) and np.array_equal(vc[s], v[t])
    untouched = [s for s in range(40) if s not in g["expect"]["slot_mapping"]]
    assert not kc[untouched].any() and not vc[untouched].any()


def test_kv_write_three_ways_agree():
    rng = np.random.default_rng(2)
    for trial in range(20):
        B = int(rng.choice([1, 4, 16]))
        rows = rows_of(workloads.random_batch(rng, num_reqs=4, block_size=B, max_model_len=200,
                                              num_kv_blocks=256, max_q=12, max_c=40))
        N = sum(r.num_scheduled for r in rows)
        n_pad = N + int(rng.integers(0, 5))
        slots = run_all(rows, block_size=B, n_pad=n_pad)[0]["slot_mapping"]
        nslots = 256 * B
        k, v = _kv_case(rng, n_pad, nslots, 32)
        caches = []
        for fn in ("loop", "numpy", "c"):
            kc = np.full((nslots, 32), 0xA5, np.uint8)
            vc = np.full((nslots, 32), 0x5A, np.uint8)
            if fn == "loop":
                step.reshape_and_cache(k, v, kc, vc, slots)
            elif fn == "numpy":
                vectorised.reshape_and_cache(k, v, kc, vc, slots)
            else:
                cbind.kv_scatter(k, v, kc, vc, slots, 32)
            caches.append((kc, vc))
        real = slots[:N]
        for kc, vc in caches:
            assert np.array_equal(kc[real], k[:N]) and np.array_equal(vc[real], v[:N])
            others = np.setdiff1d(np.arange(B, nslots), real)   # null block excluded
            assert (kc[others] == 0xA5).all() and (vc[others] == 0x5A).all()
        for kc, vc in caches[1:]:
            assert np.array_equal(np.delete(kc, np.arange(B), 0), np.delete(caches[0][0], np.arange(B), 0))


def test_padded_block_table_definition():
    """nano-vllm pads each request's block list with -1 to the longest one
    (prepare_block_tables); width may also cut a row."""
    from tests.oracle_helpers import Row
    rows = [Row(0, 1, 1, np.arange(3), np.array([4, 5, 9])), Row(0, 1, 1, np.arange(3), np.array([7])),
            Row(0, 1, 1, np.arange(3), np.array([], np.int64))]
    assert step.padded_block_table(rows, 3) == [[4, 5, 9], [7, -1, -1], [-1, -1, -1]]
    assert step.padded_block_table(rows, 2, fill=0) == [[4, 5], [7, 0], [0, 0]]


def test_append_sampled_then_decode():
    """Appending last step's sampled ids through a row -> sample-position map
    and then compiling one decode token per row feeds exactly those ids."""
    b = _mk()
    for k in range(5):
        b.add_request(k, [100 + k] * (k + 2), k + 2, k + 2, [k + 1])
    sampled = [900, 901, 902, 903, 904]
    src = [4, 2, 0, 1, 3]                  # the batch was reordered since sampling
    toks = {i: b.rows[i].tokens for i in range(5)}
    step.append_sampled(toks, list(range(5)), src, sampled)
    T = [len(b.rows[i].tokens) for i in range(5)]
    b.schedule([t - 1 for t in T], [1] * 5)
    out = step.compile_step(b.step_rows(), block_size=16, max_num_reqs=8, max_model_len=64,
                            max_num_batched_tokens=8, num_kv_blocks=100, n_pad=5)
    assert out["input_ids"] == [sampled[j] for j in src]
    assert out["positions"] == [t - 1 for t in T]


def test_kernel_block_expansion_pin():
    g = golden("p1_kernel_blocks.json")
    ratio = g["manager_block_size"] // g["kernel_block_size"]
    assert step.expand_kernel_blocks(g["manager_ids"], ratio) == g["expect"]["kernel_ids"]


def test_kernel_blocks_give_the_same_slots():
    """Slots through manager blocks of size k*Bk equal slots through the
    expanded kernel blocks of size Bk, for every position: the expansion
    changes the table an attention kernel reads, not where K/V lands."""
    rng = np.random.default_rng(51)
    for trial in range(200):
        Bk = int(rng.integers(1, 9))
        k = int(rng.integers(1, 5))
        ids = rng.permutation(np.arange(1, 64))[:int(rng.integers(1, 8))]
        kern = step.expand_kernel_blocks(ids, k)
        for p in range(len(ids) * k * Bk):
            via_manager = int(ids[p // (k * Bk)]) * (k * Bk) + p % (k * Bk)
            via_kernel = kern[p // Bk] * Bk + p % Bk
            assert via_manager == via_kernel


def test_group_slot_mapping_matches_compile_for_one_group():
    """With a single group, the per-group slot routine reproduces the
    compile's slot_mapping, padding included."""
    rng = np.random.default_rng(52)
    for trial in range(50):
        B = int(rng.integers(1, 9))
        rows = rows_of(workloads.random_batch(rng, num_reqs=4, block_size=B, max_model_len=200,
                                              num_kv_blocks=400, max_q=9, max_c=40))
        n_pad = sum(r.num_scheduled for r in rows) + 3
        out = step.compile_step(rows, block_size=B, max_num_reqs=4, max_model_len=200, max_num_batched_tokens=n_pad,
                                num_kv_blocks=400, n_pad=n_pad)
        got = step.group_slot_mapping(out["positions"], out["req_indices"], [r.blocks for r in rows], B)
        assert got == out["slot_mapping"]


def test_spec_decode_reduces_to_plain_logits_without_drafts():
    """No drafts: one logits row per request, at query_start_loc[1:] - 1 (the
    closed form the second page prints for [0,2,9,12] -> [1,8,11])."""
    g = golden("p2_logits.json")
    qsl = g["query_start_loc"]
    m = step.spec_decode_metadata(qsl, list(range(qsl[-1])), [0, 0, 0])
    assert m["logits_indices"] == g["expect"]["logits_indices"]
    assert m["bonus_logits_indices"] == [0, 1, 2] and m["target_logits_indices"] == []
    assert m["cu_num_logits"] == [0, 1, 2, 3]


def test_spec_decode_invariants_bruteforce():
    """Every logits position lies inside its request and the request's last
    position is always among them; a request's d drafts are its last d input
    ids, checked by the rows right before its bonus row."""
    rng = np.random.default_rng(31)
    for trial in range(300):
        R = int(rng.integers(1, 6))
        q = rng.integers(1, 7, R)
        d = [int(rng.integers(0, qi)) for qi in q]          # d + 1 <= q
        qsl = [0] + list(np.cumsum(q))
        ids = rng.integers(0, 1000, qsl[-1])
        m = step.spec_decode_metadata(qsl, ids, d)
        assert len(m["logits_indices"]) == sum(d) + R and len(m["draft_token_ids"]) == sum(d)
        pos = 0
        for i in range(R):
            rows = m["logits_indices"][m["cu_num_logits"][i]:m["cu_num_logits"][i + 1]]
            assert rows == list(range(qsl[i + 1] - d[i] - 1, qsl[i + 1]))
            assert m["bonus_logits_indices"][i] == m["cu_num_logits"][i + 1] - 1
            assert m["logits_indices"][m["bonus_logits_indices"][i]] == qsl[i + 1] - 1
            for k in range(d[i]):
                t = m["target_logits_indices"][pos + k]
                # the target row for draft k sits at the flat position right before that draft
                assert m["logits_indices"][t] + 1 == qsl[i + 1] - d[i] + k
                assert m["draft_token_ids"][pos + k] == ids[qsl[i + 1] - d[i] + k]
            pos += d[i]


def test_gather_three_ways_agree():
    rng = np.random.default_rng(3)
    src = rng.integers(0, 256, size=(50, 24), dtype=np.uint8)
    idx = np.array([3, 0, 49, -1, 7], np.int64)
    a = np.stack(step.gather_rows(list(src), idx, 5, np.zeros(24, np.uint8)))
    b = vectorised.gather_rows(src, idx, 5)
    c = np.zeros((5, 24), np.uint8)
    cbind.gather(src, 24, idx, 5, c)
    assert np.array_equal(a, b) and np.array_equal(a, c)
    assert np.array_equal(a[0], src[3]) and not a[3].any()
