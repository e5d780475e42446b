"""The oracle against values the pages print (tests/golden) and closed forms.

Every fixture is checked against all three oracle formulations (per-token
Python, numpy library routines, plain C block-range loop)."""
import numpy as np
import pytest

from oracle import batch, cbind, step
from tests.oracle_helpers import golden, labelled_rows, run_all, Row


def _check(results, key, expect, n=None):
    for name, res in zip(("python", "numpy", "c"), results):
        got = res[key] if n is None else res[key][:n]
        assert list(got) == list(expect), f"{name} {key}: {list(got)} != {expect}"


def test_scan_2_5_3():
    g = golden("scan_2_5_3.json")
    q = g["num_scheduled"]
    rows = labelled_rows([0, 0, 0], q, q, block_size=16)
    res = run_all(rows, block_size=16)
    e = g["expect"]
    _check(res, "query_start_loc", e["query_start_loc"])
    _check(res, "req_indices", e["req_indices"])
    _check(res, "logits_indices", e["logits_indices"])
    # with c = 0 the position is the in-request offset
    _check(res, "positions", e["query_pos"])
    qsl = np.asarray(res[0]["query_start_loc"])
    assert list(qsl[1:]) == e["cu_num_tokens"]
    assert list(qsl[res[0]["req_indices"]]) == e["cumsums_offsets"]


def test_p1_worked_example():
    g = golden("p1_worked_example.json")
    rows = labelled_rows(g["num_computed"], g["num_scheduled"], g["num_prompt"],
                         g["block_size"], blocks=g["blocks"])
    res = run_all(rows, block_size=g["block_size"])
    e = g["expect"]
    for k in ("req_indices", "query_start_loc", "input_ids", "positions", "seq_lens",
              "slot_mapping", "logits_indices"):
        _check(res, k, e[k])
    qsl = res[0]["query_start_loc"]
    qpos = np.arange(6) - qsl[res[0]["req_indices"]]
    assert list(qpos) == e["query_pos"]
    # visible key length of each query = its position + 1 (causal within the request)
    assert list(res[0]["positions"] + 1) == e["visible_key_lengths"]
    for r in res:
        assert r["discard"][1] == e["discard_B"]


def test_p1_min_repro():
    g = golden("p1_min_repro.json")
    rows = labelled_rows(g["num_computed"], g["num_scheduled"], g["num_prompt"], 16)
    res = run_all(rows, block_size=16)
    for k, v in g["expect"].items():
        _check(res, k, v)


@pytest.mark.parametrize("name", ["p3_layout.json", "p3_verify_step2.json"])
def test_p3_examples(name):
    g = golden(name)
    rows = labelled_rows(g["num_computed"], g["num_scheduled"], g["num_prompt"], 16)
    res = run_all(rows, block_size=16)
    e = dict(g["expect"])
    n = e.pop("num_actual_tokens", None)
    if n is not None:
        assert res[0]["num_actual_tokens"] == n
    for k, v in e.items():
        _check(res, k, v)


def test_p3_exercise_compacted_logits():
    g = golden("p3_exercise1.json")
    rows = labelled_rows(g["num_computed"], g["num_scheduled"], g["num_prompt"], 16)
    res = run_all(rows, block_size=16)
    e = g["expect"]
    _check(res, "query_start_loc", e["query_start_loc"])
    _check(res, "seq_lens", e["seq_lens"])
    _check(res, "positions", e["positions"])
    for r in res:
        assert r["num_sampled"] == len(e["sample_indices"])
        assert list(r["sample_indices"][:r["num_sampled"]]) == e["sample_indices"]


def test_p5_slot_ranges():
    g = golden("p5_slot_ranges.json")
    B, start, end = g["block_size"], g["start"], g["end"]
    rows = [Row(start, end - start, end, np.arange(end, dtype=np.int64),
                np.asarray(g["blocks"], np.int64))]
    res = run_all(rows, block_size=B)
    expect = [s for a, b in g["expect"]["ranges"] for s in range(a, b)]
    assert len(expect) == g["expect"]["count"]
    _check(res, "slot_mapping", expect)


def test_p5_flatten_and_cu_seqlens_k():
    g = golden("p5_flatten.json")
    f = g["first"]
    rows = labelled_rows(f["num_computed"], f["num_scheduled"], f["num_scheduled"], 16)
    res = run_all(rows, block_size=16)
    _check(res, "positions", f["expect"]["positions"])
    _check(res, "query_start_loc", f["expect"]["cu_seqlens_q"])
    _check(res, "cu_seqlens_k", f["expect"]["cu_seqlens_k"])
    s = g["second"]
    rows = labelled_rows(s["num_computed"], s["num_scheduled"], [8], 16)
    res = run_all(rows, block_size=16)
    assert res[0]["seq_lens"][0] == s["expect"]["seqlen_k"]
    _check(res, "cu_seqlens_k", s["expect"]["cu_seqlens_k"])


def test_p1_condense():
    g = golden("p1_condense.json")
    b = batch.RefBatch(max_num_reqs=4, max_model_len=8, max_blocks_per_req=2, num_kv_blocks=16)
    ids = {name: k for k, name in enumerate(g["rows"])}
    for name in g["rows"]:
        b.add_request(ids[name], [1, 2], 2, 0, [ids[name] + 1])
    for name in g["remove"]:
        b.remove_request(ids[name])
    b.condense()
    names = {v: k for k, v in ids.items()}
    got = [names[r] for r in b.req_ids_by_row() if r is not None]
    assert got == g["expect"]["rows"]
    assert b.num_used_rows() == len(got)


def test_p2_logits_closed_form():
    g = golden("p2_logits.json")
    qsl = g["query_start_loc"]
    q = [qsl[i + 1] - qsl[i] for i in range(len(qsl) - 1)]
    rows = labelled_rows([0] * len(q), q, q, 16)
    res = run_all(rows, block_size=16)
    _check(res, "query_start_loc", qsl)
    _check(res, "logits_indices", g["expect"]["logits_indices"])


def test_p2_padding():
    g = golden("p2_padding.json")
    for n, padded, waste in g["cases"]:
        got = step.padded_size(g["capture_sizes"], n)
        assert got == padded
        assert round(100 * (1 - n / got)) == waste
    # above the largest captured size the step is not padded
    assert step.padded_size(g["capture_sizes"], 257) == 257


def test_p3_padding_waste():
    g = golden("p3_padding_waste.json")
    q = g["num_scheduled"]
    rows = labelled_rows([0] * len(q), q, q, 16)
    res = run_all(rows, block_size=16)
    e = g["expect"]
    flat = res[0]["num_actual_tokens"]
    rect = len(q) * res[0]["max_query_len"]
    assert (flat, rect) == (e["flat_tokens"], e["rectangular_tokens"])
    assert round(100 * (1 - flat / rect)) == e["waste_percent_rounded"]


def test_nano_decode_identity():
    """A decode's slot is the last block's base plus (tokens in that block) - 1,
    its position len-1 and its context length len (the decode path of the
    nano-vllm runner, prepare_decode)."""
    rng = np.random.default_rng(7)
    for B in (1, 2, 3, 4, 8, 16):
        for T in range(1, 40):
            nb = -(-T // B)
            blocks = rng.permutation(np.arange(1, 100))[:nb]
            rows = [Row(T - 1, 1, T, np.arange(T, dtype=np.int64), blocks)]
            res = run_all(rows, block_size=B)
            last_block_num_tokens = T - (nb - 1) * B
            expect_slot = int(blocks[-1]) * B + last_block_num_tokens - 1
            _check(res, "slot_mapping", [expect_slot])
            _check(res, "positions", [T - 1])
            _check(res, "seq_lens", [T])


def test_padding_tail_reading():
    """Pad tokens and pseudo-requests take the values this oracle defines."""
    rows = labelled_rows([5, 0], [1, 2], [6, 2], 4)
    res = run_all(rows, block_size=4, max_num_reqs=4, n_pad=8, null_block=0)
    for r in res:
        assert list(r["input_ids"][3:]) == [0] * 5
        assert list(r["positions"][3:]) == [0] * 5
        assert list(r["req_indices"][3:]) == [-1] * 5
        assert list(r["slot_mapping"][3:]) == [0] * 5
        assert list(r["query_start_loc"]) == [0, 1, 3, 3, 3]
        assert list(r["seq_lens"]) == [6, 2, 0, 0]
        assert list(r["logits_indices"]) == [0, 2, -1, -1]
        assert list(r["discard"]) == [0, 0, 1, 1]
        assert list(r["sample_indices"]) == [0, 2, -1, -1]


def test_step_rejects_bad_input():
    ok = dict(block_size=4, max_num_reqs=2, max_model_len=16, max_num_batched_tokens=8,
              num_kv_blocks=10, n_pad=4)
    good = labelled_rows([0], [2], [2], 4)
    step.compile_step(good, **ok)
    with pytest.raises(step.StepError):           # nothing scheduled
        step.compile_step([Row(0, 0, 1, np.arange(2), np.array([1]))], **ok)
    with pytest.raises(step.StepError):           # past the token history
        step.compile_step([Row(1, 2, 2, np.arange(2), np.array([1]))], **ok)
    with pytest.raises(step.StepError):           # too few blocks
        step.compile_step([Row(0, 5, 5, np.arange(5), np.array([1]))], **ok)
    with pytest.raises(step.StepError):           # null block owned
        step.compile_step([Row(0, 2, 2, np.arange(2), np.array([0]))], **ok)
    with pytest.raises(step.StepError):           # shared block -> duplicate slots
        step.compile_step([Row(0, 2, 2, np.arange(2), np.array([1])),
                           Row(0, 2, 2, np.arange(2), np.array([1]))], **ok)
    with pytest.raises(step.StepError):           # padded size below N
        step.compile_step(good, **{**ok, "n_pad": 1})
    with pytest.raises(step.StepError):           # padded size above budget
        step.compile_step(good, **{**ok, "n_pad": 9})
    with pytest.raises(ValueError):
        cbind.compile_step(good, block_size=4, max_num_reqs=2, n_pad=1)
