"""Brute force, invariants and metamorphic relations for the oracle.

The three formulations must agree on every tiny batch, and each output must
satisfy the invariants the first page lists (section 八条必须成立的不变量),
checked here with constructions that avoid the oracle's own formulas (list
slicing of the token history, explicit expansion of a block list into its
slots)."""
import itertools

import numpy as np
import pytest

import workloads
from tests.oracle_helpers import KEYS, Row, labelled_rows, rows_of, run_all


def _owned_slots(blocks, B):
    """Every slot the request owns, in logical order: block k contributes
    k*B..k*B+B-1 of the sequence."""
    out = []
    for b in blocks:
        out.extend(int(b) * B + o for o in range(B))
    return out


def check_invariants(rows, res, B, n_pad, max_num_reqs, null_block=0):
    R = len(rows)
    q = [r.num_scheduled for r in rows]
    N = sum(q)
    qsl = list(res["query_start_loc"])
    assert qsl[0] == 0 and all(qsl[i] <= qsl[i + 1] for i in range(max_num_reqs))
    assert qsl[R] == N and all(x == N for x in qsl[R:])
    for i, r in enumerate(rows):
        a, b = qsl[i], qsl[i + 1]
        assert b - a == r.num_scheduled
        seg = slice(a, b)
        assert all(x == i for x in res["req_indices"][seg])
        assert list(res["positions"][seg]) == list(range(r.num_computed, r.num_computed + r.num_scheduled))
        assert list(res["input_ids"][seg]) == list(r.tokens[r.num_computed:r.num_computed + r.num_scheduled])
        owned = _owned_slots(r.blocks, B)
        assert list(res["slot_mapping"][seg]) == owned[r.num_computed:r.num_computed + r.num_scheduled]
        assert res["seq_lens"][i] == r.num_computed + r.num_scheduled
        assert res["seq_lens"][i] <= len(r.blocks) * B
        li = res["logits_indices"][i]
        assert res["req_indices"][li] == i and (li + 1 == N or res["req_indices"][li + 1] != i)
        assert res["discard"][i] == (1 if r.num_computed + r.num_scheduled < r.num_prompt else 0)
    keep = [res["logits_indices"][i] for i in range(R) if res["discard"][i] == 0]
    assert res["num_sampled"] == len(keep)
    assert list(res["sample_indices"][:len(keep)]) == keep
    real = list(res["slot_mapping"][:N])
    assert len(set(real)) == N
    assert all(s // B != null_block for s in real)
    assert list(res["slot_mapping"][N:n_pad]) == [null_block * B] * (n_pad - N)
    assert list(res["req_indices"][N:n_pad]) == [-1] * (n_pad - N)


def _agree(results):
    base = results[0]
    for name, other in zip(("numpy", "c"), results[1:]):
        for k in KEYS:
            assert np.array_equal(base[k], other[k]), f"{name} disagrees on {k}"
        assert base["num_sampled"] == other["num_sampled"]
    assert results[0]["max_query_len"] == results[2]["max_query_len"]
    assert results[0]["max_seq_len"] == results[2]["max_seq_len"]


def _prompt(mode, c, q):
    return {"short": max(1, c + q - 1), "exact": c + q, "long": c + q + 1}[mode]


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_bruteforce_single_request(B):
    rng = np.random.default_rng(100 + B)
    for q, c, mode in itertools.product(range(1, 5), range(0, 7), ("short", "exact", "long")):
        for _ in range(3):
            P = _prompt(mode, c, q)
            nb = -(-(c + q) // B)
            blocks = rng.permutation(np.arange(1, 40))[:nb]
            rows = [Row(c, q, P, np.arange(100, 100 + max(P, c + q)), blocks)]
            n_pad = q + int(rng.integers(0, 3))
            res = run_all(rows, block_size=B, max_num_reqs=2, n_pad=n_pad)
            _agree(res)
            check_invariants(rows, res[0], B, n_pad, 2)


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_bruteforce_pairs(B):
    """Every (q, c) combination for two requests, random prompts and block
    permutations."""
    rng = np.random.default_rng(200 + B)
    grid = list(itertools.product(range(1, 5), range(0, 7)))
    for (q0, c0), (q1, c1) in itertools.product(grid, grid):
        modes = [("short", "exact", "long")[int(rng.integers(0, 3))] for _ in range(2)]
        P = [_prompt(modes[0], c0, q0), _prompt(modes[1], c1, q1)]
        perm = rng.permutation(np.arange(1, 60))
        n0 = -(-(c0 + q0) // B)
        n1 = -(-(c1 + q1) // B)
        rows = [Row(c0, q0, P[0], np.arange(max(P[0], c0 + q0)) + 10, perm[:n0]),
                Row(c1, q1, P[1], np.arange(max(P[1], c1 + q1)) + 500, perm[n0:n0 + n1])]
        n_pad = q0 + q1 + int(rng.integers(0, 4))
        res = run_all(rows, block_size=B, max_num_reqs=4, n_pad=n_pad)
        _agree(res)
        check_invariants(rows, res[0], B, n_pad, 4)


def test_bruteforce_three_requests_random():
    rng = np.random.default_rng(300)
    for trial in range(600):
        B = int(rng.integers(1, 5))
        reqs = workloads.random_batch(rng, num_reqs=3, block_size=B, max_model_len=64,
                                      num_kv_blocks=80, max_q=4, max_c=6)
        rows = rows_of(reqs)
        n_pad = sum(r.num_scheduled for r in rows) + int(rng.integers(0, 5))
        res = run_all(rows, block_size=B, max_num_reqs=3 + int(rng.integers(0, 3)), n_pad=n_pad)
        _agree(res)
        check_invariants(rows, res[0], B, n_pad, len(res[0]["seq_lens"]))


def test_concatenation_invariance():
    """Each request's segment of a batch equals compiling that request alone,
    shifted by its query_start_loc (the mixed batch computes what separate
    runs compute; third page, section 验证：一次混合前向)."""
    rng = np.random.default_rng(400)
    for trial in range(50):
        B = int(rng.choice([1, 3, 4, 16]))
        rows = rows_of(workloads.random_batch(rng, num_reqs=int(rng.integers(1, 6)), block_size=B,
                                              max_model_len=200, num_kv_blocks=400, max_q=20, max_c=60))
        whole = run_all(rows, block_size=B)[0]
        qsl = whole["query_start_loc"]
        for i, r in enumerate(rows):
            alone = run_all([r], block_size=B)[0]
            seg = slice(qsl[i], qsl[i + 1])
            for k in ("input_ids", "positions", "slot_mapping"):
                assert np.array_equal(whole[k][seg], alone[k])
            assert whole["logits_indices"][i] == qsl[i] + alone["logits_indices"][0]
            assert whole["seq_lens"][i] == alone["seq_lens"][0]
            assert whole["discard"][i] == alone["discard"][0]


def test_phase_invariance_chunked_prefill():
    """A prompt computed in one step and the same prompt computed in chunks
    produce the same per-token stream (prefill, chunk and decode differ only
    in their (cached, new) lengths; third page, section 布局与元数据)."""
    rng = np.random.default_rng(500)
    for trial in range(40):
        B = int(rng.choice([1, 2, 4, 16]))
        P = int(rng.integers(1, 90))
        tokens = rng.integers(0, 1000, size=P)
        blocks = rng.permutation(np.arange(1, 200))[:-(-P // B)]
        one = run_all([Row(0, P, P, tokens, blocks)], block_size=B)[0]
        cuts = sorted(set(int(x) for x in rng.integers(1, P, size=int(rng.integers(0, 4))))) if P > 1 else []
        bounds = [0] + cuts + [P]
        chunks = {k: [] for k in ("input_ids", "positions", "slot_mapping")}
        for a, b in zip(bounds[:-1], bounds[1:]):
            res = run_all([Row(a, b - a, P, tokens, blocks)], block_size=B)[0]
            for k in chunks:
                chunks[k].extend(res[k].tolist())
            assert res["discard"][0] == (1 if b < P else 0)
        for k in chunks:
            assert chunks[k] == one[k].tolist()


def test_row_permutation_equivariance():
    rng = np.random.default_rng(600)
    for trial in range(30):
        B = 4
        rows = rows_of(workloads.random_batch(rng, num_reqs=5, block_size=B, max_model_len=100,
                                              num_kv_blocks=300, max_q=8, max_c=30))
        perm = rng.permutation(5)
        a = run_all(rows, block_size=B)[0]
        b = run_all([rows[k] for k in perm], block_size=B)[0]
        for new_i, old_i in enumerate(perm):
            sa = slice(a["query_start_loc"][old_i], a["query_start_loc"][old_i + 1])
            sb = slice(b["query_start_loc"][new_i], b["query_start_loc"][new_i + 1])
            for k in ("input_ids", "positions", "slot_mapping"):
                assert np.array_equal(a[k][sa], b[k][sb])


@pytest.mark.parametrize("name", ["worked_example", "decode_heavy", "mixed", "long_context",
                                  "long_context_forced"])
def test_configs_formulations_agree(name):
    w = workloads.get(name)
    rows = rows_of(w.live_requests())
    from oracle import step
    n_pad = step.padded_size(w.capture_sizes, sum(r.num_scheduled for r in rows))
    res = run_all(rows, block_size=w.block_size, max_num_reqs=w.max_num_reqs, n_pad=n_pad,
                  max_model_len=w.max_model_len, num_kv_blocks=w.num_kv_blocks)
    _agree(res)
    check_invariants(rows, res[0], w.block_size, n_pad, w.max_num_reqs)


def test_worked_example_config_values():
    """The worked-example configuration reproduces the third page's printed
    query_start_loc, seq_lens and logits indices, padded to 32."""
    w = workloads.get("worked_example")
    rows = rows_of(w.live_requests())
    from oracle import step
    n_pad = step.padded_size(w.capture_sizes, 20)
    assert n_pad == 32
    res = run_all(rows, block_size=16, max_num_reqs=4, n_pad=n_pad)[0]
    assert list(res["query_start_loc"][:4]) == [0, 7, 8, 20]
    assert list(res["seq_lens"][:3]) == [7, 6, 22]
    assert list(res["logits_indices"][:3]) == [6, 7, 19]
