"""Planted mistakes in the oracle routines beyond the compile (K/V write, row
gather, condense, kernel-block expansion, padded tables, per-group slots,
sampled-token append, the correction of optimistic computed counts,
speculative-decoding indices): each mutant copy must fail a pin that holds
for the unmutated oracle.  The pins are values the pages
print (golden files), library special cases and invariants written here
independently of the oracle's code.  Mutations are planted in copies, on the
CPU."""
import sys
import types

import numpy as np
import pytest

import oracle.batch as batch_mod
import oracle.step as step_mod
from tests.oracle_helpers import Row, golden


def _check(cond, what):
    if not cond:
        raise AssertionError(what)


def _pins_step(step):
    """Pins of the step-level routines; ``step`` is the module under test."""
    rng = np.random.default_rng(7)

    # K/V write: [P1] worked example slots (B=4), every row lands whole at its
    # slot, K and V stay apart, untouched rows keep their sentinel.
    slots = golden("p1_worked_example.json")["expect"]["slot_mapping"]
    k = [bytes([t, 0xAA]) for t in range(len(slots))]
    v = [bytes([t, 0xBB]) for t in range(len(slots))]
    kc, vc = [b"--"] * 32, [b"--"] * 32
    step.reshape_and_cache(k, v, kc, vc, slots)
    for t, s in enumerate(slots):
        _check(kc[s] == k[t] and vc[s] == v[t], "kv row at its slot")
    _check(all(kc[i] == b"--" for i in range(32) if i not in slots), "kv untouched rows")

    # Row gather: equals numpy fancy indexing for valid rows, zero row for -1.
    src = rng.integers(0, 256, (9, 4), dtype=np.uint8)
    idx = [8, 0, -1, 3]
    got = step.gather_rows(list(src), idx, 3, np.zeros(4, np.uint8))
    _check(len(got) == 3, "gather count")
    _check(np.array_equal(np.stack(got[:2]), src[[8, 0]]), "gather rows")
    _check(not np.any(got[2]), "gather zero row")

    # Manager -> kernel block expansion, printed example.
    g = golden("p1_kernel_blocks.json")
    ratio = g["manager_block_size"] // g["kernel_block_size"]
    _check(step.expand_kernel_blocks(g["manager_ids"], ratio) == g["expect"]["kernel_ids"], "expansion")
    _check(step.expand_kernel_blocks([3, 7], 2) == [6, 7, 14, 15], "expansion 2")

    # Padded table: nano pads each block list with -1 to the longest one.
    rows = [Row(0, 1, 1, np.arange(3), np.array([4, 5, 9])), Row(0, 1, 1, np.arange(3), np.array([7])),
            Row(0, 1, 1, np.arange(3), np.array([], np.int64))]
    _check(step.padded_block_table(rows, 3) == [[4, 5, 9], [7, -1, -1], [-1, -1, -1]], "padded table")
    _check(step.padded_block_table(rows, 4, fill=0, ratio=2) ==
           [[8, 9, 10, 11], [14, 15, 0, 0], [0, 0, 0, 0]], "padded table expanded")

    # Per-group slots: the [P5 Q&A 14] hand-worked ranges (B=8, table
    # [4,5,9,3,11], positions 1..37), plus a padded token at the null slot.
    g = golden("p5_slot_ranges.json")
    pos = list(range(g["start"], g["end"])) + [0]
    req = [0] * (len(pos) - 1) + [-1]
    want = [s for a, b in g["expect"]["ranges"] for s in range(a, b)] + [0]
    _check(step.group_slot_mapping(pos, req, [g["blocks"]], g["block_size"]) == want, "group slots")
    _check(step.group_slot_mapping([5], [-1], [[1]], 4, null_block=2) == [8], "group null slot")

    # Sampled-token append through a row -> sample-position map.
    toks = {0: [1, 2], 1: [3], 2: [4, 5, 6]}
    step.append_sampled(toks, [2, 0, 1], [1, 2, 0], [70, 71, 72])
    _check(toks == {0: [1, 2, 72], 1: [3, 70], 2: [4, 5, 6, 71]}, "append through the map")
    toks = {0: [1], 1: [2]}
    step.append_sampled(toks, [1, 0], None, [8, 9])
    _check(toks == {0: [1, 9], 1: [2, 8]}, "append in order")

    # Correction of optimistic counts under asynchronous speculative decoding,
    # pinned by the synchronous path: a host that knows what the sampler kept
    # extends the history with the kept tokens itself and sets the count to
    # the positions whose K/V stays valid (the last committed token and the
    # accepted drafts).  The corrected asynchronous row (drafts in its history,
    # one placeholder for the next input, count advanced by d + 1) must agree
    # on the count and on the history through the new first input.  Rows are
    # reordered between the steps, so the sampler's order differs from the
    # rows' (a permutation maps them).
    for _ in range(200):
        R = int(rng.integers(1, 6))
        c0 = [int(rng.integers(0, 20)) for _ in range(R)]
        d = [int(rng.integers(0, 5)) for _ in range(R)]
        hist = [[int(x) for x in rng.integers(0, 1000, c0[i] + 1)] for i in range(R)]
        drafts = [[int(x) for x in rng.integers(1000, 2000, d[i])] for i in range(R)]
        n_acc = [int(rng.integers(0, d[i] + 1)) for i in range(R)]       # accepted drafts
        own = [int(rng.integers(2000, 3000)) for _ in range(R)]          # the sampler's own token
        pos_of = [int(x) for x in rng.permutation(R)]                    # sampler position of row i
        width = max(d) + 1
        sampled = [[-1] * width for _ in range(R)]
        kept_n = [0] * R
        for i in range(R):
            kept = drafts[i][:n_acc[i]] + [own[i]]
            sampled[pos_of[i]][:len(kept)] = kept
            kept_n[pos_of[i]] = len(kept)
        sync_hist = [hist[i] + drafts[i][:n_acc[i]] + [own[i]] for i in range(R)]
        sync_c = [c0[i] + 1 + n_acc[i] for i in range(R)]
        async_hist = [hist[i] + drafts[i] + [-7] for i in range(R)]
        async_c = [c0[i] + d[i] + 1 for i in range(R)]
        order = [int(x) for x in rng.permutation(R)]
        bad = step.correct_computed(async_c, async_hist, order, [pos_of[i] for i in order],
                                    [d[i] for i in order], kept_n, sampled)
        _check(bad == 0, "correction: no bad counts")
        for i in range(R):
            _check(async_c[i] == sync_c[i], "correction: count")
            _check(async_hist[i][:async_c[i] + 1] == sync_hist[i], "correction: history through the first input")
        # without sampled tokens only the count moves
        c_only = [c0[i] + d[i] + 1 for i in range(R)]
        h_only = [list(h) for h in async_hist]
        step.correct_computed(c_only, h_only, order, [pos_of[i] for i in order], [d[i] for i in order], kept_n)
        _check(c_only == sync_c and h_only == async_hist, "correction: count only")
    # kept counts outside [1, d + 1] leave their rows as they were
    c = [10, 10, 10]
    h = [list(range(12)) for _ in range(3)]
    bad = step.correct_computed(c, h, [0, 1, 2], [0, 1, 2], [2, 2, 2], [0, 4, 3], [[5, 6, 7, 8]] * 3)
    _check(bad == 2 and c == [10, 10, 10], "correction: out-of-range counts")
    _check(h[0] == list(range(12)) and h[1] == list(range(12)) and h[2][10] == 7, "correction: rows untouched")

    # Spec decode: no drafts reduces to the printed closed form; with drafts,
    # invariants stated independently.
    g = golden("p2_logits.json")
    qsl = g["query_start_loc"]
    m = step.spec_decode_metadata(qsl, list(range(qsl[-1])), [0, 0, 0])
    _check(m["logits_indices"] == g["expect"]["logits_indices"], "spec closed form")
    _check(m["bonus_logits_indices"] == [0, 1, 2] and m["cu_num_logits"] == [0, 1, 2, 3], "spec bonus")
    for _ in range(60):
        R = int(rng.integers(1, 5))
        q = rng.integers(1, 6, R)
        d = [int(rng.integers(0, qi)) for qi in q]
        qsl = [0] + [int(x) for x in np.cumsum(q)]
        ids = [int(x) for x in rng.integers(0, 1000, qsl[-1])]
        m = step.spec_decode_metadata(qsl, ids, d)
        pos = 0
        for i in range(R):
            lo, hi = m["cu_num_logits"][i], m["cu_num_logits"][i + 1]
            _check(hi - lo == d[i] + 1, "spec count")
            _check(m["logits_indices"][lo:hi] == list(range(qsl[i + 1] - d[i] - 1, qsl[i + 1])), "spec rows")
            _check(m["logits_indices"][m["bonus_logits_indices"][i]] == qsl[i + 1] - 1, "spec bonus row")
            for kk in range(d[i]):
                draft_pos = qsl[i + 1] - d[i] + kk
                _check(m["logits_indices"][m["target_logits_indices"][pos + kk]] == draft_pos - 1, "spec target")
                _check(m["draft_token_ids"][pos + kk] == ids[draft_pos], "spec draft id")
            pos += d[i]


def _pins_batch(batch):
    """Condense pins: the printed A,B,C,D example and invariants over random
    removal patterns (live rows end exactly [0, R), no request is lost, rows
    already below R stay put, the k-th hole takes the k-th highest row); and
    history truncation as the inverse of an append."""
    g = golden("p1_condense.json")
    b = batch.RefBatch(8, 16, 4, 100)
    for i, name in enumerate(g["rows"]):
        b.add_request(name, [1], 1, 0, [i + 1])
    for name in g["remove"]:
        b.remove_request(name)
    b.condense()
    _check([r.req_id for r in b.rows[:b.num_used_rows()]] == g["expect"]["rows"], "p1 condense")

    # Truncation undoes an append (rejected drafts leave the history), keeps
    # every other column, refuses to cut into the prompt.
    b = batch.RefBatch(2, 32, 4, 100)
    b.add_request(5, [10, 11, 12, 13], 3, 2, [7])
    b.append_tokens(5, [20, 21, 22])
    b.truncate_tokens(5, 5)
    r = b.rows[0]
    _check(r.tokens == [10, 11, 12, 13, 20], "truncate keeps the prefix")
    _check((r.num_prompt, r.num_computed, r.blocks) == (3, 2, [7]), "truncate keeps the columns")
    b.truncate_tokens(5, 5)
    _check(r.tokens == [10, 11, 12, 13, 20], "truncate to the length is a no-op")
    b.truncate_tokens(5, 3)
    _check(r.tokens == [10, 11, 12], "truncate to the prompt")
    for bad_len in (2, 4):
        try:
            b.truncate_tokens(5, bad_len)
        except batch.BatchError:
            continue
        raise AssertionError("truncate outside [prompt, length] accepted")
    rng = np.random.default_rng(9)
    for _ in range(100):
        n = int(rng.integers(1, 20))
        b = batch.RefBatch(n, 16, 4, 100)
        for i in range(n):
            b.add_request(i, [1], 1, 0, [1])
        gone = [i for i in range(n) if rng.random() < 0.4]
        for i in gone:
            b.remove_request(i)
        before = {i: b.row_of[i] for i in range(n) if i not in gone}
        R = len(before)
        pairs = b.condense()
        rows = [r.req_id if r is not None else None for r in b.rows[:n]]
        _check(all(x is not None for x in rows[:R]) and all(x is None for x in rows[R:]), "condensed")
        _check(sorted(x for x in rows[:R]) == sorted(before), "no request lost")
        _check(all(b.row_of[i] == r for i, r in before.items() if r < R), "low rows stay")
        holes = sorted(h for h in range(R) if h not in before.values())
        movers = sorted((r for r in before.values() if r >= R), reverse=True)
        _check(pairs == list(zip(holes, movers)), "k-th hole takes k-th highest row")


def _mutant(mod, old, new, name):
    src = open(mod.__file__, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    m = types.ModuleType(name)
    m.__file__ = mod.__file__
    sys.modules[name] = m           # dataclasses look their module up while the class is built
    try:
        exec(compile(src.replace(old, new), name, "exec"), m.__dict__)
    finally:
        del sys.modules[name]
    return m


STEP_MUTANTS = [
    ("k_cache[s] = k_rows[t]", "k_cache[s] = v_rows[t]"),                              # swapped operand
    ("v_cache[s] = v_rows[t]", "v_cache[t] = v_rows[t]"),                              # wrong index
    ("out.append(zero_row if idx < 0 else src_rows[idx])", "out.append(src_rows[idx])"),  # dropped case
    ("for m in range(count):", "for m in range(len(indices)):"),                       # ignores the count
    ("out.append(int(m) * ratio + j)", "out.append(int(m) + j)"),                      # dropped factor
    ("ids[j] if j < len(ids) else fill", "ids[j] if j < len(ids) else -1"),            # ignores fill
    ("ids = expand_kernel_blocks(r.blocks if blocks_of is None else blocks_of(i, r), ratio)",
     "ids = list(r.blocks if blocks_of is None else blocks_of(i, r))"),                # no expansion
    ("out.append(int(group_blocks[r][p // block_size]) * block_size + p % block_size)",
     "out.append(int(group_blocks[r][p % block_size]) * block_size + p // block_size)"),  # transposed
    ("out.append(null_block * block_size)", "out.append(-1)"),
    ("rows_tokens[row].append(int(sampled[src_index[k] if src_index is not None else k]))",
     "rows_tokens[row].append(int(sampled[k]))"),                                      # map ignored
    ("logits.append(end - (d + 1) + k)", "logits.append(end - d + k)"),                # off by one
    ("target.append(cu[-1] + k)", "target.append(cu[-1] + k + 1)"),
    ("drafts.append(int(input_ids[end - d + k]))", "drafts.append(int(input_ids[end - d + k - 1]))"),
    ("bonus.append(cu[-1] - 1)", "bonus.append(cu[-1])"),
    ("cu.append(cu[-1] + d + 1)", "cu.append(cu[-1] + d)"),
    ("num_computed[row] -= d + 1 - v", "num_computed[row] -= d - v"),                 # off by one
    ("v = int(num_accepted[p])", "v = int(num_accepted[k])"),                         # map ignored
    ("rows_tokens[row][num_computed[row]] = int(sampled[p][v - 1])",
     "rows_tokens[row][num_computed[row]] = int(sampled[k][v - 1])"),                 # map ignored
    ("rows_tokens[row][num_computed[row]] = int(sampled[p][v - 1])",
     "rows_tokens[row][num_computed[row] + 1] = int(sampled[p][v - 1])"),             # wrong position
    ("rows_tokens[row][num_computed[row]] = int(sampled[p][v - 1])",
     "rows_tokens[row][num_computed[row]] = int(sampled[p][0])"),                     # first, not last kept
    ("if v < 1 or v > d + 1:", "if v < 1 or v > d + 2:"),                             # bound off by one
    ("if v < 1 or v > d + 1:", "if v > d + 1:"),                                      # lower bound dropped
]

BATCH_MUTANTS = [
    ("live = [i for i in range(used - 1, -1, -1) if self.rows[i] is not None]",
     "live = [i for i in range(used) if self.rows[i] is not None]"),                  # lowest instead of highest
    ("            self.rows[l] = None\n", "            pass\n"),                      # source row kept
    ("holes = [i for i in range(used) if self.rows[i] is None]",
     "holes = [i for i in range(used - 1, -1, -1) if self.rows[i] is None]"),         # highest hole first
    ("del r.tokens[num_tokens:]", "del r.tokens[num_tokens + 1:]"),                   # keeps one too many
    ("if num_tokens < r.num_prompt or num_tokens > len(r.tokens):",
     "if num_tokens > len(r.tokens):"),                                               # cuts into the prompt
]


def test_unmutated_oracle_passes_the_pins():
    _pins_step(step_mod)
    _pins_batch(batch_mod)


@pytest.mark.parametrize("old,new", STEP_MUTANTS)
def test_step_mutant_is_caught(old, new):
    mod = _mutant(step_mod, old, new, "step_mutant_next")
    with pytest.raises(Exception):
        _pins_step(mod)


@pytest.mark.parametrize("old,new", BATCH_MUTANTS)
def test_batch_mutant_is_caught(old, new):
    mod = _mutant(batch_mod, old, new, "batch_mutant_next")
    with pytest.raises(Exception):
        _pins_batch(mod)
