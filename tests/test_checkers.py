"""The whole-cache K/V checker the GPU parity tests use, pinned on the CPU
with planted mistakes: it must pass a correct write and fail a stray write
outside the step, a wrong real row, a real row left unwritten and a shifted
slot list, while ignoring writes into the null block."""
import numpy as np
import pytest
import torch

from tests.gpu_helpers import check_cache_exact


def _case(seed=3, num_slots=400, n=120, row_elems=64, null=(0, 16)):
    rng = np.random.default_rng(seed)
    sentinel = 0x2B2B
    slots = (rng.permutation(num_slots - null[1]) + null[1])[:n].astype(np.int64)
    src = torch.from_numpy(rng.integers(-30000, 30000, (n, row_elems)).astype(np.int16))
    cache = torch.full((num_slots, row_elems), sentinel, dtype=torch.int16)
    cache[torch.from_numpy(slots)] = src
    return cache, src, slots, sentinel, num_slots, null


def test_checker_accepts_a_correct_write():
    cache, src, slots, s, ns, null = _case()
    check_cache_exact(cache, src, slots, len(slots), s, ns, null, "ok", chunk_rows=64)
    cache[3, 5] = 77                      # pad tokens write the null block: ignored
    check_cache_exact(cache, src, slots, len(slots), s, ns, null, "null block", chunk_rows=64)


@pytest.mark.parametrize("mistake", ["stray", "wrong_row", "unwritten", "shifted", "last_byte"])
def test_checker_rejects_planted_mistakes(mistake):
    cache, src, slots, s, ns, null = _case()
    if mistake == "stray":
        free = sorted(set(range(null[1], ns)) - set(slots.tolist()))
        cache[free[-1], 0] = 1
    elif mistake == "wrong_row":
        cache[int(slots[7])] = src[8]
    elif mistake == "unwritten":
        cache[int(slots[-1])] = s
    elif mistake == "shifted":
        free = sorted(set(range(null[1], ns)) - set(slots.tolist()))
        slots = slots.copy()
        slots[0] = free[0]                # the oracle's slot list disagrees with the write
    else:
        free = sorted(set(range(null[1], ns)) - set(slots.tolist()))
        cache[free[0], -1] = s + 1     # one word in the last 8 bytes of a free row
    with pytest.raises(AssertionError):
        check_cache_exact(cache, src, slots, len(slots), s, ns, null, mistake, chunk_rows=64)
