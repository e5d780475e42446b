"""The allocation-free slot-collision check (static device bitmap) against the
check with a caller workspace, through the C ABI: the same counts on two
calls in a row, the second with fewer tokens and fewer slots (the bitmap keeps
the first call's bits until the second clears its own range), on compiled
slots and on planted collisions; sizes above the static bitmap are refused."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import expected_step, replay_history

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_input_compilation_amd import _ric, runner
    return _ric, runner


def _both(ric, runner, slots_ptr, n, num_slots, dev_n=0):
    nbytes = ric.ric_check_slots_workspace_bytes(num_slots)
    ws = torch.full((nbytes // 4,), -1, dtype=torch.int32, device="cuda")
    with_ws = torch.zeros(2, dtype=torch.int32, device="cuda")
    no_alloc = torch.zeros(2, dtype=torch.int32, device="cuda")
    st = runner.current_stream()
    ric.ric_check_slots(slots_ptr, n, num_slots, ws.data_ptr(), nbytes, with_ws.data_ptr(), dev_n, st)
    ric.ric_check_slots_noalloc(slots_ptr, n, num_slots, no_alloc.data_ptr(), dev_n, st)
    torch.cuda.synchronize()
    return with_ws.tolist(), no_alloc.tolist()


def _planted(rng, num_slots, n, dups, bad):
    uniq = min(n - dups - bad, num_slots)
    base = rng.choice(num_slots, size=uniq, replace=False)
    slots = np.concatenate([base, rng.choice(base, size=n - uniq - bad), np.full(bad, num_slots)])
    rng.shuffle(slots)
    return torch.from_numpy(slots.astype(np.int32)).cuda()


def test_no_alloc_check_matches_workspace_check(rt):
    ric, runner = rt
    rng = np.random.default_rng(2024)
    # first call: the largest bitmap the static array holds, many collisions
    big = _planted(rng, 1 << 25, 200000, 5000, 9)
    a, b = _both(ric, runner, big.data_ptr(), big.numel(), 1 << 25)
    assert a == b == [5000, 9]
    # second call, smaller: the first call's bits are still in the array
    small = _planted(rng, 4000, 1500, 77, 2)
    a, b = _both(ric, runner, small.data_ptr(), small.numel(), 4000)
    assert a == b == [77, 2]
    # a device count below n
    cnt = torch.tensor([700], dtype=torch.int32, device="cuda")
    a, b = _both(ric, runner, small.data_ptr(), small.numel(), 4000, cnt.data_ptr())
    assert a == b


@pytest.mark.parametrize("name", ["churn", "mixed", "worked_example"])
def test_no_alloc_check_on_compiled_slots(rt, name):
    ric, runner = rt
    w = workloads.get(name)
    b = runner.Batch(runner.config_of(w))
    b.load_history(w)
    ref, order = replay_history(w)
    b.schedule_from(w, order)
    exp = expected_step(w, ref)
    s = b.compile(exp["n_pad"])
    num_slots = w.num_kv_blocks * w.block_size
    for n, dev_n in ((exp["n_pad"], s.dev_scalars + 4), (exp["n_pad"], 0)):
        x, y = _both(ric, runner, s.slot_mapping, n, num_slots, dev_n)
        assert x == y
        if dev_n:
            assert y == [0, 0]
    b.close()


def test_no_alloc_check_refuses_above_its_bitmap(rt):
    ric, runner = rt
    slots = torch.zeros(4, dtype=torch.int32, device="cuda")
    res = torch.zeros(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ric.RicError) as e:
        ric.ric_check_slots_noalloc(slots.data_ptr(), 4, (1 << 25) + 1, res.data_ptr())
    assert e.value.code == ric.RIC_ERANGE
    assert res.tolist() == [0, 0]
