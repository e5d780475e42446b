"""The slot-collision check on the GPU: every configuration's compiled slots
have no collision; planted collisions and out-of-range slots are counted as
the definition says (a token counts when an earlier token of the call holds
its slot; tokens past the device count are not looked at)."""
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


def _check(ric, runner, slots_ptr, n, num_slots, dev_n=0):
    nbytes = ric.ric_check_slots_workspace_bytes(num_slots)
    ws = torch.full((nbytes // 4,), -1, dtype=torch.int32, device="cuda")     # stale bits must not matter
    res = torch.zeros(2, dtype=torch.int32, device="cuda")
    ric.ric_check_slots(slots_ptr, n, num_slots, ws.data_ptr(), nbytes, res.data_ptr(), dev_n,
                        runner.current_stream())
    torch.cuda.synchronize()
    return res.tolist()


def _expected(slots, num_slots):
    s = np.asarray(slots, np.int64)
    ok = (s >= 0) & (s < num_slots)
    return [int(ok.sum() - np.unique(s[ok]).size), int((~ok).sum())]


@pytest.mark.parametrize("name", ["worked_example", "decode_heavy", "mixed", "churn", "long_context"])
def test_compiled_slots_have_no_collision(rt, name):
    ric, runner = rt
    w = workloads.get(name)
    b = runner.Batch(runner.config_of(w))
    b.load_history(w)
    ref, order = replay_history(w)
    b.schedule_from(w, order)
    exp = expected_step(w, ref)
    s = b.compile(exp["n_pad"])
    num_slots = w.num_kv_blocks * w.block_size
    # the real tokens, counted on the device (dev_scalars[1] = N)
    assert _check(ric, runner, s.slot_mapping, exp["n_pad"], num_slots, s.dev_scalars + 4) == [0, 0]
    if exp["n_pad"] > exp["num_actual_tokens"] + 1:
        # the padded tail shares the null block's first slot
        pad = exp["n_pad"] - exp["num_actual_tokens"]
        assert _check(ric, runner, s.slot_mapping, exp["n_pad"], num_slots) == [pad - 1, 0]
    b.close()


@pytest.mark.parametrize("num_slots,n,dups,bad", [(1000, 300, 40, 5), (1 << 24, 70000, 3000, 17),
                                                  (1 << 31, 5000, 100, 3), (37, 37, 0, 0), (64, 200, 150, 0)])
def test_planted_collisions_are_counted(rt, num_slots, n, dups, bad):
    ric, runner = rt
    rng = np.random.default_rng(n + dups)
    uniq = min(n - dups - bad, num_slots)
    base = rng.choice(num_slots, size=uniq, replace=False) if num_slots < (1 << 26) else \
        np.unique(rng.integers(0, num_slots, size=uniq * 2))[:uniq]
    slots = np.concatenate([base, rng.choice(base, size=n - uniq - bad), np.full(bad, -3)])
    slots[-bad // 2 if bad else len(slots):] = num_slots if num_slots < (1 << 31) else -7
    rng.shuffle(slots)
    dev = torch.from_numpy(slots.astype(np.int32)).cuda()
    assert _check(ric, runner, dev.data_ptr(), n, num_slots) == _expected(slots, num_slots)
    # a device count below n: only that prefix is looked at
    k = n // 3
    cnt = torch.tensor([k], dtype=torch.int32, device="cuda")
    assert _check(ric, runner, dev.data_ptr(), n, num_slots, cnt.data_ptr()) == _expected(slots[:k], num_slots)


def test_check_slots_argument_errors(rt):
    ric, runner = rt
    slots = torch.zeros(4, dtype=torch.int32, device="cuda")
    res = torch.zeros(2, dtype=torch.int32, device="cuda")
    ws = torch.zeros(64, dtype=torch.int32, device="cuda")
    for args in ((slots.data_ptr(), 4, 100 * 32 * 64, ws.data_ptr(), 256, res.data_ptr()),   # workspace too small
                 (slots.data_ptr(), 4, 0, ws.data_ptr(), 256, res.data_ptr()),                # no slots
                 (slots.data_ptr(), -1, 10, ws.data_ptr(), 256, res.data_ptr()),              # negative count
                 (slots.data_ptr(), 4, 10, 0, 256, res.data_ptr()),                           # no workspace
                 (slots.data_ptr(), 4, 10, ws.data_ptr(), 256, 0)):                           # no result
        with pytest.raises(ric.RicError) as e:
            ric.ric_check_slots(*args)
        assert e.value.code == ric.RIC_EINVAL
    assert ric.ric_check_slots_workspace_bytes(0) == 0
    assert ric.ric_check_slots_workspace_bytes((1 << 31) + 1) == 0
    assert ric.ric_check_slots_workspace_bytes(33) == 256
