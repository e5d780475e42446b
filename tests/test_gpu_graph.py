"""The step's output buffers keep their addresses for the handle's lifetime,
so a caller can capture compile + K/V write + gather in a HIP graph and replay
it.  Every replay is checked against the eager step, with eager work (clearing
the outputs, new K/V sources and hidden rows) and synchronisations between
replays."""
import numpy as np
import pytest
import torch

import workloads
from tests.gpu_helpers import assert_step_equal, expected_step, replay_history

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ragged_input_compilation_amd import _ric, runner
    return _ric, runner


@pytest.mark.parametrize("name,single", [("worked_example", False), ("worked_example", True), ("mixed", False),
                                         ("mixed", True), ("decode_heavy", True)])
def test_captured_step_replays_match_eager(rt, name, single):
    """`single`: the step is ric_compile_and_cache (one kernel for these rows:
    256 B in the worked example, 2 KiB otherwise) + gather instead of three
    calls."""
    ric, runner = rt
    w = workloads.get(name)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        st = runner.current_stream()
        b = runner.Batch(runner.config_of(w), stream=st)
        b.load_history(w)
        ref, order = replay_history(w)
        b.schedule_from(w, order)
        exp = expected_step(w, ref, use_python=(name == "worked_example"))
        n_pad = exp["n_pad"]
        R = exp["num_reqs"]
        kc, vc = runner.alloc_caches(w, fill=0)
        k, v = runner.alloc_sources(w, n_pad, seed=w.seed + 3)
        kv = runner.KVSet(k, v, kc, vc, w.row_bytes, w.num_kv_blocks * w.block_size)
        hidden = torch.randn((n_pad, w.hidden_size), device="cuda").to(torch.bfloat16)
        out = torch.zeros((R, w.hidden_size), dtype=torch.bfloat16, device="cuda")

        def step():
            if single:
                s = runner.compile_and_cache(b, n_pad, kv, flags=ric.RIC_FUSE_ALWAYS)
            else:
                s = b.compile(n_pad)
                runner.reshape_and_cache(kv, s.slot_mapping, n_pad, stream=st)
            runner.gather(hidden, s.logits_indices, 0, R, out, stream=st)
            return s

        s0 = step()                 # eager: flushes every staged delta before the capture
        torch.cuda.synchronize()
        eager = b.step_outputs(s0)
        assert_step_equal(eager, exp, f"{name} eager")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step()
    slots = torch.from_numpy(np.asarray(exp["slot_mapping"][:exp["num_actual_tokens"]], np.int64)).cuda()
    logits = torch.from_numpy(np.asarray(exp["logits_indices"][:R], np.int64)).cuda()
    for rep in range(4):
        # eager work between replays: clear the outputs, new sources and hidden rows
        with torch.cuda.stream(side):
            for ptr, n in ((s0.input_ids, n_pad), (s0.positions, n_pad), (s0.slot_mapping, n_pad),
                           (s0.query_start_loc, w.max_num_reqs + 1), (s0.logits_indices, w.max_num_reqs)):
                runner._view_u8(b.workspace, ptr, 4 * n).zero_()
            for t in kc + vc:
                t.view(torch.int16).zero_()
            for t in k + v:
                t.copy_(torch.randn(t.shape, device=t.device).to(t.dtype))
            hidden.copy_(torch.randn_like(hidden, dtype=torch.float32).to(hidden.dtype))
            out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = b.step_outputs(s0)
        assert_step_equal(got, exp, f"{name} replay {rep}")
        for l in range(w.num_layers):
            for src, cache in ((k[l], kc[l]), (v[l], vc[l])):
                flat = cache.view(torch.int16).reshape(w.num_kv_blocks * w.block_size, -1)
                srcf = src.view(torch.int16).reshape(n_pad, -1)
                assert torch.equal(flat[slots], srcf[:exp["num_actual_tokens"]]), \
                    f"{name} replay {rep} layer {l}: K/V rows"
        assert torch.equal(out.view(torch.int16), hidden[logits].view(torch.int16)), f"{name} replay {rep}: gather"
    del g, kv, kc, vc, k, v
    b.close()
    torch.cuda.empty_cache()


def test_capture_with_staged_deltas_is_refused(rt):
    """A compile whose schedule is still staged must not be captured: the
    upload would replay from a pinned log that later flushes rewrite.  The
    call inside the capture fails with ESTATE and changes nothing; after the
    capture the same compile runs eagerly and equals the oracle."""
    ric, runner = rt
    w = workloads.get("worked_example")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        st = runner.current_stream()
        b = runner.Batch(runner.config_of(w), stream=st)
        b.load_history(w)
        ref, order = replay_history(w)
        b.schedule_from(w, order)            # the counts are staged, not yet uploaded
        exp = expected_step(w, ref, use_python=True)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        codes = []
        with torch.cuda.graph(g, stream=side):
            for fn, a in ((ric.ric_compile, (b.h, exp["n_pad"])), (ric.ric_flush, (b.h,))):
                try:
                    fn(*a)
                    codes.append(0)
                except ric.RicError as e:
                    codes.append(e.code)
        assert codes == [ric.RIC_ESTATE, ric.RIC_ESTATE]
        s = b.compile(exp["n_pad"])
        torch.cuda.synchronize()
        assert_step_equal(b.step_outputs(s), exp, "after a refused capture")
    del g
    b.close()
