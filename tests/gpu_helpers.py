"""Helpers for the GPU parity tests: oracle expectations for a workload and
device readback.  Expectations come only from ``oracle`` and the seeded
generators; the library's outputs are only ever compared against them."""
import numpy as np
import torch

from oracle import batch as ref_batch, cbind, step as ref_step
from tests.oracle_helpers import KEYS


def replay_history(w):
    """Replay the workload's request history on the reference batch; returns
    (RefBatch, row order as request ids)."""
    b = ref_batch.RefBatch(w.max_num_reqs, w.max_model_len, w.max_blocks_per_req, w.num_kv_blocks)
    for r in w.initial:
        b.add_request(r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks,
                      (r.temperature, r.top_p, r.rep_penalty, r.top_k))
    for rid in w.finished:
        b.remove_request(rid)
    if w.finished:
        b.condense()
    for r in w.refill:
        b.add_request(r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks,
                      (r.temperature, r.top_p, r.rep_penalty, r.top_k))
    order = [rid for rid in b.req_ids_by_row() if rid is not None]
    by_id = w.by_id()
    b.schedule([by_id[i].num_computed for i in order], [by_id[i].num_scheduled for i in order])
    return b, order


def expected_step(w, b, use_python: bool = False):
    rows = b.step_rows()
    n = sum(r.num_scheduled for r in rows)
    n_pad = ref_step.padded_size(w.capture_sizes, n)
    if use_python:
        res = ref_step.compile_step(rows, block_size=w.block_size, max_num_reqs=w.max_num_reqs,
                                    max_model_len=w.max_model_len,
                                    max_num_batched_tokens=w.max_num_batched_tokens,
                                    num_kv_blocks=w.num_kv_blocks, n_pad=n_pad)
    else:
        res = cbind.compile_step(rows, block_size=w.block_size, max_num_reqs=w.max_num_reqs, n_pad=n_pad)
    out = {k: np.asarray(res[k], np.int64) for k in KEYS}
    for k in ("num_sampled", "max_query_len", "max_seq_len", "num_actual_tokens"):
        out[k] = int(res[k])
    out["n_pad"] = n_pad
    out["num_reqs"] = len(rows)
    return out


def assert_step_equal(got: dict, exp: dict, label: str = ""):
    for k in KEYS:
        g = np.asarray(got[k], np.int64)
        e = exp[k]
        assert g.shape == e.shape, f"{label} {k}: shape {g.shape} vs {e.shape}"
        if not np.array_equal(g, e):
            bad = np.nonzero(g != e)[0]
            i = int(bad[0])
            raise AssertionError(f"{label} {k}: {bad.size} mismatches, first at {i}: got {g[i]} expected {e[i]}")
    ds = got["dev_scalars"]
    assert list(ds[:6]) == [exp["num_reqs"], exp["num_actual_tokens"], exp["n_pad"], exp["max_query_len"],
                            exp["max_seq_len"], exp["num_sampled"]], f"{label} dev_scalars {list(ds)}"


def u16(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


def check_cache_exact(cache: torch.Tensor, src: torch.Tensor, slots: np.ndarray, num_real: int,
                      sentinel16: int, num_slots: int, null_rows=(0, 0), label: str = "",
                      chunk_rows: int = 1 << 18) -> None:
    """Whole-cache byte check of one K or V cache after a write, on the device.

    ``slots``: the oracle's slot list (int, at least num_real entries); token t
    of ``src`` (rows of the same byte size as a cache row) belongs at slot[t].
    Checks (1) every real row: cache[slot[t]] == src[t] for all t < num_real;
    (2) every other row outside ``null_rows`` = [lo, hi) still holds the
    sentinel in every byte: the set of rows holding any non-sentinel word,
    null rows excluded, must equal the set of real slots.  The null block is
    excluded because padded tokens write there."""
    row_bytes = cache.numel() * cache.element_size() // num_slots
    assert row_bytes % 8 == 0
    flat16 = cache.view(torch.int16).reshape(num_slots, row_bytes // 2)
    src16 = src.reshape(src.shape[0], -1).view(torch.int16)
    assert src16.shape[1] == row_bytes // 2
    s_all = torch.from_numpy(np.asarray(slots[:num_real], np.int64)).to(cache.device)
    for a in range(0, num_real, 8192):
        b = min(num_real, a + 8192)
        got = flat16[s_all[a:b]]
        want = src16[a:b]
        if not torch.equal(got, want):
            bad = (got != want).any(dim=1).nonzero().flatten()
            t = a + int(bad[0])
            raise AssertionError(f"{label}: {bad.numel()} real rows differ in tokens [{a},{b}); first token {t} "
                                 f"at slot {int(s_all[t])}")
    pat = np.array([sentinel16 & 0xFFFF] * 4, np.uint16).view(np.int64)[0]
    flat64 = cache.view(torch.int64).reshape(num_slots, row_bytes // 8)
    found = []
    for a in range(0, num_slots, chunk_rows):
        b = min(num_slots, a + chunk_rows)
        found.append((flat64[a:b] != int(pat)).any(dim=1).nonzero().flatten() + a)
    found = torch.cat(found)
    lo, hi = null_rows
    found = found[(found < lo) | (found >= hi)]
    expected = torch.unique(s_all)
    expected = expected[(expected < lo) | (expected >= hi)]
    if not torch.equal(found, expected):
        extra = found[~torch.isin(found, expected)]
        missing = expected[~torch.isin(expected, found)]
        raise AssertionError(f"{label}: {extra.numel()} rows outside the step were written (first "
                             f"{extra[:4].tolist()}), {missing.numel()} real slots still hold the sentinel "
                             f"(first {missing[:4].tolist()})")


def read_rows_i32(ptr_base_tensor, ptr, stride, rows, n) -> np.ndarray:
    """Rows [rows] of an int32 device matrix (at ptr, row stride in elements),
    first n columns, as numpy."""
    from ragged_input_compilation_amd.runner import _view_u8
    out = np.zeros((len(rows), n), np.int32)
    for k, r in enumerate(rows):
        v = _view_u8(ptr_base_tensor, ptr + 4 * stride * r, 4 * n).view(torch.int32)
        out[k] = v.cpu().numpy()
    return out
