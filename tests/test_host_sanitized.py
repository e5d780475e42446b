"""The library's host control plane (ric_host.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: it is built with g++ together with a
test double for the device (tests/host_fake/fake_device.cpp: "device" memory
is host memory; only the column-store kernels act), loaded through the normal
binding, and driven through a seeded random sequence of adds, removals,
token appends and truncations, block appends and replacements (two KV-cache
groups), condense,
sampled-token appends, schedules, corrections of optimistic computed counts
and compiles, with a staging log small
enough to force split uploads.  After every flush the column store equals the
reference batch.  The stateless K/V-write and gather calls then run their
argument checks.  Any out-of-bounds access or undefined behaviour aborts."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import ctypes, sys
import numpy as np
sys.path.insert(0, {root!r})
from ragged_input_compilation_amd import _ric as ric
from oracle.batch import RefBatch
from oracle import step as ref_step

MR, M, MB, POOL, B = 24, 96, 24, 60000, 4
GB1 = 8                          # group 1 block size (its table holds M / GB1 entries)
cfg = ric.make_config(max_num_reqs=MR, max_model_len=M, block_size=B, max_blocks_per_req=MB,
                      max_num_batched_tokens=256, num_kv_blocks=POOL, null_block=0,
                      staging_bytes=2 * 12 * MR * 4 + (64 << 10), num_kv_groups=2,
                      group_block_size=[0, GB1], group_num_kv_blocks=[0, POOL], group_slot_mode=[0, 0])
h = ric.ric_create(cfg, 0)
ref = RefBatch(MR, M, MB, POOL)
rng = np.random.default_rng(17)
free = list(rng.permutation(np.arange(1, POOL)))
next_id = 0
corrections = 0

def words(ptr, n):
    return np.ctypeslib.as_array((ctypes.c_int32 * max(n, 1)).from_address(ptr))[:n].copy()

def check():
    ric.ric_flush(h)
    cols = ric.ric_get_columns(h)
    for row, r in enumerate(ref.rows):
        if r is None:
            continue
        T = len(r.tokens)
        assert words(cols.num_tokens + 4 * row, 1)[0] == T, row
        assert words(cols.num_prompt + 4 * row, 1)[0] == r.num_prompt, row
        assert words(cols.num_blocks + 4 * row, 1)[0] == len(r.blocks), row
        assert list(words(cols.tokens + 4 * row * cols.token_stride, T)) == r.tokens, row
        assert list(words(cols.blocks + 4 * row * cols.block_stride, len(r.blocks))) == r.blocks, row
        g1 = r.group_blocks.get(1, [])
        assert words(cols.group_num_blocks[1] + 4 * row, 1)[0] == len(g1), row
        assert list(words(cols.group_blocks[1] + 4 * row * cols.group_block_stride[1], len(g1))) == g1, row
        temp = np.ctypeslib.as_array((ctypes.c_float * 1).from_address(cols.temperature + 4 * row))[0]
        assert temp == np.float32(r.sampling[0]), row
    assert ric.ric_num_reqs(h) == ref.num_live()
    for row in range(MR):
        want = ref.rows[row].req_id if ref.rows[row] is not None else None
        assert ric.ric_req_at(h, row) == want, row

def take(n):
    return [int(free.pop()) for _ in range(n)]

for step in range(600):
    op = rng.integers(0, 9)
    live = [r.req_id for r in ref.rows if r is not None]
    if op <= 1 and ref.num_live() < MR:
        T = int(rng.integers(1, M - 10))
        toks = rng.integers(0, 1 << 20, T).tolist()
        blocks = take(-(-T // B))
        samp = (float(rng.random()), float(rng.random()), 1.0, int(rng.integers(0, 50)))
        c = int(rng.integers(0, T))
        ric.ric_add_request(h, next_id, toks, T, c, blocks, samp)
        ref.add_request(next_id, toks, T, c, blocks, samp)
        g1 = take(-(-T // GB1))
        ric.ric_append_blocks_group(h, next_id, 1, g1)
        ref.append_blocks_group(next_id, 1, g1)
        next_id += 1
    elif op in (2, 3) and live:
        for rid in rng.choice(live, size=int(rng.integers(1, min(4, len(live)) + 1)), replace=False):
            ric.ric_remove_request(h, int(rid))
            ref.remove_request(int(rid))
    elif op == 4 and live:
        rid = int(rng.choice(live))
        r = ref.rows[ref.row_of[rid]]
        n = int(rng.integers(0, min(8, M - len(r.tokens)) + 1))
        ids = rng.integers(0, 1 << 20, n).tolist()
        ric.ric_append_tokens(h, rid, ids)
        ref.append_tokens(rid, ids)
        if n and rng.random() < 0.5:
            # drafts rejected: cut back into what was just appended (still
            # staged) and append other ids over the same positions
            keep = max(r.num_prompt, len(r.tokens) - int(rng.integers(1, n + 1)))
            ric.ric_truncate_tokens(h, rid, keep)
            ref.truncate_tokens(rid, keep)
            more = rng.integers(0, 1 << 20, int(rng.integers(0, 4))).tolist()
            ric.ric_append_tokens(h, rid, more)
            ref.append_tokens(rid, more)
        need = -(-len(r.tokens) // B) - len(r.blocks)
        if need > 0:
            more = take(need)
            ric.ric_append_blocks(h, rid, more)
            ref.append_blocks(rid, more)
        need1 = -(-len(r.tokens) // GB1) - len(r.group_blocks.get(1, []))
        if need1 > 0:
            more = take(need1)
            ric.ric_append_blocks_group(h, rid, 1, more)
            ref.append_blocks_group(rid, 1, more)
    elif op == 5 and live:
        rid = int(rng.choice(live))
        r = ref.rows[ref.row_of[rid]]
        ids = take(len(r.blocks))
        ric.ric_replace_blocks(h, rid, ids)
        ref.replace_blocks(rid, ids)
        ids1 = take(len(r.group_blocks.get(1, [])))
        ric.ric_replace_blocks_group(h, rid, 1, ids1)
        ref.replace_blocks_group(rid, 1, ids1)
    elif op == 6:
        assert ric.ric_condense(h) == len(ref.condense())
        check()
    elif op == 7 and live:
        ric.ric_condense(h)
        ref.condense()
        rows = [i for i, r in enumerate(ref.rows) if r is not None and len(r.tokens) < M
                and -(-(len(r.tokens) + 1) // B) <= len(r.blocks) and -(-(len(r.tokens) + 1) // GB1)
                <= len(r.group_blocks.get(1, []))]
        if rows:
            sampled = np.asarray(rng.integers(0, 1 << 20, len(rows)), np.int32)
            src = list(rng.permutation(len(rows)))
            ric.ric_append_sampled(h, rows, sampled.ctypes.data, len(rows), src)
            for k, row in enumerate(rows):
                ref.rows[row].tokens.append(int(sampled[src[k]]))
        check()
    elif op == 8 and live:
        ric.ric_condense(h)
        ref.condense()
        R = ref.num_live()
        c, q = [], []
        for i in range(R):
            r = ref.rows[i]
            T = len(r.tokens)
            ci = int(rng.integers(0, T))
            qi = int(rng.integers(1, T - ci + 1))
            c.append(ci)
            q.append(qi)
        if sum(q) <= 256:
            ric.ric_schedule(h, c, q)
            ref.schedule(c, q)
            if rng.random() < 0.5:
                # optimistic counts corrected from "device" accepted counts
                n = int(rng.integers(1, R + 1))
                rows_k = [int(x) for x in rng.choice(R, size=n, replace=False)]
                d = [int(rng.integers(0, min(c[i], 3) + 1)) for i in rows_k]
                prev_len = R + 2
                pos = [int(x) for x in rng.choice(prev_len, size=n, replace=False)]
                acc = np.asarray(rng.integers(0, 6, prev_len), np.int32)     # some outside [1, d + 1]
                samp = np.asarray(rng.integers(0, 1 << 20, (prev_len, 4)), np.int32)
                status = np.zeros(1, np.int32)
                ric.ric_correct_computed(h, rows_k, pos, d, acc.ctypes.data, prev_len, samp.ctypes.data, 4,
                                         status.ctypes.data)
                try:
                    ric.ric_correct_computed(h, rows_k, pos, d, acc.ctypes.data, prev_len)
                    raise AssertionError("second correction accepted")
                except ric.RicError as e:
                    assert e.code == ric.RIC_ESTATE
                cc = [ref.rows[i].num_computed for i in range(R)]
                bad = ref_step.correct_computed(cc, [ref.rows[i].tokens for i in range(R)], rows_k, pos, d, acc,
                                                samp.tolist())
                for i in range(R):
                    ref.rows[i].num_computed = cc[i]
                ric.ric_flush(h)
                cols = ric.ric_get_columns(h)
                assert status[0] == bad
                assert list(words(cols.num_computed, R)) == cc
                corrections += 1
            s = ric.ric_compile(h, sum(q))
            assert (s.num_reqs, s.num_actual_tokens) == (R, sum(q))
            d = [min(x - 1, 2) for x in q]
            m = ric.ric_spec_decode_metadata(h, d)
            assert m.num_logits == sum(d) + R
            check()
check()
ric.ric_destroy(h)

# Uploads are refused while the stream is being captured, with nothing
# changed; once the capture ends the same calls go through.
cfg2 = ric.make_config(max_num_reqs=4, max_model_len=16, block_size=4, max_blocks_per_req=4,
                       max_num_batched_tokens=16, num_kv_blocks=32, null_block=0, staging_bytes=0)
h2 = ric.ric_create(cfg2, 0)
ric.ric_add_request(h2, 4, [9], 1, 0, [5])
ric.ric_add_request(h2, 5, [1, 2, 3, 4, 5], 5, 0, [3, 4])
ric.ric_flush(h2)
ric.ric_remove_request(h2, 4)                 # a hole at row 0
ric.lib().fake_set_capturing(1)
for fn, a in ((ric.ric_condense, (h2,)),):
    try:
        fn(*a)
        raise AssertionError(f"{{fn.__name__}} uploaded during a capture")
    except ric.RicError as e:
        assert e.code == ric.RIC_ESTATE, (fn.__name__, e.code)
ric.lib().fake_set_capturing(0)
assert ric.ric_condense(h2) == 1 and ric.ric_row_of(h2, 5) == 0
ric.ric_schedule(h2, [0], [5])
ric.lib().fake_set_capturing(1)
for fn, a in ((ric.ric_compile, (h2, 8)), (ric.ric_flush, (h2,)), (ric.ric_spec_decode_metadata, (h2, [0]))):
    try:
        fn(*a)
        raise AssertionError(f"{{fn.__name__}} uploaded during a capture")
    except ric.RicError as e:
        assert e.code == ric.RIC_ESTATE, (fn.__name__, e.code)
ric.lib().fake_set_capturing(0)
s2 = ric.ric_compile(h2, 8)
assert (s2.num_reqs, s2.num_actual_tokens) == (1, 5)
cols2 = ric.ric_get_columns(h2)
assert list(words(cols2.tokens, 5)) == [1, 2, 3, 4, 5] and list(words(cols2.num_scheduled, 1)) == [5]
ric.lib().fake_set_capturing(1)
s2 = ric.ric_compile(h2, 8)        # nothing staged: a capture may record the compile
ric.lib().fake_set_capturing(0)
ric.ric_destroy(h2)

# The stateless entry points' argument checks (the fake device runs no kernels).
def rejects(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except ric.RicError as e:
        return e.code
    raise AssertionError("accepted")

buf = np.zeros(1 << 16, np.uint8)
base = (buf.ctypes.data + 255) // 256 * 256
slots = np.zeros(8, np.int32)
idx = np.zeros(8, np.int32)
P = [base] * 40
kv = ric.ric_reshape_and_cache
kv(P, P, P, P, slots.ctypes.data, 8, 64, 100)                        # 40 layers: two launches
kv(P[:3], P[:3], P[:3], P[:3], slots.ctypes.data, 8, 64, 100, src_row_stride=128)
kv(P[:3], P[:3], P[:3], P[:3], slots.ctypes.data, 0, 64, 100)         # nothing to write
for args, kw in (((P, P, P, P, slots.ctypes.data, 8, 24, 100), {{}}),                   # row not 16-byte multiple
                 ((P, P, P, P, slots.ctypes.data, 8, 64, 100), dict(src_row_stride=32)),  # stride below the row
                 ((P, P, P, [base + 8] * 40, slots.ctypes.data, 8, 64, 100), {{}}),        # misaligned cache
                 ((P, P, P, P, slots.ctypes.data, (1 << 24) + 1, 64, 100), {{}}),         # above the launch limit
                 ((P, P, P, P, slots.ctypes.data, 8, 64, 0), {{}}),                       # no slots
                 ((P, P, P, P, slots.ctypes.data, 8, 64, 100), dict(flags=1)),          # unknown flag
                 ((P, P, P, P, 0, 8, 64, 100), {{}})):                                   # no slot mapping
    assert rejects(kv, *args, **kw) == ric.RIC_EINVAL, (args[5:], kw)
g = ric.ric_gather_rows
g(base, 64, 8, idx.ctypes.data, 0, 8, 64, base + 4096)
g(base, 64, 8, idx.ctypes.data, 0, 0, 64, base + 4096)                # no rows
for args in ((base, 64, 8, idx.ctypes.data, 0, 8, 40, base + 4096),     # row not 16-byte multiple
             (base, 32, 8, idx.ctypes.data, 0, 8, 64, base + 4096),     # source stride below the row
             (base + 8, 64, 8, idx.ctypes.data, 0, 8, 64, base + 4096), # misaligned source
             (base, 64, -1, idx.ctypes.data, 0, 8, 64, base + 4096),    # negative source rows
             (base, 64, 8, idx.ctypes.data, 0, (1 << 24) + 1, 64, base + 4096)):
    assert rejects(g, *args) == ric.RIC_EINVAL, args
# The slot-collision check: host argument checks, and the counts through the
# device double.
cs = ric.ric_check_slots
nslots = 1000
ws = np.zeros(ric.ric_check_slots_workspace_bytes(nslots) // 4, np.uint32)
res = np.zeros(2, np.int32)
sl = np.asarray([5, 7, 5, 999, 1000, -1, 7, 7], np.int32)
cs(sl.ctypes.data, 8, nslots, ws.ctypes.data, ws.nbytes, res.ctypes.data)
assert list(res) == [3, 2], list(res)
cnt = np.asarray([3], np.int32)
res[:] = 0
cs(sl.ctypes.data, 8, nslots, ws.ctypes.data, ws.nbytes, res.ctypes.data, cnt.ctypes.data)
assert list(res) == [1, 0], list(res)
for args in ((sl.ctypes.data, 8, nslots, ws.ctypes.data, ws.nbytes - 256, res.ctypes.data),
             (sl.ctypes.data, 8, 0, ws.ctypes.data, ws.nbytes, res.ctypes.data),
             (sl.ctypes.data, (1 << 24) + 1, nslots, ws.ctypes.data, ws.nbytes, res.ctypes.data),
             (sl.ctypes.data, 8, nslots, ws.ctypes.data + 2, ws.nbytes, res.ctypes.data),
             (0, 8, nslots, ws.ctypes.data, ws.nbytes, res.ctypes.data)):
    assert rejects(cs, *args) == ric.RIC_EINVAL, args
print("sanitized control plane ok", next_id, "corrections", corrections)
"""


def test_host_control_plane_under_asan_and_ubsan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime for gcc here")
    so = tmp_path / "libric_fake_device.so"
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "ragged_input_compilation_amd", "csrc", "ric_host.cpp"),
                    os.path.join(ROOT, "tests", "host_fake", "fake_device.cpp"), "-o", str(so)], check=True)
    preload = ":".join(x for x in (asan, os.environ.get("LD_PRELOAD", "")) if x)   # ASan first, nothing removed
    env = {**os.environ, "LD_PRELOAD": preload, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "RIC_LIBRARY": str(so)}
    child = subprocess.run([sys.executable, "-c", _CHILD.format(root=ROOT)], capture_output=True, text=True,
                           timeout=600, env=env)
    assert child.returncode == 0, child.stdout[-2000:] + child.stderr[-4000:]
    assert "sanitized control plane ok" in child.stdout
    assert int(child.stdout.split("corrections")[1]) > 10, child.stdout
    assert "AddressSanitizer" not in child.stderr and "runtime error" not in child.stderr
