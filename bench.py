#!/usr/bin/env python3
"""Benchmark of the ragged-input step on one MI355X.

One step = compile the persistent batch into the flat token stream and its
metadata (one kernel), write the step's K/V rows into the paged caches of every
layer (one kernel), gather the hidden rows that produce logits (one kernel).
Inputs (column store, K/V sources, hidden states) are resident in HBM before
the timed region.  Steps rotate over independently seeded instances of the
same configuration (different block tables, token histories and K/V sources),
so a step never finds the previous steps' bytes in the 256 MB Infinity Cache.

Prints one JSON line.  Extra fields: per-kernel times from HIP events, the
step's algorithmic bytes and GB/s, the rate including the host-to-device
upload of the step's counts, and the CPU oracle's rate (single thread)."""
import argparse
import ctypes
import hashlib
import json
import math
import mmap
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
KV_EVENT_EVERY = 8      # timed steps carrying events around the K/V launch: 1 in 8 (each pair perturbs its step)
METRIC = "scheduled tokens/sec per step (compile + KV write); achieved HBM GB/s vs peak"
DESCRIPTIONS = {
    "worked_example": "3 requests (prefill 7, decode 5+1, chunk 10..21), N=20 padded to 32, block 16, "
                      "f16 K/V 2x64, 1 layer",
    "decode_heavy": "256 single-token decodes, contexts U[128,4096], block 16, bf16 K/V 8x128, 32 layers",
    "mixed": "prefills 2000+512, two 2048-token chunk middles, 120 decodes (N=6728), block 16, "
             "bf16 K/V 8x128, 1 layer",
    "churn": "1024-row persistent batch after 10% churn + condense + refill, 960 decodes + 64 prefill "
             "chunks (N=16384), block 16, bf16 K/V 8x128, 1M-block pool, 1 layer",
    "long_context": "4 requests x 8192-token chunks of 131072-token prompts, cached prefix U[0,122880], "
                    "block 64, bf16 K/V 8x128, 1 layer, compacted hidden gather",
    "long_context_forced": "long_context with request 0 at its last chunk (one compacted gather row)",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="long_context", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--sets", type=int, default=0, help="rotation instances (0: enough for >= 1 GiB/cycle)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB copy (identity-index row gather) for counter scaling")
    return ap.parse_args()


def step_bytes(w):
    """Algorithmic bytes of one step (what the method must read and write;
    padding, over-fetch and cache-line granularity excluded)."""
    live = w.live_requests()
    R = len(live)
    N = sum(r.num_scheduled for r in live)
    B = w.block_size
    touched = sum(-(-(r.num_computed + r.num_scheduled) // B) - r.num_computed // B for r in live)
    compile_b = 12 * R + 4 * N + 4 * touched + 16 * N + 4 * (R + 1) + 4 * R + 4 * R + 4 * R + R
    kv_b = w.num_layers * (2 * N * w.row_bytes + 4 * N + 2 * N * w.row_bytes)
    if w.gather == "all":
        m = R
    else:
        m = sum(1 for r in live if r.num_computed + r.num_scheduled >= r.num_prompt)
    gather_b = 2 * m * w.hidden_size * 2 + 4 * m
    return dict(R=R, N=N, compile=compile_b, kv=kv_b, gather=gather_b, gather_rows=m,
                total=compile_b + kv_b + gather_b)


def kv_kernel_name(w, n_tokens):
    """Which K/V launch shape the library picks (mirrors its launcher: wave
    rows for <= 8192 tokens of 1/2/4 KiB rows, otherwise chunk tiles)."""
    cpl = w.row_bytes // 1024
    if w.row_bytes % 1024 == 0 and cpl in (1, 2, 4) and n_tokens <= 8192:
        return "kv_wave_kernel"
    return "kv_chunk_kernel"


def code_digest(text):
    """sha256 of C++ source with comments and whitespace removed, so that a
    comment edit keeps counter readings valid and any code edit voids them."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


def kernel_source_digest(text=None):
    """Digest of the K/V write's code: its load/store helpers, both kernels and
    their launcher (the source from the load helper up to the row-gather
    kernel), so that changes elsewhere in the file keep its counters valid.
    ``text``: the kernel source (default: the file in the package)."""
    if text is None:
        with open(os.path.join(ROOT, "ragged_input_compilation_amd", "csrc", "ric_kernels.hip"),
                  encoding="utf-8") as f:
            text = f.read()
    start, end = text.find("u32x4 load16("), text.find("gather_kernel(")
    if start < 0 or end <= start:
        raise ValueError("the K/V write's code is not where the digest expects it")
    return code_digest(text[start:end])


def load_traffic(kernel_name, workload_name):
    """HBM bytes per launch of the K/V kernel from the committed counter runs
    (profiles/<kernel>_<workload>_pmc.md), or None when there are none or they
    were taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_{workload_name}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    digest = re.search(r"^kernel_code_sha256: ([0-9a-f]{64})$", text, re.M)
    traffic = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    if not digest or not traffic or digest.group(1) != kernel_source_digest():
        return None
    return int(traffic.group(1))


class Event:
    """A HIP timing event created with hipEventDisableSystemFence.  Recording a
    default event (torch.cuda.Event) performs a system-scope release: the L2s
    are written back and invalidated, which lengthens the bracketed interval by
    1-2 us and slows the next kernel.  These events only timestamp.  They are
    recorded on `Event.stream` (the library's stream) through the HIP runtime
    that torch already loaded (the same library instance libric uses)."""
    DISABLE_SYSTEM_FENCE = 0x20000000
    stream = None
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            paths = [line.split()[-1] for line in open("/proc/self/maps") if "libamdhip64" in line]
            if not paths:
                raise RuntimeError("the HIP runtime is not loaded in this process")
            lib = ctypes.CDLL(paths[0])
            vp = ctypes.c_void_p
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [vp, vp]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            lib.hipEventDestroy.argtypes = [vp]
            cls._hip = lib
        return cls._hip

    def __init__(self):
        self.h = ctypes.c_void_p()
        if self._lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self._rec = self._hip.hipEventRecord
        self._st = ctypes.c_void_p(Event.stream or None)

    def record(self):
        if self._rec(self.h, self._st) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.h, end.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def __del__(self):
        if self.h and self._hip is not None:
            self._hip.hipEventDestroy(self.h)


class GpuStep:
    """Prebuilt library calls for one rotation instance."""

    def __init__(self, ric, runner, torch, w, kc, vc, hidden, out, seed):
        self.w = w
        self.batch = runner.Batch(runner.config_of(w))
        self.condense = self._history_with_timed_condense(ric, torch, w) if w.finished else None
        if not w.finished:
            self.batch.load_history(w)
        self.batch.schedule_from(w)
        live = w.live_requests()
        self.N = sum(r.num_scheduled for r in live)
        self.n_pad = ric.ric_padded_size(w.capture_sizes, self.N)
        self.step = ric.ric_compile(self.batch.h, self.n_pad)
        self.k, self.v = runner.alloc_sources(w, self.n_pad, seed=seed)
        L = w.num_layers
        P = ctypes.c_void_p * L
        self._ptrs = [P(*[t.data_ptr() for t in lst]) for lst in (self.k, self.v, kc, vc)]
        pp = ctypes.POINTER(ctypes.c_void_p)
        self.stream = runner.current_stream()
        st = ctypes.c_void_p(self.stream or None)
        lib = ric.lib()
        self.lib = lib
        self.kv_flags = 0
        self.kv_args = [ctypes.cast(a, pp) for a in self._ptrs] + [
            L, ctypes.c_void_p(self.step.slot_mapping), self.n_pad, 0, w.row_bytes,
            w.num_kv_blocks * w.block_size, None, self.kv_flags, st]
        row = w.hidden_size * 2
        if w.gather == "all":
            idx, cnt, rows = self.step.logits_indices, None, len(live)
        else:
            # the compacted rows; the host already knows how many there are (the
            # schedule's num_sampled), so a step where no request completes its
            # prompt launches no gather (the device count serves callers that
            # do not know it)
            idx, cnt, rows = self.step.sample_indices, None, self.step.num_sampled
        self.gather_rows = rows
        self.gather_args = [ctypes.c_void_p(hidden.data_ptr()), row, hidden.shape[0], ctypes.c_void_p(idx),
                            ctypes.c_void_p(cnt), rows, row, ctypes.c_void_p(out.data_ptr()), row, None, st]
        self.h = ctypes.c_void_p(self.batch.h)
        self.step_out = ric.ric_step()
        self.ric = ric

    def _check(self, rc):
        if rc != 0:
            raise RuntimeError(self.ric.ric_last_error())

    def _history_with_timed_condense(self, ric, torch, w):
        """The workload's history (adds, removals, condense, refills) with HIP
        events around the condense alone; returns its time, the rows it moved
        and their algorithmic bytes (each moved row reads and writes its token
        history, its block row and the 12 scalar columns)."""
        h = self.batch.h
        for r in w.initial:
            self.batch.add(r)
        for rid in w.finished:
            ric.ric_remove_request(h, rid)
        ric.ric_flush(h)
        by_row = [ric.ric_req_at(h, row) for row in range(w.max_num_reqs)]
        plan = ric.ric_condense_plan([x is not None for x in by_row])
        by_id = w.by_id()
        nbytes = sum(2 * (4 * len(by_id[by_row[src]].tokens) + 4 * len(by_id[by_row[src]].blocks) + 4 * 12)
                     for _, src in plan)
        torch.cuda.synchronize()
        a, b = Event(), Event()
        a.record()
        moved = ric.ric_condense(h)
        b.record()
        for r in w.refill:
            self.batch.add(r)
        ric.ric_flush(h)
        torch.cuda.synchronize()
        return dict(us=a.elapsed_time(b) * 1e3, rows_moved=moved, bytes=nbytes)

    def compile(self):
        self._check(self.lib.ric_compile(self.h, self.n_pad, ctypes.byref(self.step_out)))

    def kv(self):
        self._check(self.lib.ric_reshape_and_cache(*self.kv_args))

    def gather(self):
        self._check(self.lib.ric_gather_rows(*self.gather_args))

    def reschedule(self):
        """Host counts -> pinned staging (uploaded by the next compile)."""
        if not hasattr(self, "_sched"):          # the counts a scheduler would hand over, built once
            live_rows = self.batch.row_order()
            by_id = self.w.by_id()
            c = [by_id[i].num_computed for i in live_rows]
            q = [by_id[i].num_scheduled for i in live_rows]
            self._sched = [self.ric._i32(c), self.ric._i32(q)]
        (ca, cp), (qa, qp) = self._sched
        self._check(self.lib.ric_schedule(self.h, ca.shape[0], cp, qp))


def cpu_baseline(w, seconds):
    """The plain C oracle, single thread: compile + K/V scatter into mmap'd host
    caches of the full size + gather, repeated over the full step."""
    import numpy as np
    from oracle import batch as ref_batch, cbind
    from workloads import payload_numpy

    ref = ref_batch.RefBatch(w.max_num_reqs, w.max_model_len, w.max_blocks_per_req, w.num_kv_blocks)
    for r in w.initial:
        ref.add_request(r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks)
    for rid in w.finished:
        ref.remove_request(rid)
    ref.condense()
    for r in w.refill:
        ref.add_request(r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks)
    by_id = w.by_id()
    order = [rid for rid in ref.req_ids_by_row() if rid is not None]
    ref.schedule([by_id[i].num_computed for i in order], [by_id[i].num_scheduled for i in order])
    rows = ref.step_rows()
    N = sum(r.num_scheduled for r in rows)
    n_pad = N
    for s in sorted(w.capture_sizes):
        if s >= N:
            n_pad = s
            break
    tok, blk = cbind.pack_tables(rows)
    lib = cbind.lib()
    i32p = ctypes.POINTER(ctypes.c_int32)
    c = np.ascontiguousarray([r.num_computed for r in rows], np.int32)
    q = np.ascontiguousarray([r.num_scheduled for r in rows], np.int32)
    P = np.ascontiguousarray([r.num_prompt for r in rows], np.int32)
    MR = w.max_num_reqs
    outs = {k: np.zeros(n_pad, np.int32) for k in ("ids", "pos", "req", "slot")}
    per = {k: np.zeros(MR + 1, np.int32) for k in ("qsl", "cuk", "seq", "log", "smp")}
    disc = np.zeros(MR, np.uint8)
    p = lambda a: a.ctypes.data_as(i32p)
    ins = cbind._In(len(rows), w.block_size, MR, n_pad, 0, tok.shape[1], blk.shape[1], p(c), p(q), p(P),
                    p(tok), p(blk))
    out = cbind._Out(p(outs["ids"]), p(outs["pos"]), p(outs["req"]), p(outs["slot"]), p(per["qsl"]),
                     p(per["cuk"]), p(per["seq"]), p(per["log"]), disc.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)),
                     p(per["smp"]), 0, 0, 0, 0)
    rng = np.random.default_rng(w.seed + 99)
    L = w.num_layers
    row = w.row_bytes
    k_src = [payload_numpy(rng, (n_pad, row // 2), w.kv_dtype) for _ in range(L)]
    v_src = [payload_numpy(rng, (n_pad, row // 2), w.kv_dtype) for _ in range(L)]
    nslots = w.num_kv_blocks * w.block_size
    flags = mmap.MAP_PRIVATE | mmap.MAP_ANONYMOUS | getattr(mmap, "MAP_NORESERVE", 0x4000)
    maps = [mmap.mmap(-1, nslots * row, flags=flags) for _ in range(2 * L)]
    caches = [np.frombuffer(m, dtype=np.uint8) for m in maps]
    hidden = np.zeros((n_pad, w.hidden_size * 2), np.uint8)     # lazily mapped zero pages
    m_rows = MR
    gout = np.zeros((m_rows, w.hidden_size * 2), np.uint8)

    def one_step():
        if lib.nano_compile(ctypes.byref(ins), ctypes.byref(out)) != 0:
            raise RuntimeError("oracle rejected the step")
        for l in range(L):
            lib.nano_kv_scatter(k_src[l].ctypes.data, v_src[l].ctypes.data, caches[2 * l].ctypes.data,
                                caches[2 * l + 1].ctypes.data, p(outs["slot"]), n_pad, row)
        idx = per["log"] if w.gather == "all" else per["smp"]
        cnt = len(rows) if w.gather == "all" else out.num_sampled
        lib.nano_gather(hidden.ctypes.data, hidden.shape[1], p(idx), cnt, gout.ctypes.data)

    one_step()                     # pre-fault the touched cache pages
    reps, t0 = 0, time.perf_counter()
    while True:
        one_step()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 10000:
            break
    del caches
    for m in maps:
        m.close()
    return dict(value=N * reps / el, unit="tokens/s", cores=1, kind="oracle",
                host_cpu_count=os.cpu_count(), host_cpus_allowed=len(os.sched_getaffinity(0)),
                sample=f"{reps} full steps of the same configuration (seed instance 0) in {el:.1f} s; "
                       f"single-thread C oracle (nano-vllm block-range compile, memcpy K/V scatter into "
                       f"mmap'd full-size host caches, hidden-row gather)")


def kv_sources_cached(ric, torch, sets, nbytes, reps=20):
    """The K/V launch right after its sources were rewritten in place (x * 1
    by a torch kernel), so that they sit in the caches as they do when the
    write follows the K/V projection inside a model."""
    times = []
    for i in range(reps + 2):
        st = sets[i % len(sets)]
        for t in st.k + st.v:
            t.mul_(1)
        a, b = Event(), Event()
        a.record()
        st.kv()
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(b) for a, b in times[2:])[reps // 2] * 1e3
    gbps = nbytes / (us * 1e-6) / 1e9
    return dict(us=us, gbps=gbps, frac=gbps / HBM_PEAK_GBPS)


def copy_ceiling(ric, torch, sets, w, sb, reps=20):
    """What a plain copy of the K/V launch's bytes reaches on this GPU: torch's
    own device copy (half the bytes read, half written, rotating over buffers
    that together exceed 1 GiB), and the library's K/V launch with identity
    slots (each source row to consecutive cache rows; the faster of its two
    load variants)."""
    half = sb["kv"] // 2
    pairs = max(2, min(16, -(-(1 << 30) // (2 * half))))
    bufs = [(torch.empty(half, dtype=torch.uint8, device="cuda"), torch.empty(half, dtype=torch.uint8, device="cuda"))
            for _ in range(pairs)]
    for src, _ in bufs:
        src.fill_(1)
    times = []
    for i in range(reps + 2):
        src, dst = bufs[i % pairs]
        a, b = Event(), Event()
        a.record()
        dst.copy_(src)
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    t_torch = sorted(a.elapsed_time(b) for a, b in times[2:])[reps // 2]
    del bufs

    B, n_pad = w.block_size, sets[0].n_pad
    num_slots = w.num_kv_blocks * B
    slots = []
    for k, st in enumerate(sets):
        off = B + k * n_pad if B + (len(sets) + 1) * n_pad <= num_slots else B
        slots.append(torch.arange(off, off + n_pad, dtype=torch.int32, device="cuda"))
    times = []
    for i in range(reps + 2):
        k = i % len(sets)
        args = list(sets[k].kv_args)
        args[5] = ctypes.c_void_p(slots[k].data_ptr())
        a, b = Event(), Event()
        a.record()
        sets[k]._check(sets[k].lib.ric_reshape_and_cache(*args))
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    t_ident = sorted(a.elapsed_time(b) for a, b in times[2:])[reps // 2]
    return dict(bytes=sb["kv"], torch_copy_us=t_torch * 1e3, torch_copy_gbps=2 * half / (t_torch * 1e-3) / 1e9,
                identity_slots_us=t_ident * 1e3, identity_slots_gbps=sb["kv"] / (t_ident * 1e-3) / 1e9)


def next_rows(ric, runner, torch, w, st, reps=20):
    """Times of the calls beyond the step (untimed diagnostics, events around
    each call; a call that stages host data includes that host work): the
    dense padded block table, the speculative-decoding indices, the device-side
    append of sampled tokens, the device-side correction of optimistic computed
    counts, and the compile with a second KV-cache group that gets its own
    slots.  cu_seqlens_k is part of every compile."""
    import numpy as np
    median = lambda xs: sorted(xs)[len(xs) // 2]

    def timed(fn):
        pairs = []
        for _ in range(reps):
            a, b = Event(), Event()
            a.record()
            fn()
            b.record()
            pairs.append((a, b))
        torch.cuda.synchronize()
        return median([a.elapsed_time(b) for a, b in pairs]) * 1e3

    out = {}
    h = st.batch.h
    live = w.live_requests()
    by_id = w.by_id()
    order = st.batch.row_order()
    R = len(order)
    nb = [len(by_id[i].blocks) for i in order]
    width = max(nb)
    dst = torch.empty((R, width), dtype=torch.int32, device="cuda")
    us = timed(lambda: ric.ric_block_table_padded(h, width, -1, dst.data_ptr()))
    nbytes = 4 * R + 4 * sum(nb) + 4 * R * width
    out["padded_block_table"] = dict(rows=R, width=width, us=us, bytes=nbytes, gbps=nbytes / (us * 1e-6) / 1e9)

    q = [by_id[i].num_scheduled for i in order]
    d = [min(x - 1, 3) for x in q]
    m = ric.ric_spec_decode_metadata(h, d)
    us = timed(lambda: ric.ric_spec_decode_metadata(h, d))
    nbytes = 4 * R + 4 * (R + 1) + 4 * m.num_draft_tokens + 4 * m.num_logits + 4 * (R + 1) + \
        8 * m.num_draft_tokens + 4 * R
    out["spec_decode"] = dict(num_logits=m.num_logits, num_draft=m.num_draft_tokens, us_per_call=us, bytes=nbytes)

    b2 = runner.Batch(runner.config_of(w))
    b2.load_history(w)
    rows = [r for r, rid in enumerate(b2.row_order()) if len(by_id[rid].tokens) + reps + 2 <= w.max_model_len]
    if rows:
        sampled = torch.randint(0, 1 << 20, (len(rows),), dtype=torch.int32, device="cuda")
        src = list(reversed(range(len(rows))))
        us = timed(lambda: ric.ric_append_sampled(b2.h, rows, sampled.data_ptr(), len(rows), src))
        out["append_sampled"] = dict(rows=len(rows), us_per_call=us, bytes=20 * len(rows))
    else:
        out["append_sampled"] = dict(rows=0, skipped="no row has room left in its token history")
    b2.close()

    # a step whose scheduled counts are corrected on the device first (every
    # row verified min(c, 3) drafts, of which the sampler kept none but its
    # own token), against the same step without the correction
    b4 = runner.Batch(runner.config_of(w))
    b4.load_history(w)
    order4 = b4.row_order()
    # host arrays built once, as a runner keeps them, so the events time the
    # library's calls rather than Python list conversion
    c4 = np.asarray([by_id[i].num_computed for i in order4], np.int32)
    q4 = np.asarray([by_id[i].num_scheduled for i in order4], np.int32)
    d4 = np.minimum(c4, 3).astype(np.int32)
    accepted = torch.ones(R, dtype=torch.int32, device="cuda")
    kept = torch.randint(0, 1 << 20, (R, 4), dtype=torch.int32, device="cuda")
    rows4 = np.arange(R, dtype=np.int32)

    def corrected_step():
        ric.ric_schedule(b4.h, c4, q4)
        ric.ric_correct_computed(b4.h, rows4, rows4, d4, accepted.data_ptr(), R, kept.data_ptr(), 4)
        ric.ric_compile(b4.h, st.n_pad)

    def plain_step():
        ric.ric_schedule(b4.h, c4, q4)
        ric.ric_compile(b4.h, st.n_pad)

    corrected_step()
    us_corr, us_plain = timed(corrected_step), timed(plain_step)
    out["correct_computed"] = dict(rows=R, us_schedule_correct_compile=us_corr, us_schedule_compile=us_plain,
                                   added_us=us_corr - us_plain, bytes=24 * R)
    b4.close()

    # the compile with a second slotted group (the same block size and ids as
    # group 0), against a batch built the same way with one group
    us_by_groups = {}
    for groups in (1, 2):
        cfg = runner.config_of(w)
        cfg.num_kv_groups = groups
        cfg.group_block_size[1] = w.block_size
        b3 = runner.Batch(cfg)
        b3.load_history(w)
        if groups == 2:
            for rid in b3.row_order():
                ric.ric_append_blocks_group(b3.h, rid, 1, by_id[rid].blocks)
        b3.schedule_from(w)
        ric.ric_compile(b3.h, st.n_pad)
        us_by_groups[groups] = timed(lambda: ric.ric_compile(b3.h, st.n_pad))
        b3.close()
    N = sum(q)
    out["compile_two_kv_groups"] = dict(us=us_by_groups[2], us_one_group=us_by_groups[1], extra_bytes=4 * N + 4 * sum(
        -(-(r.num_computed + r.num_scheduled) // w.block_size) - r.num_computed // w.block_size for r in live))
    return out


def calibrate_copy(ric, torch, stream):
    """A plain copy of known size through the row-gather kernel with identity
    indices: 16384 rows of 16 KiB (256 MiB read, 256 MiB written)."""
    rows, row = 16384, 16384
    src = torch.empty((rows, row), dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    idx = torch.arange(rows, dtype=torch.int32, device="cuda")
    times = []
    for _ in range(5):
        a, b = Event(), Event()
        a.record()
        ric.ric_gather_rows(src.data_ptr(), row, rows, idx.data_ptr(), 0, rows, row, dst.data_ptr(), row, 0, stream)
        b.record()
        times.append((a, b))
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    ms = sorted(a.elapsed_time(b) for a, b in times)[len(times) // 2]
    return dict(bytes_read=rows * row, bytes_written=rows * row, ms=ms,
                gbps=2 * rows * row / (ms * 1e-3) / 1e9, grid=rows)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the step needs no "
              f"exchange between GPUs; under data parallelism each GPU compiles its own batch, under tensor "
              f"parallelism each runs the same compile and writes its own K/V heads, so the per-GPU figure is "
              f"the one to measure.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import workloads
    from ragged_input_compilation_amd import _ric as ric, runner

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    Event.stream = runner.current_stream()     # every library call below runs on this stream
    w0 = workloads.get(args.config)
    sb = step_bytes(w0)
    S = args.sets or max(2, min(16, math.ceil((1 << 30) / sb["total"])))
    t_setup = time.perf_counter()
    kc, vc = runner.alloc_caches(w0)
    g = torch.Generator(device="cuda")
    g.manual_seed(w0.seed + 5)
    n_pad0 = ric.ric_padded_size(w0.capture_sizes, sb["N"])
    hidden = torch.randn((n_pad0, w0.hidden_size), generator=g, device="cuda").to(torch.bfloat16)
    gout = torch.empty((w0.max_num_reqs, w0.hidden_size), dtype=torch.bfloat16, device="cuda")
    sets = []
    for k in range(S):
        w = w0 if k == 0 else workloads.get(args.config, variant=k)
        sets.append(GpuStep(ric, runner, torch, w, kc, vc, hidden, gout, seed=w.seed + 31))
        print(f"[bench] set {k + 1}/{S} ready", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    def event_pairs(n):
        return [(Event(), Event())
                for _ in range((n + KV_EVENT_EVERY - 1) // KV_EVENT_EVERY)]

    def run(n, mode, pool=None):
        """mode "none": no events; "kv": events around the K/V launch only (the
        timed region; `pool` holds the events, created beforehand since
        creating them costs host time); "all": events around each of the three
        kernels."""
        ev = []
        for i in range(n):
            st = sets[i % S]
            if mode == "none":
                st.compile()
                st.kv()
                st.gather()
            elif mode == "kv" and i % KV_EVENT_EVERY != 0:
                st.compile()
                st.kv()
                st.gather()
            elif mode == "kv":
                a, b = pool[i // KV_EVENT_EVERY]
                st.compile()
                a.record()
                st.kv()
                b.record()
                st.gather()
                ev.append((a, b))
            else:
                e = [Event() for _ in range(6)]
                e[0].record(); st.compile(); e[1].record()
                e[2].record(); st.kv(); e[3].record()
                e[4].record(); st.gather(); e[5].record()
                ev.append(e)
        return ev

    run(args.warmup, "none")
    pool = event_pairs(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev = run(args.steps, "kv", pool)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    mean = lambda xs: sum(xs) / len(xs)
    kv_mean = mean([a.elapsed_time(b) for a, b in ev])

    # Untimed diagnostics: the same steps with no events, then with events
    # around every kernel (compile and gather durations).
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    run(args.steps, "none")
    host_ms = (time.perf_counter() - t2) * 1e3 / args.steps     # enqueue only: the launches are asynchronous
    torch.cuda.synchronize()
    ms_no_events = (time.perf_counter() - t2) * 1e3 / args.steps
    evs = run(min(args.steps, 100), "all")
    torch.cuda.synchronize()
    comp_ms = [e[0].elapsed_time(e[1]) for e in evs]
    ga_ms = [e[4].elapsed_time(e[5]) for e in evs]

    # Same step with the counts uploaded from the host first (schedule + the
    # flush inside compile carry them over PCIe).
    for st in sets:                      # builds each instance's host count arrays once
        st.reschedule()
        st.compile()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_pcie = max(args.steps // 2, 1)
    for i in range(n_pcie):
        st = sets[i % S]
        st.reschedule()
        st.compile()
        st.kv()
        st.gather()
    torch.cuda.synchronize()
    pcie_ms = (time.perf_counter() - t1) * 1e3 / n_pcie

    # Cold caches: before each of 50 reps, a 1 GiB read (a sum) evicts the
    # Infinity Cache and the L2s without leaving dirty lines behind; events
    # then bracket compile + K/V (and the K/V launch alone).
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    median = lambda xs: sorted(xs)[len(xs) // 2]

    def bracketed(n, flush, with_compile):
        pairs = event_pairs(n * KV_EVENT_EVERY)
        for i in range(n):
            st = sets[i % S]
            if flush:
                flush_buf.sum()
            elif not with_compile:
                st.compile()
            a, b = pairs[i]
            a.record()
            if with_compile:
                st.compile()
            st.kv()
            b.record()
            st.gather()
        torch.cuda.synchronize()
        return median([a.elapsed_time(b) for a, b in pairs])

    kv_cold_ms = bracketed(20, True, False)
    ck_cold_ms = bracketed(50, True, True)
    ck_warm_ms = bracketed(50, False, True)
    del flush_buf
    ceiling = copy_ceiling(ric, torch, sets, w0, sb)
    cached = kv_sources_cached(ric, torch, sets, sb["kv"])
    nxt = next_rows(ric, runner, torch, w0, sets[0])

    calib = calibrate_copy(ric, torch, runner.current_stream()) if args.calibrate_copy else None

    N = sb["N"]
    achieved = sb["kv"] / (kv_mean * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {DESCRIPTIONS[args.config]}", "num_reqs": sb["R"],
                   "num_tokens": N, "num_layers": w0.num_layers, "rotation_instances": S},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": load_traffic(kv_kernel_name(w0, sets[0].n_pad), args.config),
                     "kernel": kv_kernel_name(w0, sets[0].n_pad), "kv_flags": sets[0].kv_flags,
                     "bytes_per_launch": sb["kv"],
                     "avg_launch_us": kv_mean * 1e3, "event_samples": len(ev),
                     "frac_of_copy_ceiling": achieved / max(ceiling["torch_copy_gbps"],
                                                            ceiling["identity_slots_gbps"])},
        "copy_ceiling": ceiling,
        "kv_sources_cached": cached,
        "compile_plus_kv": {"bytes": sb["compile"] + sb["kv"],
                            "warm_us": ck_warm_ms * 1e3,
                            "warm_frac_of_peak": (sb["compile"] + sb["kv"]) / (ck_warm_ms * 1e-3) / 1e9
                            / HBM_PEAK_GBPS,
                            "after_cache_flush_us": ck_cold_ms * 1e3,
                            "after_cache_flush_frac_of_peak": (sb["compile"] + sb["kv"]) / (ck_cold_ms * 1e-3)
                            / 1e9 / HBM_PEAK_GBPS},
        "step_bytes": sb["total"],
        "step_gbps": sb["total"] / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_peak": sb["total"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "ms_per_step_without_events": ms_no_events,
        "host_enqueue_us_per_step": host_ms * 1e3,
        "kernels_us": {"compile": mean(comp_ms) * 1e3, "kv_scatter": kv_mean * 1e3,
                       "gather": mean(ga_ms) * 1e3 if sets[0].gather_rows else None,
                       "kv_scatter_after_cache_flush": kv_cold_ms * 1e3},
        "pcie_inclusive_tokens_per_s": N / (pcie_ms * 1e-3),
        "next_rows": nxt,
        "condense": ({"us_with_host_planning_and_pair_upload": mean([st.condense["us"] for st in sets]),
                      "rows_moved": sets[0].condense["rows_moved"], "bytes": sets[0].condense["bytes"],
                      "instances": S} if sets[0].condense else None),
        "setup_s": setup_s,
    }
    if calib:
        res["copy_calibration"] = calib
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w0, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
