#!/usr/bin/env python3
"""Benchmark of the ragged-input step on one MI355X.

One step = compile the persistent batch into the flat token stream and its
metadata and write the step's K/V rows into the paged caches of every layer
(one library call, ric_compile_and_cache: a single kernel, or the compile and
the K/V kernel for steps of long chunks and rows that kernel does not take),
then gather the hidden
rows that produce logits.  Inputs (column store, K/V sources, hidden states)
are resident in HBM before the timed region.  Steps rotate over independently
seeded instances of the same configuration (different block tables, token
histories and K/V sources), so a step never finds the previous steps' bytes in
the 256 MB Infinity Cache.

Prints one JSON line: the headline configuration's tokens/s and roofline,
compile + K/V times of both library paths, the other configurations measured
the same way (``configs``), and the CPU oracle's rate on one core and on all
cores."""
import argparse
import ctypes
import hashlib
import json
import math
import mmap
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
EVENT_EVERY = 8         # roofline pass: events around the dominant kernel of 1 step in 8
MIN_EVENT_SAMPLES = 24  # at least this many bracketed launches, whatever --steps is
FUSE_ALWAYS, FUSE_NEVER = 1, 2
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
    "long_context_tp8": "long_context as one rank of 8-way tensor parallelism sees it: one K/V head of 128 "
                        "(256-byte rows), same schedule",
}
EXTRA_CONFIGS = ["worked_example", "decode_heavy", "mixed", "churn", "long_context", "long_context_tp8"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="long_context", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--sets", type=int, default=0, help="rotation instances (0: enough for >= 1 GiB/cycle)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU-oracle samples")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="measure only --config (default: also the other configurations, in `configs`)")
    ap.add_argument("--no-diagnostics", action="store_true",
                    help="skip the copy ceiling, cached-sources, next-row and cold-cache figures")
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
    """Which K/V launch shape the library picks for the separate K/V kernel
    (mirrors its launcher: wave rows for <= 8192 tokens of 1/2/4 KiB rows,
    otherwise chunk tiles)."""
    cpl = w.row_bytes // 1024
    if w.row_bytes % 1024 == 0 and cpl in (1, 2, 4) and n_tokens <= 8192:
        return "kv_wave_kernel"
    return "kv_chunk_kernel"


def fused_path(w):
    """Whether ric_compile_and_cache takes the single kernel for this step by
    the library's own choice (mirrors its rule: rows of 128, 256 or 512 B, or
    rows of 1, 2, 3, 4, 6 or 8 KiB with fewer than 1024 scheduled tokens per request
    on average)."""
    live = w.live_requests()
    N = sum(r.num_scheduled for r in live)
    if w.row_bytes in (128, 256, 512):
        return True
    return w.row_bytes in (1024, 2048, 3072, 4096, 6144, 8192) and N < 1024 * max(len(live), 1)


def dominant_kernel(w, n_pad, fused=None):
    """The step's dominant kernel: the single compile + K/V kernel when the
    library takes it (`fused`; default: the mirror of its rule), else the
    separate K/V kernel."""
    fused = fused_path(w) if fused is None else fused
    return "compile_kv_kernel" if fused else kv_kernel_name(w, n_pad)


def library_takes_single_kernel(st, w):
    """Whether ric_compile_and_cache took the single kernel for this step by
    its own choice, as the call reports it (ric_step.kv_path); the bench's
    mirror of the rule must agree."""
    st.compile_kv(0)
    fused = int(st.step_out.kv_path) == 1
    if fused != fused_path(w):
        raise RuntimeError(f"{w.name}: the library took kv_path {int(st.step_out.kv_path)}, the bench's mirror "
                           f"of its rule expected {'1' if fused_path(w) else '2'}")
    return fused


def code_digest(text):
    """sha256 of C++ source with comments and whitespace removed, so that a
    comment edit keeps counter readings valid and any code edit voids them."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return hashlib.sha256(" ".join(text.split()).encode()).hexdigest()


# Source regions whose code a kernel's counters depend on: the K/V kernels
# (load/store helpers, both shapes, their launcher); the compile kernel (its
# scan, per-token and per-request parts); the single compile + K/V kernel
# (all of the above and its own code).
DIGEST_REGIONS = {
    "kv": ("u32x4 load16(", "// Compile and K/V write in one launch."),
    "compile": ("int wave_inclusive_scan(", "hipError_t launch_compile("),
    "compile_kv": ("int wave_inclusive_scan(", "gather_kernel("),
}
KERNEL_REGION = {"kv_chunk_kernel": "kv", "kv_wave_kernel": "kv", "compile_kernel": "compile",
                 "compile_kv_kernel": "compile_kv"}


def kernel_source_digest(text=None, region="kv"):
    """Digest of one region of the kernel source (DIGEST_REGIONS), so that
    changes elsewhere in the file keep that kernel's counters valid.
    ``text``: the kernel source (default: the file in the package)."""
    if text is None:
        with open(os.path.join(ROOT, "ragged_input_compilation_amd", "csrc", "ric_kernels.hip"),
                  encoding="utf-8") as f:
            text = f.read()
    a, b = DIGEST_REGIONS[region]
    start, end = text.find(a), text.find(b)
    if start < 0 or end <= start:
        raise ValueError(f"the {region} code is not where the digest expects it")
    return code_digest(text[start:end])


def load_traffic(kernel_name, workload_name):
    """HBM bytes per launch of a kernel from the committed counter runs
    (profiles/<kernel>_<workload>_pmc.md), or None when there are none or they
    were taken on another version of the kernel's source."""
    path = os.path.join(ROOT, "profiles", f"{kernel_name}_{workload_name}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    digest = re.search(r"^kernel_code_sha256: ([0-9a-f]{64})$", text, re.M)
    traffic = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
    region = KERNEL_REGION.get(kernel_name, "kv")
    if not digest or not traffic or digest.group(1) != kernel_source_digest(region=region):
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
        # ric_compile_and_cache with the same K/V arguments (flags last but one)
        self.ck_args = [self.h, self.n_pad] + self.kv_args[:5] + [
            0, w.row_bytes, w.num_kv_blocks * w.block_size, None, 0, ctypes.byref(self.step_out)]

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

    def compile_kv(self, flags=0):
        """Compile + K/V write of every layer in one library call; flags 0 is
        the library's own choice of path."""
        self.ck_args[-2] = flags
        self._check(self.lib.ric_compile_and_cache(*self.ck_args))

    def kv(self):
        self._check(self.lib.ric_reshape_and_cache(*self.kv_args))

    def whole_step(self):
        """One whole step: compile + K/V (the library's path), gather."""
        self.compile_kv()
        self.gather()

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


class _CpuStep:
    """The step on the host with the plain C oracle: the compile (nano-vllm
    block-range formulation), a memcpy K/V scatter into mmap'd host caches of
    the full size (touched pages pre-faulted) and the hidden-row gather."""

    def __init__(self, w):
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
        self.np, self.cbind, self.w = np, cbind, w
        self.R = len(rows)
        self.N = sum(r.num_scheduled for r in rows)
        self.n_pad = self.N
        for sz in sorted(w.capture_sizes):
            if sz >= self.N:
                self.n_pad = sz
                break
        self.tok, self.blk = cbind.pack_tables(rows)
        self.lib = cbind.lib()
        self.c = np.ascontiguousarray([r.num_computed for r in rows], np.int32)
        self.q = np.ascontiguousarray([r.num_scheduled for r in rows], np.int32)
        self.P = np.ascontiguousarray([r.num_prompt for r in rows], np.int32)
        MR = w.max_num_reqs
        self.outs = {k: np.zeros(self.n_pad, np.int32) for k in ("ids", "pos", "req", "slot")}
        self.per = {k: np.zeros(MR + 1, np.int32) for k in ("qsl", "cuk", "seq", "log", "smp")}
        self.disc = np.zeros(MR, np.uint8)
        rng = np.random.default_rng(w.seed + 99)
        self.row = w.row_bytes
        self.k_src = [payload_numpy(rng, (self.n_pad, self.row // 2), w.kv_dtype) for _ in range(w.num_layers)]
        self.v_src = [payload_numpy(rng, (self.n_pad, self.row // 2), w.kv_dtype) for _ in range(w.num_layers)]
        nslots = w.num_kv_blocks * w.block_size
        flags = mmap.MAP_PRIVATE | mmap.MAP_ANONYMOUS | getattr(mmap, "MAP_NORESERVE", 0x4000)
        self.maps = [mmap.mmap(-1, nslots * self.row, flags=flags) for _ in range(2 * w.num_layers)]
        self.caches = [np.frombuffer(m, dtype=np.uint8) for m in self.maps]
        self.hidden = np.zeros((self.n_pad, w.hidden_size * 2), np.uint8)     # lazily mapped zero pages
        self.gout = np.zeros((MR, w.hidden_size * 2), np.uint8)
        self.i32p = ctypes.POINTER(ctypes.c_int32)
        p = self.p
        self.ins = cbind._In(self.R, w.block_size, MR, self.n_pad, 0, self.tok.shape[1], self.blk.shape[1],
                             p(self.c), p(self.q), p(self.P), p(self.tok), p(self.blk))
        self.out = cbind._Out(p(self.outs["ids"]), p(self.outs["pos"]), p(self.outs["req"]), p(self.outs["slot"]),
                              p(self.per["qsl"]), p(self.per["cuk"]), p(self.per["seq"]), p(self.per["log"]),
                              self.disc.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)), p(self.per["smp"]),
                              0, 0, 0, 0)

    def p(self, a, off=0):
        return ctypes.cast(a.ctypes.data + 4 * off, self.i32p)

    def close(self):
        self.caches = None
        for m in self.maps:
            m.close()

    def gather(self):
        w = self.w
        idx = self.per["log"] if w.gather == "all" else self.per["smp"]
        cnt = self.R if w.gather == "all" else self.out.num_sampled
        self.lib.nano_gather(self.hidden.ctypes.data, self.hidden.shape[1], self.p(idx), cnt, self.gout.ctypes.data)

    def scatter(self, t0, t1):
        row = self.row
        for l in range(self.w.num_layers):
            self.lib.nano_kv_scatter(self.k_src[l].ctypes.data + t0 * row, self.v_src[l].ctypes.data + t0 * row,
                                     self.caches[2 * l].ctypes.data, self.caches[2 * l + 1].ctypes.data,
                                     self.p(self.outs["slot"], t0), t1 - t0, row)

    def single(self):
        """The whole step on one thread."""
        if self.lib.nano_compile(ctypes.byref(self.ins), ctypes.byref(self.out)) != 0:
            raise RuntimeError("oracle rejected the step")
        self.scatter(0, self.n_pad)
        self.gather()


class _CpuParallel:
    """The same step on a pool of threads, in two phases: thread k < R
    compiles one contiguous range of requests (balanced by scheduled tokens)
    as a batch of its own and shifts its range's request-relative outputs into
    place; after a barrier every thread of the pool writes the K/V rows of
    one contiguous range of tokens (the bulk of the work, independent of the
    request count); the main thread then fills in the running totals across
    ranges, the compacted sample list, the padding and the gather.  The C
    calls release the interpreter lock."""

    def __init__(self, cs, threads):
        np = cs.np
        self.cs = cs
        cu = np.concatenate([[0], np.cumsum(cs.q, dtype=np.int64)])
        T = max(1, min(threads, cs.R))
        cuts = [0] + [int(np.searchsorted(cu, cs.N * k / T, side="left")) for k in range(1, T)] + [cs.R]
        self.ranges = [(a, b, int(cu[a]), int(cu[b])) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
        self.locals = []
        w = cs.w
        for r0, r1, t0, t1 in self.ranges:
            n = r1 - r0
            loc = {k: np.zeros(n + 1, np.int32) for k in ("qsl", "cuk", "log", "smp")}
            p = cs.p
            ins = cs.cbind._In(n, w.block_size, n, t1 - t0, 0, cs.tok.shape[1], cs.blk.shape[1], p(cs.c, r0),
                               p(cs.q, r0), p(cs.P, r0), p(cs.tok, r0 * cs.tok.shape[1]),
                               p(cs.blk, r0 * cs.blk.shape[1]))
            out = cs.cbind._Out(p(cs.outs["ids"], t0), p(cs.outs["pos"], t0), p(cs.outs["req"], t0),
                                p(cs.outs["slot"], t0), p(loc["qsl"]), p(loc["cuk"]), p(cs.per["seq"], r0),
                                p(loc["log"]),
                                ctypes.cast(cs.disc.ctypes.data + r0, ctypes.POINTER(ctypes.c_uint8)),
                                p(loc["smp"]), 0, 0, 0, 0)
            self.locals.append((loc, ins, out))
        self.threads_used = max(1, threads)
        self.compile_threads = len(self.ranges)
        P = self.threads_used
        self.tranges = [(cs.N * k // P, cs.N * (k + 1) // P) for k in range(P)]
        self.start = threading.Barrier(P + 1)
        self.mid = threading.Barrier(P)
        self.done = threading.Barrier(P + 1)
        self.stop = False
        self.workers = [threading.Thread(target=self._work, args=(k,), daemon=True) for k in range(P)]
        for t in self.workers:
            t.start()

    def _work(self, k):
        cs = self.cs
        while True:
            self.start.wait()
            if self.stop:
                return
            if k < self.compile_threads:
                r0, r1, t0, t1 = self.ranges[k]
                loc, ins, out = self.locals[k]
                if cs.lib.nano_compile(ctypes.byref(ins), ctypes.byref(out)) != 0:
                    raise RuntimeError("oracle rejected a range")
                cs.outs["req"][t0:t1] += r0
                cs.per["qsl"][r0 + 1:r1 + 1] = loc["qsl"][1:] + t0
                cs.per["log"][r0:r1] = loc["log"][:r1 - r0] + t0
            self.mid.wait()
            a, b = self.tranges[k]
            if b > a:
                cs.scatter(a, b)
            self.done.wait()

    def step(self):
        cs, np = self.cs, self.cs.np
        self.start.wait()
        self.done.wait()
        R, N, MR = cs.R, cs.N, cs.w.max_num_reqs
        per = cs.per
        base = 0
        for (r0, r1, t0, t1), (loc, _, _) in zip(self.ranges, self.locals):
            per["cuk"][r0 + 1:r1 + 1] = loc["cuk"][1:r1 - r0 + 1] + base
            base += int(loc["cuk"][r1 - r0])
        per["qsl"][0] = per["cuk"][0] = 0
        per["qsl"][R + 1:] = N
        per["cuk"][R + 1:] = base
        per["seq"][R:MR] = 0
        per["log"][R:MR] = -1
        cs.disc[R:MR] = 1
        keep = per["log"][:R][cs.disc[:R] == 0]
        per["smp"][:keep.shape[0]] = keep
        per["smp"][keep.shape[0]:MR] = -1
        cs.out.num_sampled = int(keep.shape[0])
        o = cs.outs
        o["ids"][N:] = 0
        o["pos"][N:] = 0
        o["req"][N:] = -1
        o["slot"][N:] = cs.w.null_block * cs.w.block_size
        if N < cs.n_pad:
            cs.scatter(N, cs.n_pad)
        cs.gather()

    def close(self):
        self.stop = True
        self.start.wait()
        for t in self.workers:
            t.join()


def _median_rate(fn, tokens, seconds, blocks=5):
    """Median over `blocks` timed blocks of the scheduled tokens per second,
    each block running whole steps for about seconds / blocks."""
    rates, steps = [], 0
    for _ in range(blocks):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds / blocks or n >= 5000:
                break
        rates.append(tokens * n / el)
        steps += n
    return sorted(rates)[blocks // 2], steps


def cpu_baseline(w, seconds):
    """The plain C oracle timed on this host: one thread, then the per-request
    parallel split on every core this process may use.  Each is the median of
    5 timed blocks of whole steps; the parallel step's outputs are checked
    against the single-thread step's before timing."""
    cs = _CpuStep(w)
    cs.single()                    # pre-fault the touched cache pages
    want = {k: v.copy() for k, v in cs.outs.items()}
    want.update({k: v.copy() for k, v in cs.per.items()})
    want_disc = cs.disc.copy()
    # the cores this process may use, at most the host share a thread pool
    # should take (OMP_NUM_THREADS when set)
    allowed = len(os.sched_getaffinity(0))
    allowed = max(1, min(allowed, int(os.environ.get("OMP_NUM_THREADS") or allowed)))
    one, n1 = _median_rate(cs.single, cs.N, seconds / 2)
    par = _CpuParallel(cs, allowed)
    for d in list(cs.outs.values()) + list(cs.per.values()):
        d.fill(-9)
    par.step()
    got = dict(cs.outs, **cs.per)
    R, MR = cs.R, w.max_num_reqs
    for k in ("ids", "pos", "req", "slot"):
        assert (got[k] == want[k]).all(), f"parallel CPU step differs in {k}"
    for k in ("qsl", "cuk"):
        assert (got[k][:MR + 1] == want[k][:MR + 1]).all(), f"parallel CPU step differs in {k}"
    for k in ("seq", "log", "smp"):
        assert (got[k][:MR] == want[k][:MR]).all(), f"parallel CPU step differs in {k}"
    assert (cs.disc == want_disc).all()
    many, n2 = _median_rate(par.step, cs.N, seconds / 2)
    par.close()
    cs.close()
    return dict(value=one, unit="tokens/s", cores=1, kind="oracle", host_cpu_count=os.cpu_count(),
                host_cpus_allowed=allowed,
                sample=f"median of 5 blocks of whole steps of the same configuration (seed instance 0), "
                       f"{n1} steps in {seconds / 2:.0f} s; single-thread C oracle (nano-vllm block-range "
                       f"compile, memcpy K/V scatter into mmap'd full-size host caches, hidden-row gather)",
                all_cores=dict(value=many, unit="tokens/s", cores=par.threads_used, pool=allowed,
                               compile_threads=par.compile_threads,
                               sample=f"median of 5 blocks, {n2} steps in {seconds / 2:.0f} s; the same oracle "
                                      f"on {par.threads_used} threads: the compile split into "
                                      f"{par.compile_threads} contiguous ranges of requests (balanced by scheduled "
                                      f"tokens; never more ranges than requests), then the K/V rows split into "
                                      f"{par.threads_used} contiguous ranges of tokens"))


def kv_sources_cached(ric, torch, sets, nbytes, reps=20):
    """Compile + K/V (the library's path) right after the K/V sources were
    rewritten in place (x * 1 by a torch kernel), so that they sit in the
    caches as they do when the write follows the K/V projection inside a
    model."""
    times = []
    for i in range(reps + 2):
        st = sets[i % len(sets)]
        for t in st.k + st.v:
            t.mul_(1)
        a, b = Event(), Event()
        a.record()
        st.compile_kv()
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

    # host arrays built once, as a runner keeps them, so the events time the
    # library's calls rather than Python list conversion
    q = [by_id[i].num_scheduled for i in order]
    d = np.asarray([min(x - 1, 3) for x in q], np.int32)
    m = ric.ric_spec_decode_metadata(h, d)
    us = timed(lambda: ric.ric_spec_decode_metadata(h, d))
    nbytes = 4 * R + 4 * (R + 1) + 4 * m.num_draft_tokens + 4 * m.num_logits + 4 * (R + 1) + \
        8 * m.num_draft_tokens + 4 * R
    out["spec_decode"] = dict(num_logits=m.num_logits, num_draft=m.num_draft_tokens, us_per_call=us, bytes=nbytes)

    b2 = runner.Batch(runner.config_of(w))
    b2.load_history(w)
    rows = np.asarray([r for r, rid in enumerate(b2.row_order())
                       if len(by_id[rid].tokens) + reps + 2 <= w.max_model_len], np.int32)
    if len(rows):
        sampled = torch.randint(0, 1 << 20, (len(rows),), dtype=torch.int32, device="cuda")
        src = np.arange(len(rows) - 1, -1, -1, dtype=np.int32)
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


def build_sets(ric, runner, torch, workloads, name, nsets=0):
    """Rotation instances of one configuration (enough that a cycle moves
    >= 1 GiB unless `nsets` is given), sharing one set of caches, hidden rows
    and gather output."""
    w0 = workloads.get(name)
    sb = step_bytes(w0)
    S = nsets or max(2, min(16, math.ceil((1 << 30) / sb["total"])))
    kc, vc = runner.alloc_caches(w0)
    g = torch.Generator(device="cuda")
    g.manual_seed(w0.seed + 5)
    n_pad0 = ric.ric_padded_size(w0.capture_sizes, sb["N"])
    hidden = torch.randn((n_pad0, w0.hidden_size), generator=g, device="cuda").to(torch.bfloat16)
    gout = torch.empty((w0.max_num_reqs, w0.hidden_size), dtype=torch.bfloat16, device="cuda")
    sets = []
    for k in range(S):
        w = w0 if k == 0 else workloads.get(name, variant=k)
        sets.append(GpuStep(ric, runner, torch, w, kc, vc, hidden, gout, seed=w.seed + 31))
        print(f"[bench] {name}: set {k + 1}/{S} ready", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    return w0, sb, sets


def release(torch, sets):
    for st in sets:
        st.batch.close()
    sets.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def timed_steps(torch, sets, steps, warmup):
    """Wall-clock ms per step of `steps` whole steps after `warmup` untimed
    ones, bracketed by device synchronisation on both sides."""
    for i in range(warmup):
        sets[i % len(sets)].whole_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        sets[i % len(sets)].whole_step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def bracketed(torch, sets, before, body, after, reps, flush_buf=None):
    """Median ms of `body(st)` between two events over `reps` rotating steps;
    `before` / `after` run outside the events (the rest of the step), and a
    1 GiB read evicts the caches before each rep when flush_buf is given."""
    pairs = [(Event(), Event()) for _ in range(reps)]
    for i in range(reps):
        st = sets[i % len(sets)]
        if flush_buf is not None:
            flush_buf.sum()
        before(st)
        a, b = pairs[i]
        a.record()
        body(st)
        b.record()
        after(st)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in pairs)[reps // 2]


def compile_kv_paths(torch, sets, sb, reps, cold_reps, flush_buf):
    """Compile + K/V write of every layer through ric_compile_and_cache, for
    the library's own choice of path and for each path forced: events around
    the call (warm: back to back, rotating instances; after flush: a 1 GiB
    read first), gather outside."""
    nbytes = sb["compile"] + sb["kv"]
    out = {"bytes": nbytes}
    nothing = lambda st: None
    for name, flags in (("auto", 0), ("single_kernel", FUSE_ALWAYS), ("two_kernels", FUSE_NEVER)):
        for st in sets:
            st.compile_kv(flags)
        body = lambda st, f=flags: st.compile_kv(f)
        gather = lambda st: st.gather()
        warm = bracketed(torch, sets, nothing, body, gather, reps)
        cold = bracketed(torch, sets, nothing, body, gather, cold_reps, flush_buf)
        sustained = sustained_steps(torch, sets, flags)
        out[name] = {"warm_us": warm * 1e3, "warm_frac_of_peak": nbytes / (warm * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "after_cache_flush_us": cold * 1e3,
                     "after_cache_flush_frac_of_peak": nbytes / (cold * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                     "sustained_step_us": sustained * 1e3}
    return out


def sustained_steps(torch, sets, flags, steps=200):
    """Wall-clock ms per step of `steps` back-to-back rotating steps (compile +
    K/V through the given path, then the gather), bracketed by device
    synchronisation: the steady rate, where per-call events can favour a
    kernel that benefits from following itself."""
    for i in range(10):
        sets[i % len(sets)].compile_kv(flags)
        sets[i % len(sets)].gather()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        st = sets[i % len(sets)]
        st.compile_kv(flags)
        st.gather()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def extra_config(ric, runner, torch, workloads, name, steps, warmup, with_next_rows=False):
    """Another configuration measured the same way as the headline (fewer
    diagnostics): whole-step tokens/s, and compile + K/V by both paths; with
    `with_next_rows`, also the calls beyond the step (next_rows)."""
    t0 = time.perf_counter()
    w0, sb, sets = build_sets(ric, runner, torch, workloads, name)
    ms = timed_steps(torch, sets, steps, warmup)
    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    ck = compile_kv_paths(torch, sets, sb, 30, 10, flush_buf)
    del flush_buf
    fused = library_takes_single_kernel(sets[0], w0)
    path = "single_kernel" if fused else "two_kernels"
    kernel = dominant_kernel(w0, sets[0].n_pad, fused)
    res = {"workload": f"{name}: {DESCRIPTIONS[name]}", "num_reqs": sb["R"], "num_tokens": sb["N"],
           "num_layers": w0.num_layers, "tokens_per_s": sb["N"] / (ms * 1e-3), "ms_per_step": ms,
           "step_bytes": sb["total"], "library_path": path, "compile_plus_kv": ck,
           "dominant_kernel": kernel, "dominant_kernel_traffic": load_traffic(kernel, name),
           "rotation_instances": len(sets), "seconds": None}
    # a plain copy of this step's K/V bytes on the same GPU, and how compile +
    # K/V (the library's path, warm) compares with it
    cc = copy_ceiling(ric, torch, sets, w0, sb)
    fastest = min(cc["torch_copy_us"], cc["identity_slots_us"])
    cc["compile_plus_kv_over_copy"] = ck["auto"]["warm_us"] / fastest
    res["copy_ceiling"] = cc
    if sets[0].gather_rows:
        # the gather alone (events around it, rotating instances): M rows of
        # hidden states read and written, plus the M indices
        ga = bracketed(torch, sets, lambda st: None, lambda st: st.gather(), lambda st: None, 30) * 1e3
        gb = sb["gather"]
        res["gather"] = {"rows": sets[0].gather_rows, "us": ga, "bytes": gb, "gbps": gb / (ga * 1e-6) / 1e9}
    if with_next_rows and name != "worked_example":
        res["next_rows"] = next_rows(ric, runner, torch, w0, sets[0])
    release(torch, sets)
    res["seconds"] = time.perf_counter() - t0
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}): the step needs no "
              f"exchange between GPUs; under data parallelism each GPU compiles its own batch, under tensor "
              f"parallelism each runs the same compile and writes its own K/V heads, so the per-GPU figure is "
              f"the one to measure.", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads
    from ragged_input_compilation_amd import _ric as ric, runner

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    Event.stream = runner.current_stream()     # every library call below runs on this stream
    t_setup = time.perf_counter()
    w0, sb, sets = build_sets(ric, runner, torch, workloads, args.config, args.sets)
    S = len(sets)
    setup_s = time.perf_counter() - t_setup
    fused = library_takes_single_kernel(sets[0], w0)
    kernel = dominant_kernel(w0, sets[0].n_pad, fused)

    # The timed region: whole steps, no events.
    ms_per_step = timed_steps(torch, sets, args.steps, args.warmup)

    # Roofline pass: the same steps, with events around the dominant kernel
    # of one step in EVENT_EVERY, at least MIN_EVENT_SAMPLES of them.
    n_roof = max(args.steps, MIN_EVENT_SAMPLES * EVENT_EVERY)
    pairs = [(Event(), Event()) for _ in range(-(-n_roof // EVENT_EVERY))]
    for i in range(n_roof):
        st = sets[i % S]
        if i % EVENT_EVERY:
            st.whole_step()
            continue
        a, b = pairs[i // EVENT_EVERY]
        if fused:
            a.record(); st.compile_kv(); b.record()
        else:
            st.compile(); a.record(); st.kv(); b.record()
        st.gather()
    torch.cuda.synchronize()
    dom_ms = sum(a.elapsed_time(b) for a, b in pairs) / len(pairs)
    dom_bytes = sb["compile"] + sb["kv"] if fused else sb["kv"]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9

    flush_buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    ck = compile_kv_paths(torch, sets, sb, 50, 30, flush_buf)
    nothing = lambda st: None
    comp_ms = bracketed(torch, sets, nothing, lambda st: st.compile(), lambda st: (st.kv(), st.gather()), 50)
    kv_ms = bracketed(torch, sets, lambda st: st.compile(), lambda st: st.kv(), lambda st: st.gather(), 50)
    kv_cold_ms = bracketed(torch, sets, lambda st: st.compile(), lambda st: st.kv(), lambda st: st.gather(), 20,
                           flush_buf)
    ga_ms = bracketed(torch, sets, lambda st: st.compile_kv(), lambda st: st.gather(), nothing, 50) \
        if sets[0].gather_rows else None
    del flush_buf

    diag = {}
    if not args.no_diagnostics:
        # host enqueue cost of a step, and the step with its counts uploaded
        # from the host first (schedule + the flush inside the compile)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(args.steps):
            sets[i % S].whole_step()
        diag["host_enqueue_us_per_step"] = (time.perf_counter() - t2) * 1e6 / args.steps
        torch.cuda.synchronize()
        for st in sets:
            st.reschedule()
            st.compile_kv()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        n_pcie = max(args.steps // 2, 1)
        for i in range(n_pcie):
            st = sets[i % S]
            st.reschedule()
            st.whole_step()
        torch.cuda.synchronize()
        diag["pcie_inclusive_tokens_per_s"] = sb["N"] / ((time.perf_counter() - t1) / n_pcie)
        diag["copy_ceiling"] = copy_ceiling(ric, torch, sets, w0, sb)
        diag["kv_sources_cached"] = kv_sources_cached(ric, torch, sets, sb["compile"] + sb["kv"])
        diag["next_rows"] = next_rows(ric, runner, torch, w0, sets[0])
    calib = calibrate_copy(ric, torch, runner.current_stream()) if args.calibrate_copy else None
    condense = ({"us_with_host_planning_and_pair_upload": sum(st.condense["us"] for st in sets) / S,
                 "rows_moved": sets[0].condense["rows_moved"], "bytes": sets[0].condense["bytes"],
                 "instances": S} if sets[0].condense else None)
    release(torch, sets)

    configs = {}
    if not args.no_extra_configs:
        for name in EXTRA_CONFIGS:
            if name != args.config:
                configs[name] = extra_config(ric, runner, torch, workloads, name, max(args.steps, 50),
                                             max(args.warmup, 10), with_next_rows=not args.no_diagnostics)

    N = sb["N"]
    ceiling = diag.get("copy_ceiling")
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
                   "num_tokens": N, "num_layers": w0.num_layers, "rotation_instances": S,
                   "library_path": "single_kernel" if fused else "two_kernels"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": load_traffic(kernel, args.config),
                     "kernel": kernel, "bytes_per_launch": dom_bytes, "avg_launch_us": dom_ms * 1e3,
                     "event_samples": len(pairs),
                     "frac_of_copy_ceiling": (achieved / max(ceiling["torch_copy_gbps"], ceiling["identity_slots_gbps"])
                                              if ceiling else None)},
        "compile_plus_kv": ck,
        "kernels_us": {"compile": comp_ms * 1e3, "kv_scatter": kv_ms * 1e3,
                       "kv_scatter_after_cache_flush": kv_cold_ms * 1e3,
                       "gather": ga_ms * 1e3 if ga_ms is not None else None},
        "step_bytes": sb["total"],
        "step_gbps": sb["total"] / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_peak": sb["total"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "condense": condense,
        "setup_s": setup_s,
        "configs": configs,
    }
    res.update(diag)
    if calib:
        res["copy_calibration"] = calib
    res["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(w0, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
