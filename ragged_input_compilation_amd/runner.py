"""Step driver: runs one workload through libric with PyTorch-owned device
memory and streams.

PyTorch supplies device buffers (workspace, K/V sources, caches, hidden
states) and the stream; every step computation is a libric call.  The driver
only sequences the calls: load the request history into the persistent batch
(adds, removals, condense, refills), schedule, compile, write K/V for every
layer, gather hidden rows."""
from __future__ import annotations

import os
from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

from . import _ric as ric

_TORCH_DT = {"f16": torch.float16, "bf16": torch.bfloat16}
DEBUG = os.environ.get("RIC_DEBUG", "") not in ("", "0")


def config_of(w) -> ric.ric_config:
    return ric.make_config(max_num_reqs=w.max_num_reqs, max_model_len=w.max_model_len,
                           block_size=w.block_size, max_blocks_per_req=w.max_blocks_per_req,
                           max_num_batched_tokens=w.max_num_batched_tokens,
                           num_kv_blocks=w.num_kv_blocks, null_block=w.null_block, staging_bytes=0)


def current_stream() -> int:
    return int(torch.cuda.current_stream().cuda_stream)


class Batch:
    """A libric handle whose workspace is a torch tensor."""

    def __init__(self, cfg: ric.ric_config, device="cuda", stream: Optional[int] = None):
        self.cfg = cfg
        self.stream = current_stream() if stream is None else stream
        nbytes = ric.ric_workspace_bytes(cfg)
        if nbytes == 0:
            raise ric.RicError(ric.RIC_EINVAL, ric.ric_last_error())
        # torch's caching allocator returns blocks aligned to at least 512 bytes
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.h = ric.ric_create(cfg, self.stream, self.workspace.data_ptr(), nbytes)

    def close(self):
        if self.h:
            ric.ric_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # history -------------------------------------------------------------
    def add(self, r) -> int:
        return ric.ric_add_request(self.h, r.req_id, r.tokens, r.num_prompt, r.num_computed, r.blocks,
                                   (r.temperature, r.top_p, r.rep_penalty, r.top_k))

    def load_history(self, w) -> int:
        """Add the initial requests, remove the finished ones, condense, add the
        refills.  Returns the number of rows condense moved."""
        for r in w.initial:
            self.add(r)
        for rid in w.finished:
            ric.ric_remove_request(self.h, rid)
        moved = ric.ric_condense(self.h) if w.finished else 0
        for r in w.refill:
            self.add(r)
        ric.ric_flush(self.h)
        return moved

    def row_order(self) -> List[int]:
        n = ric.ric_num_reqs(self.h)
        return [ric.ric_req_at(self.h, i) for i in range(n)]

    def schedule_from(self, w, order: Optional[List[int]] = None) -> None:
        """Schedule every live request with its workload (c, q), rows in
        ``order`` (request ids by row; default: the handle's own rows)."""
        order = self.row_order() if order is None else order
        by_id = w.by_id()
        ric.ric_schedule(self.h, [by_id[i].num_computed for i in order], [by_id[i].num_scheduled for i in order])

    def compile(self, n_pad: int) -> ric.ric_step:
        s = ric.ric_compile(self.h, n_pad)
        if DEBUG:
            self.debug_dump(s)
        return s

    def slot_collisions(self, s: ric.ric_step) -> tuple:
        """(collisions, out-of-range slots) among the step's real tokens, by
        the library's device-side check (debugging; synchronises)."""
        res = torch.zeros(2, dtype=torch.int32, device=self.workspace.device)
        num_slots = self.cfg.num_kv_blocks * self.cfg.block_size
        if num_slots <= ric.RIC_CHECK_SLOTS_NOALLOC_MAX_SLOTS:
            ric.ric_check_slots_noalloc(s.slot_mapping, s.num_tokens_padded, num_slots, res.data_ptr(),
                                        dev_num_tokens=s.dev_scalars + 4, stream=self.stream)
        else:
            nbytes = ric.ric_check_slots_workspace_bytes(num_slots)
            ws = torch.empty(nbytes, dtype=torch.uint8, device=self.workspace.device)
            ric.ric_check_slots(s.slot_mapping, s.num_tokens_padded, num_slots, ws.data_ptr(), nbytes,
                                res.data_ptr(), dev_num_tokens=s.dev_scalars + 4, stream=self.stream)
        torch.cuda.synchronize()
        return tuple(int(x) for x in res.tolist())

    def debug_dump(self, s: ric.ric_step, limit: int = 32) -> None:
        """Print the small per-step arrays a developer checks first when a step
        goes wrong (request order, counts, boundaries, positions, slots,
        logits rows, discard), not the tables, and the device-side count of
        real tokens sharing a slot.  Synchronises: debugging only, enabled by
        RIC_DEBUG=1."""
        R, n = s.num_reqs, s.num_tokens_padded
        cols = ric.ric_get_columns(self.h)
        show = lambda a: " ".join(str(int(x)) for x in a[:limit]) + (" ..." if len(a) > limit else "")
        print(f"[ric] R={R} N={s.num_actual_tokens} N_pad={n} max_q={s.max_query_len} "
              f"max_seq={s.max_seq_len} sampled={s.num_sampled}")
        print(f"[ric] req_ids    {show(self.row_order())}")
        print(f"[ric] computed   {show(self.device_i32(cols.num_computed, R))}")
        print(f"[ric] scheduled  {show(self.device_i32(cols.num_scheduled, R))}")
        print(f"[ric] qsl        {show(self.device_i32(s.query_start_loc, R + 1))}")
        print(f"[ric] positions  {show(self.device_i32(s.positions, n))}")
        print(f"[ric] seq_lens   {show(self.device_i32(s.seq_lens, R))}")
        print(f"[ric] slots      {show(self.device_i32(s.slot_mapping, n))}")
        print(f"[ric] logits     {show(self.device_i32(s.logits_indices, R))}")
        print(f"[ric] discard    {show(self.device_u8(s.discard, R))}")
        dup, bad = self.slot_collisions(s)
        print(f"[ric] slot collisions {dup}, out-of-range slots {bad}", flush=True)

    # inspection (tests) ------------------------------------------------------
    def device_i32(self, ptr: int, n: int) -> np.ndarray:
        """Copy n int32 values from a device address to the host (test use)."""
        if n == 0:
            return np.zeros(0, np.int32)
        t = torch.empty(n, dtype=torch.int32, device=self.workspace.device)
        nbytes = 4 * n
        src = _view_u8(self.workspace, ptr, nbytes)
        t.view(torch.uint8).copy_(src)
        return t.cpu().numpy()

    def device_u8(self, ptr: int, n: int) -> np.ndarray:
        if n == 0:
            return np.zeros(0, np.uint8)
        return _view_u8(self.workspace, ptr, n).cpu().numpy()

    def step_outputs(self, s: ric.ric_step) -> dict:
        MR = self.cfg.max_num_reqs
        n = s.num_tokens_padded
        out = {
            "input_ids": self.device_i32(s.input_ids, n),
            "positions": self.device_i32(s.positions, n),
            "req_indices": self.device_i32(s.req_indices, n),
            "slot_mapping": self.device_i32(s.slot_mapping, n),
            "query_start_loc": self.device_i32(s.query_start_loc, MR + 1),
            "cu_seqlens_k": self.device_i32(s.cu_seqlens_k, MR + 1),
            "seq_lens": self.device_i32(s.seq_lens, MR),
            "logits_indices": self.device_i32(s.logits_indices, MR),
            "discard": self.device_u8(s.discard, MR),
            "sample_indices": self.device_i32(s.sample_indices, MR),
            "dev_scalars": self.device_i32(s.dev_scalars, 8),
        }
        out["num_sampled"] = int(out["dev_scalars"][5])
        return out


def _view_u8(anchor: torch.Tensor, ptr: int, nbytes: int) -> torch.Tensor:
    """A uint8 view of [ptr, ptr+nbytes) inside the anchor tensor's storage."""
    base = anchor.data_ptr()
    off = ptr - base
    if off < 0 or off + nbytes > anchor.numel():
        raise ValueError("address outside the workspace")
    return anchor.view(torch.uint8)[off:off + nbytes]


@dataclass
class KVSet:
    """Per-layer K/V sources [n_pad, H, D] and paged caches [num_blocks, B, H, D]."""
    k: List[torch.Tensor]
    v: List[torch.Tensor]
    kc: List[torch.Tensor]
    vc: List[torch.Tensor]
    row_bytes: int
    num_slots: int


def alloc_caches(w, num_layers: Optional[int] = None, device="cuda", fill: Optional[int] = None):
    L = w.num_layers if num_layers is None else num_layers
    dt = _TORCH_DT[w.kv_dtype]
    shape = (w.num_kv_blocks, w.block_size, w.kv_heads, w.head_dim)
    kc, vc = [], []
    for _ in range(L):
        for lst in (kc, vc):
            t = torch.empty(shape, dtype=dt, device=device)
            if fill is not None:
                t.view(torch.int16).fill_(fill)
            lst.append(t)
    return kc, vc


def alloc_sources(w, n_tokens: int, seed: int, num_layers: Optional[int] = None, device="cuda",
                  host: bool = False):
    """Seeded N(0,1) K/V sources per layer; ``host`` draws them with numpy
    (bit-reproducible on the CPU) and uploads them."""
    from workloads import payload_numpy, payload_torch  # seeded generators only
    L = w.num_layers if num_layers is None else num_layers
    shape = (n_tokens, w.kv_heads, w.head_dim)
    k, v = [], []
    for l in range(L):
        for j, lst in enumerate((k, v)):
            s = seed + 2 * l + j
            if host:
                bits = payload_numpy(np.random.default_rng(s), shape, w.kv_dtype)
                t = torch.from_numpy(bits.view(np.int16)).to(device).view(_TORCH_DT[w.kv_dtype])
            else:
                t = payload_torch(shape, w.kv_dtype, s, device)
            lst.append(t)
    return k, v


def reshape_and_cache(kv: KVSet, slot_mapping: int, num_tokens: int, dev_status: int = 0,
                      stream: Optional[int] = None, flags: int = 0) -> None:
    ric.ric_reshape_and_cache([t.data_ptr() for t in kv.k], [t.data_ptr() for t in kv.v],
                              [t.data_ptr() for t in kv.kc], [t.data_ptr() for t in kv.vc],
                              slot_mapping, num_tokens, kv.row_bytes, kv.num_slots,
                              src_row_stride=kv.k[0].stride(0) * kv.k[0].element_size(),
                              dev_status=dev_status, flags=flags,
                              stream=current_stream() if stream is None else stream)


def compile_and_cache(batch: "Batch", n_pad: int, kv: KVSet, dev_status: int = 0, flags: int = 0) -> ric.ric_step:
    """Compile plus the K/V write of every layer in one library call (one
    kernel for rows of 128 B to 8 KiB, unless the rows are 1 KiB or more and
    the step is mostly long chunks; flags RIC_FUSE_ALWAYS / RIC_FUSE_NEVER
    force the path)."""
    return ric.ric_compile_and_cache(batch.h, n_pad, [t.data_ptr() for t in kv.k], [t.data_ptr() for t in kv.v],
                                     [t.data_ptr() for t in kv.kc], [t.data_ptr() for t in kv.vc], kv.row_bytes,
                                     kv.num_slots, src_row_stride=kv.k[0].stride(0) * kv.k[0].element_size(),
                                     dev_status=dev_status, flags=flags)


def gather(hidden: torch.Tensor, idx_ptr: int, dev_count_ptr: int, max_rows: int, out: torch.Tensor,
           dev_status: int = 0, stream: Optional[int] = None) -> None:
    row_bytes = hidden.shape[1] * hidden.element_size()
    ric.ric_gather_rows(hidden.data_ptr(), hidden.stride(0) * hidden.element_size(), hidden.shape[0],
                        idx_ptr, dev_count_ptr, max_rows, row_bytes, out.data_ptr(),
                        out.stride(0) * out.element_size(), dev_status,
                        current_stream() if stream is None else stream)
