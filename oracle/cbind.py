"""ctypes access to the plain C oracle (test infrastructure only)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)


class _In(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_num_reqs", ctypes.c_int32), ("n_pad", ctypes.c_int32),
                ("null_block", ctypes.c_int32), ("tok_stride", ctypes.c_int64),
                ("blk_stride", ctypes.c_int64), ("num_computed", _i32p),
                ("num_scheduled", _i32p), ("num_prompt", _i32p), ("tokens", _i32p),
                ("blocks", _i32p)]


class _Out(ctypes.Structure):
    _fields_ = [("input_ids", _i32p), ("positions", _i32p), ("req_indices", _i32p),
                ("slot_mapping", _i32p), ("query_start_loc", _i32p), ("cu_seqlens_k", _i32p),
                ("seq_lens", _i32p), ("logits_indices", _i32p), ("discard", _u8p),
                ("sample_indices", _i32p), ("num_sampled", ctypes.c_int32),
                ("num_actual_tokens", ctypes.c_int32), ("max_seqlen_q", ctypes.c_int32),
                ("max_seqlen_k", ctypes.c_int32)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = ctypes.CDLL(_build.LIB)
        _lib.nano_compile.argtypes = [ctypes.POINTER(_In), ctypes.POINTER(_Out)]
        _lib.nano_compile.restype = ctypes.c_int
        _lib.nano_kv_scatter.argtypes = [ctypes.c_void_p] * 4 + [_i32p, ctypes.c_int32, ctypes.c_int64]
        _lib.nano_kv_scatter.restype = None
        _lib.nano_gather.argtypes = [ctypes.c_void_p, ctypes.c_int64, _i32p, ctypes.c_int32, ctypes.c_void_p]
        _lib.nano_gather.restype = None
    return _lib


def _p(a, t=_i32p):
    return a.ctypes.data_as(t)


def pack_tables(rows, tok_stride=None, blk_stride=None):
    """Row lists -> dense int32 tables (unused tail entries are -7, never read)."""
    R = len(rows)
    tok_stride = tok_stride or max([len(r.tokens) for r in rows] + [1])
    blk_stride = blk_stride or max([len(r.blocks) for r in rows] + [1])
    tok = np.full((max(R, 1), tok_stride), -7, np.int32)
    blk = np.full((max(R, 1), blk_stride), -7, np.int32)
    for i, r in enumerate(rows):
        tok[i, :len(r.tokens)] = r.tokens
        blk[i, :len(r.blocks)] = r.blocks
    return tok, blk


class Compiled(dict):
    pass


def compile_step(rows, *, block_size, max_num_reqs, n_pad, null_block=0, tables=None):
    """Run ``nano_compile`` on rows (objects with num_computed / num_scheduled /
    num_prompt / tokens / blocks).  ``tables`` may pass pre-packed (tok, blk)."""
    L = lib()
    R = len(rows)
    c = np.ascontiguousarray([r.num_computed for r in rows] or [0], np.int32)
    q = np.ascontiguousarray([r.num_scheduled for r in rows] or [0], np.int32)
    P = np.ascontiguousarray([r.num_prompt for r in rows] or [0], np.int32)
    tok, blk = tables if tables is not None else pack_tables(rows)
    o = {k: np.zeros(max(n_pad, 1), np.int32) for k in ("input_ids", "positions", "req_indices", "slot_mapping")}
    for k in ("query_start_loc", "cu_seqlens_k"):
        o[k] = np.zeros(max_num_reqs + 1, np.int32)
    for k in ("seq_lens", "logits_indices", "sample_indices"):
        o[k] = np.zeros(max_num_reqs, np.int32)
    o["discard"] = np.zeros(max_num_reqs, np.uint8)
    ins = _In(R, block_size, max_num_reqs, n_pad, null_block, tok.shape[1], blk.shape[1],
              _p(c), _p(q), _p(P), _p(tok), _p(blk))
    outs = _Out(*[_p(o[k]) for k in ("input_ids", "positions", "req_indices", "slot_mapping",
                                    "query_start_loc", "cu_seqlens_k", "seq_lens", "logits_indices")],
                _p(o["discard"], _u8p), _p(o["sample_indices"]), 0, 0, 0, 0)
    rc = L.nano_compile(ctypes.byref(ins), ctypes.byref(outs))
    if rc != 0:
        raise ValueError("nano_compile rejected the step")
    res = Compiled({k: v[:n_pad] if k in ("input_ids", "positions", "req_indices", "slot_mapping") else v
                    for k, v in o.items()})
    res.update(num_sampled=outs.num_sampled, num_actual_tokens=outs.num_actual_tokens,
               max_query_len=outs.max_seqlen_q, max_seq_len=outs.max_seqlen_k)
    return res


def kv_scatter(k, v, k_cache, v_cache, slot, row_bytes):
    """k, v: contiguous arrays [n, row]; caches: writable contiguous [slots, row]."""
    slot = np.ascontiguousarray(slot, np.int32)
    lib().nano_kv_scatter(k.ctypes.data, v.ctypes.data, k_cache.ctypes.data, v_cache.ctypes.data,
                          _p(slot), int(slot.shape[0]), int(row_bytes))


def gather(src, row_bytes, idx, count, out):
    idx = np.ascontiguousarray(idx, np.int32)
    lib().nano_gather(src.ctypes.data, int(row_bytes), _p(idx), int(count), out.ctypes.data)
