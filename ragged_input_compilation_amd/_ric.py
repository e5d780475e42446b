"""ctypes binding of libric (include/ric.h): the same entry points, same
names, argument marshalling only.  Every computation runs in the library's
HIP kernels; if the library is not built this module raises at load time.

Device pointers and streams are plain integers (e.g. ``tensor.data_ptr()`` and
``torch.cuda.current_stream().cuda_stream``); host arrays are numpy arrays or
sequences, converted to contiguous int32."""
from __future__ import annotations

import ctypes
import os

import numpy as np

# RIC_LIBRARY may name another build of the same library (tests load a
# host-only build through it); by default the in-tree libric.so.
LIB_PATH = os.environ.get("RIC_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libric.so")

RIC_OK, RIC_EINVAL, RIC_ENOMEM, RIC_EFULL, RIC_ENOENT, RIC_EEXIST, RIC_ERANGE, RIC_EHIP, RIC_ESTATE = \
    0, -1, -2, -3, -4, -5, -6, -7, -8
ERROR_NAMES = {RIC_EINVAL: "EINVAL", RIC_ENOMEM: "ENOMEM", RIC_EFULL: "EFULL", RIC_ENOENT: "ENOENT",
               RIC_EEXIST: "EEXIST", RIC_ERANGE: "ERANGE", RIC_EHIP: "EHIP", RIC_ESTATE: "ESTATE"}

_i32p = ctypes.POINTER(ctypes.c_int32)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_vp = ctypes.c_void_p


class RicError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {msg}")
        self.code = code


RIC_MAX_KV_GROUPS, RIC_SLOTS_PER_TOKEN, RIC_SLOTS_NONE = 4, 0, 1
RIC_FUSE_ALWAYS, RIC_FUSE_NEVER = 1, 2
RIC_CHECK_SLOTS_NOALLOC_MAX_SLOTS = 1 << 25


class ric_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "max_num_reqs", "max_model_len", "block_size", "max_blocks_per_req",
        "max_num_batched_tokens", "num_kv_blocks", "null_block", "staging_bytes", "num_kv_groups")] + \
        [(n, ctypes.c_int32 * RIC_MAX_KV_GROUPS) for n in (
            "group_block_size", "group_num_kv_blocks", "group_slot_mode")]


class ric_sampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_p", ctypes.c_float),
                ("repetition_penalty", ctypes.c_float), ("top_k", ctypes.c_int32)]


class ric_step(ctypes.Structure):
    _fields_ = [("input_ids", _vp), ("positions", _vp), ("req_indices", _vp), ("slot_mapping", _vp),
                ("query_start_loc", _vp), ("seq_lens", _vp), ("logits_indices", _vp), ("discard", _vp),
                ("sample_indices", _vp), ("dev_scalars", _vp), ("cu_seqlens_k", _vp),
                ("group_slot_mapping", _vp * RIC_MAX_KV_GROUPS)] + \
               [(n, ctypes.c_int32) for n in ("num_reqs", "num_actual_tokens", "num_tokens_padded",
                                              "max_query_len", "max_seq_len", "num_sampled", "kv_path")]


class ric_columns(ctypes.Structure):
    _fields_ = [("tokens", _vp), ("blocks", _vp), ("token_stride", ctypes.c_int64),
                ("block_stride", ctypes.c_int64)] + \
               [(n, _vp) for n in ("num_tokens", "num_prompt", "num_computed", "num_scheduled",
                                   "num_blocks", "top_k", "temperature", "top_p", "repetition_penalty")] + \
               [("group_blocks", _vp * 4), ("group_block_stride", ctypes.c_int64 * 4),
                ("group_num_blocks", _vp * 4)]


class ric_spec_decode(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("logits_indices", "cu_num_logits", "target_logits_indices",
                                   "bonus_logits_indices", "draft_token_ids")] + \
               [("num_logits", ctypes.c_int32), ("num_draft_tokens", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m ragged_input_compilation_amd.build` "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "ric_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(ric_config)]),
        "ric_create": (ctypes.c_int, [ctypes.POINTER(ric_config), _vp, _vp, ctypes.c_size_t,
                                      ctypes.POINTER(_vp)]),
        "ric_destroy": (ctypes.c_int, [_vp]),
        "ric_set_stream": (ctypes.c_int, [_vp, _vp]),
        "ric_last_error": (ctypes.c_char_p, []),
        "ric_add_request": (ctypes.c_int, [_vp, ctypes.c_uint64, _i32p, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.c_int32, _i32p, ctypes.c_int32,
                                           ctypes.POINTER(ric_sampling), _i32p]),
        "ric_remove_request": (ctypes.c_int, [_vp, ctypes.c_uint64, _i32p]),
        "ric_append_tokens": (ctypes.c_int, [_vp, ctypes.c_uint64, _i32p, ctypes.c_int32]),
        "ric_append_blocks": (ctypes.c_int, [_vp, ctypes.c_uint64, _i32p, ctypes.c_int32]),
        "ric_replace_blocks": (ctypes.c_int, [_vp, ctypes.c_uint64, _i32p, ctypes.c_int32]),
        "ric_condense": (ctypes.c_int, [_vp, _i32p]),
        "ric_flush": (ctypes.c_int, [_vp]),
        "ric_append_sampled": (ctypes.c_int, [_vp, ctypes.c_int32, _i32p, _i32p, _vp, ctypes.c_int32]),
        "ric_block_table_padded": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.c_int32, _vp]),
        "ric_append_blocks_group": (ctypes.c_int, [_vp, ctypes.c_uint64, ctypes.c_int32, _i32p, ctypes.c_int32]),
        "ric_replace_blocks_group": (ctypes.c_int, [_vp, ctypes.c_uint64, ctypes.c_int32, _i32p, ctypes.c_int32]),
        "ric_spec_decode_metadata": (ctypes.c_int, [_vp, _i32p, ctypes.POINTER(ric_spec_decode)]),
        "ric_truncate_tokens": (ctypes.c_int, [_vp, ctypes.c_uint64, ctypes.c_int32]),
        "ric_correct_computed": (ctypes.c_int, [_vp, ctypes.c_int32, _i32p, _i32p, _i32p, _vp, ctypes.c_int32,
                                                 _vp, ctypes.c_int64, _vp]),
        "ric_num_reqs": (ctypes.c_int32, [_vp]),
        "ric_row_of": (ctypes.c_int32, [_vp, ctypes.c_uint64]),
        "ric_req_at": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint64)]),
        "ric_get_columns": (ctypes.c_int, [_vp, ctypes.POINTER(ric_columns)]),
        "ric_sync": (ctypes.c_int, [_vp]),
        "ric_read_device": (ctypes.c_int, [_vp, _vp, ctypes.c_size_t]),
        "ric_schedule": (ctypes.c_int, [_vp, ctypes.c_int32, _i32p, _i32p]),
        "ric_compile": (ctypes.c_int, [_vp, ctypes.c_int32, ctypes.POINTER(ric_step)]),
        "ric_compile_and_cache": (ctypes.c_int, [_vp, ctypes.c_int32] + [ctypes.POINTER(_vp)] * 4 + [
            ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, _vp, ctypes.c_uint32,
            ctypes.POINTER(ric_step)]),
        "ric_reshape_and_cache": (ctypes.c_int, [ctypes.POINTER(_vp)] * 4 + [
            ctypes.c_int32, _vp, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, _vp,
            ctypes.c_uint32, _vp]),
        "ric_gather_rows": (ctypes.c_int, [_vp, ctypes.c_int64, ctypes.c_int64, _vp, _vp, ctypes.c_int32,
                                           ctypes.c_int32, _vp, ctypes.c_int64, _vp, _vp]),
        "ric_check_slots_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64]),
        "ric_check_slots": (ctypes.c_int, [_vp, ctypes.c_int32, _vp, ctypes.c_int64, _vp, ctypes.c_size_t, _vp,
                                           _vp]),
        "ric_check_slots_noalloc": (ctypes.c_int, [_vp, ctypes.c_int32, _vp, ctypes.c_int64, _vp, _vp]),
        "ric_padded_size": (ctypes.c_int32, [_i32p, ctypes.c_int32, ctypes.c_int32]),
        "ric_condense_plan": (ctypes.c_int32, [_u8p, ctypes.c_int32, _i32p, _i32p]),
        "ric_check_step": (ctypes.c_int, [ctypes.POINTER(ric_config), ctypes.c_int32] + [_i32p] * 5 +
                           [ctypes.c_int32, ctypes.POINTER(ric_step)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()
EXPORTS = tuple(n for n in dir(_lib) if n.startswith("ric_"))


def lib():
    return _lib


def _err(code):
    if code < 0:
        raise RicError(code, _lib.ric_last_error().decode(errors="replace"))
    return code


def _i32(a):
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return arr, arr.ctypes.data_as(_i32p)


def make_config(**kw) -> ric_config:
    """Fields by name; the per-group fields take a sequence indexed by group."""
    c = ric_config()
    for k, v in kw.items():
        if isinstance(v, (list, tuple)):
            arr = getattr(c, k)
            for i, x in enumerate(v):
                arr[i] = int(x)
        else:
            setattr(c, k, int(v))
    return c


# ---- handle -----------------------------------------------------------------

def ric_workspace_bytes(cfg: ric_config) -> int:
    return int(_lib.ric_workspace_bytes(ctypes.byref(cfg)))


def ric_create(cfg: ric_config, stream: int = 0, workspace: int = 0, workspace_bytes: int = 0) -> int:
    h = _vp()
    _err(_lib.ric_create(ctypes.byref(cfg), _vp(stream or None), _vp(workspace or None),
                         ctypes.c_size_t(workspace_bytes), ctypes.byref(h)))
    return h.value


def ric_destroy(h: int) -> None:
    _err(_lib.ric_destroy(_vp(h)))


def ric_set_stream(h: int, stream: int) -> None:
    _err(_lib.ric_set_stream(_vp(h), _vp(stream or None)))


def ric_last_error() -> str:
    return _lib.ric_last_error().decode(errors="replace")


# ---- column-store deltas --------------------------------------------------------

def ric_add_request(h: int, req_id: int, tokens, num_prompt: int, num_computed: int, blocks,
                    sampling=None) -> int:
    tok, tp = _i32(tokens)
    blk, bp = _i32(blocks)
    sp = None
    if sampling is not None:
        t, p, rp, k = sampling
        sp = ctypes.byref(ric_sampling(t, p, rp, k))
    row = ctypes.c_int32(-1)
    _err(_lib.ric_add_request(_vp(h), req_id, tp, tok.shape[0], num_prompt, num_computed, bp, blk.shape[0],
                              sp, ctypes.byref(row)))
    return row.value


def ric_remove_request(h: int, req_id: int) -> int:
    row = ctypes.c_int32(-1)
    _err(_lib.ric_remove_request(_vp(h), req_id, ctypes.byref(row)))
    return row.value


def ric_append_tokens(h: int, req_id: int, ids) -> None:
    a, p = _i32(ids)
    _err(_lib.ric_append_tokens(_vp(h), req_id, p, a.shape[0]))


def ric_append_blocks(h: int, req_id: int, ids) -> None:
    a, p = _i32(ids)
    _err(_lib.ric_append_blocks(_vp(h), req_id, p, a.shape[0]))


def ric_replace_blocks(h: int, req_id: int, ids) -> None:
    a, p = _i32(ids)
    _err(_lib.ric_replace_blocks(_vp(h), req_id, p, a.shape[0]))


def ric_condense(h: int) -> int:
    n = ctypes.c_int32(0)
    _err(_lib.ric_condense(_vp(h), ctypes.byref(n)))
    return n.value


def ric_flush(h: int) -> None:
    _err(_lib.ric_flush(_vp(h)))


def ric_append_sampled(h: int, rows, dev_tokens: int, dev_tokens_len: int, src_index=None) -> None:
    r, rp = _i32(rows)
    if src_index is None:
        sp = None
    else:
        s, sp = _i32(src_index)
        if s.shape != r.shape:
            raise ValueError("rows and src_index differ in length")
    _err(_lib.ric_append_sampled(_vp(h), r.shape[0], rp, sp, _vp(dev_tokens), dev_tokens_len))


def ric_spec_decode_metadata(h: int, num_draft_tokens) -> ric_spec_decode:
    d, dp = _i32(num_draft_tokens)
    out = ric_spec_decode()
    _err(_lib.ric_spec_decode_metadata(_vp(h), dp, ctypes.byref(out)))
    return out


def ric_truncate_tokens(h: int, req_id: int, num_tokens: int) -> None:
    _err(_lib.ric_truncate_tokens(_vp(h), req_id, num_tokens))


def ric_correct_computed(h: int, rows, prev_index, num_draft, dev_num_accepted: int, prev_len: int,
                         dev_sampled: int = 0, sampled_stride: int = 0, dev_status: int = 0) -> None:
    r, rp = _i32(rows)
    p, pp = _i32(prev_index)
    d, dp = _i32(num_draft)
    if not (r.shape == p.shape == d.shape):
        raise ValueError("rows, prev_index and num_draft differ in length")
    _err(_lib.ric_correct_computed(_vp(h), r.shape[0], rp, pp, dp, _vp(dev_num_accepted or None), prev_len,
                                   _vp(dev_sampled or None), sampled_stride, _vp(dev_status or None)))


def ric_block_table_padded(h: int, width: int, fill: int, dst: int, group: int = 0,
                           kernel_blocks_per_block: int = 1) -> None:
    _err(_lib.ric_block_table_padded(_vp(h), group, kernel_blocks_per_block, width, fill, _vp(dst or None)))


def ric_append_blocks_group(h: int, req_id: int, group: int, ids) -> None:
    a, p = _i32(ids)
    _err(_lib.ric_append_blocks_group(_vp(h), req_id, group, p, a.shape[0]))


def ric_replace_blocks_group(h: int, req_id: int, group: int, ids) -> None:
    a, p = _i32(ids)
    _err(_lib.ric_replace_blocks_group(_vp(h), req_id, group, p, a.shape[0]))


def ric_num_reqs(h: int) -> int:
    return _err(_lib.ric_num_reqs(_vp(h)))


def ric_row_of(h: int, req_id: int) -> int:
    """Row of a live request, or -1 when absent."""
    r = _lib.ric_row_of(_vp(h), req_id)
    return -1 if r == RIC_ENOENT else _err(r)


def ric_req_at(h: int, row: int):
    """Request id at a row, or None for a hole."""
    out = ctypes.c_uint64(0)
    rc = _lib.ric_req_at(_vp(h), row, ctypes.byref(out))
    if rc == RIC_ENOENT:
        return None
    _err(rc)
    return out.value


def ric_get_columns(h: int) -> ric_columns:
    c = ric_columns()
    _err(_lib.ric_get_columns(_vp(h), ctypes.byref(c)))
    return c


def ric_sync(h: int) -> None:
    _err(_lib.ric_sync(_vp(h)))


def ric_read_device(dev_src: int, nbytes: int, dtype=np.uint8) -> np.ndarray:
    """Synchronous copy of device bytes to a new host array (inspection)."""
    out = np.zeros(nbytes, np.uint8)
    _err(_lib.ric_read_device(out.ctypes.data_as(_vp), _vp(dev_src), nbytes))
    return out.view(dtype)


# ---- step -------------------------------------------------------------------

def ric_schedule(h: int, num_computed, num_scheduled) -> None:
    c, cp = _i32(num_computed)
    q, qp = _i32(num_scheduled)
    if c.shape != q.shape:
        raise ValueError("num_computed and num_scheduled differ in length")
    _err(_lib.ric_schedule(_vp(h), c.shape[0], cp, qp))


def ric_compile(h: int, num_tokens_padded: int) -> ric_step:
    s = ric_step()
    _err(_lib.ric_compile(_vp(h), num_tokens_padded, ctypes.byref(s)))
    return s


def _ptr_arrays(k_ptrs, v_ptrs, k_cache_ptrs, v_cache_ptrs):
    L = len(k_ptrs)
    if not (len(v_ptrs) == len(k_cache_ptrs) == len(v_cache_ptrs) == L):
        raise ValueError("pointer lists differ in length")
    arr = [(_vp * max(L, 1))(*[_vp(p) for p in lst]) for lst in (k_ptrs, v_ptrs, k_cache_ptrs, v_cache_ptrs)]
    return L, arr, [ctypes.cast(a, ctypes.POINTER(_vp)) for a in arr]


def ric_compile_and_cache(h: int, num_tokens_padded: int, k_ptrs, v_ptrs, k_cache_ptrs, v_cache_ptrs,
                          row_bytes: int, num_slots: int, src_row_stride: int = 0, dev_status: int = 0,
                          flags: int = 0) -> ric_step:
    L, keep, ptrs = _ptr_arrays(k_ptrs, v_ptrs, k_cache_ptrs, v_cache_ptrs)
    s = ric_step()
    _err(_lib.ric_compile_and_cache(_vp(h), num_tokens_padded, *ptrs, L, src_row_stride, row_bytes, num_slots,
                                    _vp(dev_status or None), flags, ctypes.byref(s)))
    return s


def ric_reshape_and_cache(k_ptrs, v_ptrs, k_cache_ptrs, v_cache_ptrs, slot_mapping: int, num_tokens: int,
                          row_bytes: int, num_slots: int, src_row_stride: int = 0, dev_status: int = 0,
                          flags: int = 0, stream: int = 0) -> None:
    L = len(k_ptrs)
    if not (len(v_ptrs) == len(k_cache_ptrs) == len(v_cache_ptrs) == L):
        raise ValueError("pointer lists differ in length")
    arr = [(_vp * max(L, 1))(*[_vp(p) for p in lst]) for lst in (k_ptrs, v_ptrs, k_cache_ptrs, v_cache_ptrs)]
    _err(_lib.ric_reshape_and_cache(*[ctypes.cast(a, ctypes.POINTER(_vp)) for a in arr], L,
                                    _vp(slot_mapping), num_tokens, src_row_stride, row_bytes, num_slots,
                                    _vp(dev_status or None), flags, _vp(stream or None)))


def ric_gather_rows(src: int, src_row_stride: int, src_rows: int, idx: int, dev_count: int, max_rows: int,
                    row_bytes: int, dst: int, dst_row_stride: int = 0, dev_status: int = 0,
                    stream: int = 0) -> None:
    _err(_lib.ric_gather_rows(_vp(src), src_row_stride, src_rows, _vp(idx), _vp(dev_count or None), max_rows,
                              row_bytes, _vp(dst), dst_row_stride, _vp(dev_status or None),
                              _vp(stream or None)))


def ric_check_slots_workspace_bytes(num_slots: int) -> int:
    return int(_lib.ric_check_slots_workspace_bytes(num_slots))


def ric_check_slots(slot_mapping: int, num_tokens: int, num_slots: int, workspace: int, workspace_bytes: int,
                    dev_result: int, dev_num_tokens: int = 0, stream: int = 0) -> None:
    _err(_lib.ric_check_slots(_vp(slot_mapping or None), num_tokens, _vp(dev_num_tokens or None), num_slots,
                              _vp(workspace or None), workspace_bytes, _vp(dev_result or None),
                              _vp(stream or None)))


def ric_check_slots_noalloc(slot_mapping: int, num_tokens: int, num_slots: int, dev_result: int,
                            dev_num_tokens: int = 0, stream: int = 0) -> None:
    _err(_lib.ric_check_slots_noalloc(_vp(slot_mapping or None), num_tokens, _vp(dev_num_tokens or None),
                                      num_slots, _vp(dev_result or None), _vp(stream or None)))


# ---- host-only helpers ----------------------------------------------------------

def ric_padded_size(capture_sizes, num_tokens: int) -> int:
    a, p = _i32(capture_sizes)
    return _err(_lib.ric_padded_size(p, a.shape[0], num_tokens))


def ric_condense_plan(live):
    m = np.ascontiguousarray(np.asarray(live, dtype=np.uint8))
    holes = np.zeros(max(m.shape[0], 1), np.int32)
    srcs = np.zeros(max(m.shape[0], 1), np.int32)
    n = _err(_lib.ric_condense_plan(m.ctypes.data_as(_u8p), m.shape[0], holes.ctypes.data_as(_i32p),
                                    srcs.ctypes.data_as(_i32p)))
    return list(zip(holes[:n].tolist(), srcs[:n].tolist()))


def ric_check_step(cfg: ric_config, num_computed, num_scheduled, num_prompt, num_tokens, num_blocks,
                   num_tokens_padded: int) -> ric_step:
    arrs = [_i32(a) for a in (num_computed, num_scheduled, num_prompt, num_tokens, num_blocks)]
    s = ric_step()
    _err(_lib.ric_check_step(ctypes.byref(cfg), arrs[0][0].shape[0], *[p for _, p in arrs],
                             num_tokens_padded, ctypes.byref(s)))
    return s
