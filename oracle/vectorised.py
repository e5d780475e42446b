"""The same step built from numpy library routines.

Test infrastructure only.  This is the array formulation the pages describe for
the CPU side of the runner, used here as a second, independently written
oracle that the per-token loops in ``step`` must agree with:

* request expansion by ``repeat`` of the request numbers by their scheduled
  counts ([P1 §为什么删除后还要压紧], [P2 §8.3.1.6]); a token's index
  inside its request is its flat index minus the start of its request,
  gathered from the exclusive prefix sum;
* the token gather as one ``take`` from the flattened [rows, max_model_len]
  table at ``row * max_model_len + position`` ([P2 §8.3.1.7 torch.index_select
  而不是 np.take]; [P1 §第三步：从二维 token 历史抽取本轮切片]);
* slots from the block table gathered at ``position // B``
  ([P2 §8.3.2 slot_mapping：新 token 写到哪个 KV 槽]);
* ``logits_indices = query_start_loc[1:] - 1`` ([P2 §8.6.3]).

Pad readings are the same as in ``step``.
"""
from __future__ import annotations

import numpy as np


def compile_arrays(c, q, P, token_table, block_table, *, block_size: int,
                   max_num_reqs: int, n_pad: int, null_block: int = 0):
    """``c, q, P``: int arrays [R].  ``token_table``: [R, max_model_len];
    ``block_table``: [R, max_blocks].  Returns a dict of numpy arrays."""
    c = np.asarray(c, dtype=np.int64)
    q = np.asarray(q, dtype=np.int64)
    P = np.asarray(P, dtype=np.int64)
    R = c.shape[0]
    M = token_table.shape[1]
    nblk = block_table.shape[1]

    cu = np.cumsum(q)
    N = int(cu[-1]) if R else 0
    starts = cu - q                                    # first flat index of each request
    req_indices = np.repeat(np.arange(R), q)
    query_pos = np.arange(N) - starts[req_indices]
    positions = c[req_indices] + query_pos
    input_ids = np.take(token_table.reshape(-1), req_indices * M + positions)
    block_numbers = np.take(block_table.reshape(-1), req_indices * nblk + positions // block_size)
    slots = block_numbers.astype(np.int64) * block_size + positions % block_size

    pad = n_pad - N
    out = {
        "input_ids": np.concatenate([input_ids, np.zeros(pad, np.int64)]),
        "positions": np.concatenate([positions, np.zeros(pad, np.int64)]),
        "req_indices": np.concatenate([req_indices, np.full(pad, -1)]),
        "slot_mapping": np.concatenate([slots, np.full(pad, null_block * block_size)]),
    }
    qsl = np.full(max_num_reqs + 1, N, dtype=np.int64)
    qsl[0] = 0
    qsl[1:R + 1] = cu
    seq = np.zeros(max_num_reqs, np.int64)
    seq[:R] = c + q
    logits = np.full(max_num_reqs, -1, np.int64)
    logits[:R] = qsl[1:R + 1] - 1
    discard = np.ones(max_num_reqs, np.int64)
    discard[:R] = (c + q < P)
    keep = logits[:R][discard[:R] == 0]
    sample = np.full(max_num_reqs, -1, np.int64)
    sample[:keep.shape[0]] = keep
    cu_k = np.concatenate([[0], np.cumsum(seq)])
    out.update(query_start_loc=qsl, seq_lens=seq, cu_seqlens_k=cu_k, logits_indices=logits, discard=discard,
               sample_indices=sample, num_sampled=int(keep.shape[0]))
    return {k: (v.astype(np.int64) if isinstance(v, np.ndarray) else v) for k, v in out.items()}


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping) -> None:
    """Fancy-index assignment ``cache[slot] = rows`` per tensor.  ``k``/``v``:
    [N, row_elems]; caches: [num_slots, row_elems]."""
    slot = np.asarray(slot_mapping, dtype=np.int64)
    k_cache[slot] = k
    v_cache[slot] = v


def gather_rows(src, indices, count: int):
    idx = np.asarray(indices[:count], dtype=np.int64)
    out = np.zeros((count,) + src.shape[1:], dtype=src.dtype)
    ok = idx >= 0
    out[ok] = src[idx[ok]]
    return out
