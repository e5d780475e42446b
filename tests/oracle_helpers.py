"""Shared test helpers: build oracle rows from small hand-written cases and
run all three oracle formulations on the same rows."""
import json
import os
from dataclasses import dataclass

import numpy as np

from oracle import cbind, step, vectorised

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


@dataclass
class Row:
    num_computed: int
    num_scheduled: int
    num_prompt: int
    tokens: np.ndarray
    blocks: np.ndarray


def labelled_rows(c, q, P, block_size, blocks=None, first_block=1):
    """Token p of request k is 1000*(k+1)+p; history length max(P, c+q).
    Without ``blocks`` each request gets fresh consecutive ids."""
    rows, nxt = [], first_block
    for k in range(len(q)):
        T = max(P[k], c[k] + q[k])
        tokens = np.array([1000 * (k + 1) + p for p in range(T)], np.int64)
        if blocks is None:
            nb = -(-(c[k] + q[k]) // block_size)
            b = np.arange(nxt, nxt + nb, dtype=np.int64)
            nxt += nb
        else:
            b = np.asarray(blocks[k], np.int64)
        rows.append(Row(c[k], q[k], P[k], tokens, b))
    return rows


def rows_of(reqs):
    """workloads.Req list -> Row list."""
    return [Row(r.num_computed, r.num_scheduled, r.num_prompt,
                np.asarray(r.tokens, np.int64), np.asarray(r.blocks, np.int64)) for r in reqs]


KEYS = ("input_ids", "positions", "req_indices", "slot_mapping", "query_start_loc",
        "seq_lens", "cu_seqlens_k", "logits_indices", "discard", "sample_indices")


def run_all(rows, *, block_size, max_num_reqs=None, n_pad=None, null_block=0,
            max_model_len=None, num_kv_blocks=None):
    """Run the Python, numpy and C formulations; return their outputs as
    dicts of int64 arrays (plus scalar entries)."""
    R = len(rows)
    max_num_reqs = max_num_reqs or max(R, 1)
    N = sum(r.num_scheduled for r in rows)
    n_pad = N if n_pad is None else n_pad
    max_model_len = max_model_len or max([len(r.tokens) for r in rows] + [1])
    num_kv_blocks = num_kv_blocks or (max([int(b) for r in rows for b in r.blocks] + [0]) + 1)
    py = step.compile_step(rows, block_size=block_size, max_num_reqs=max_num_reqs,
                           max_model_len=max_model_len, max_num_batched_tokens=max(n_pad, 1),
                           num_kv_blocks=num_kv_blocks, n_pad=n_pad, null_block=null_block)
    tok, blk = cbind.pack_tables(rows)
    npv = vectorised.compile_arrays([r.num_computed for r in rows], [r.num_scheduled for r in rows],
                                    [r.num_prompt for r in rows], tok, blk, block_size=block_size,
                                    max_num_reqs=max_num_reqs, n_pad=n_pad, null_block=null_block)
    cc = cbind.compile_step(rows, block_size=block_size, max_num_reqs=max_num_reqs, n_pad=n_pad,
                            null_block=null_block, tables=(tok, blk))
    out = []
    for res in (py, npv, cc):
        d = {k: np.asarray(res[k], np.int64) for k in KEYS}
        d["num_sampled"] = int(res["num_sampled"])
        out.append(d)
    out[0]["max_query_len"] = py["max_query_len"]
    out[0]["max_seq_len"] = py["max_seq_len"]
    out[0]["num_actual_tokens"] = py["num_actual_tokens"]
    out[2]["max_query_len"] = cc["max_query_len"]
    out[2]["max_seq_len"] = cc["max_seq_len"]
    return out
