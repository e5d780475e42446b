"""Reference persistent batch: row-compacted columns keyed by row number.

Test infrastructure only.  Follows the pages' description of the persistent
request batch:

* a request occupies one row; the row <-> request maps are inverses
  ([P1 §行号是一种短生命周期地址]; [P1 §八条必须成立的不变量], item 1);
* a new request takes a free row, gets its prompt tokens copied, its counters
  written, its block-table row installed and its sampling values recorded
  ([P1 §新请求建立完整状态]; [P2 §8.2.2 三种变更操作]); freed rows are reused
  before new rows are opened ([P2 §8.2.2.5 _update_states 的真实四段执行]);
* a resident request gets new block ids appended to its row; after a
  preemption its row is replaced, not appended ([P1 §驻留请求只合并差量]);
* removal leaves a hole; condense fills holes with rows from the tail, moving
  every column of the row together ([P1 §行号是一种短生命周期地址];
  [P1 §为什么删除后还要压紧]).

Reading: a new request takes the lowest free row; condense pairs
the k-th lowest hole with the k-th highest live row while the hole lies below
that row, which reproduces the A,B,C,D -> A,D,C example of the first page.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np


class BatchError(ValueError):
    pass


@dataclass
class RowState:
    req_id: int
    tokens: List[int]
    num_prompt: int
    num_computed: int
    num_scheduled: int
    blocks: List[int]
    sampling: Tuple[float, float, float, int] = (1.0, 1.0, 1.0, 0)  # temp, top_p, rep, top_k
    group_blocks: Dict[int, List[int]] = field(default_factory=dict)  # KV-cache groups 1..


@dataclass
class RefBatch:
    max_num_reqs: int
    max_model_len: int
    max_blocks_per_req: int
    num_kv_blocks: int
    null_block: int = 0
    rows: List[Optional[RowState]] = field(default_factory=list)
    row_of: Dict[int, int] = field(default_factory=dict)

    def __post_init__(self):
        self.rows = [None] * self.max_num_reqs

    # -- queries ---------------------------------------------------------
    def num_used_rows(self) -> int:
        used = [i for i, r in enumerate(self.rows) if r is not None]
        return used[-1] + 1 if used else 0

    def num_live(self) -> int:
        return sum(1 for r in self.rows if r is not None)

    def req_ids_by_row(self) -> List[Optional[int]]:
        return [None if r is None else r.req_id for r in self.rows]

    # -- mutations -------------------------------------------------------
    def _check_blocks(self, ids):
        for b in ids:
            if not (0 <= b < self.num_kv_blocks) or b == self.null_block:
                raise BatchError(f"block id {b} not usable")

    def add_request(self, req_id: int, tokens, num_prompt: int, num_computed: int, blocks,
                    sampling=(1.0, 1.0, 1.0, 0)) -> int:
        if req_id in self.row_of:
            raise BatchError("request id already live")
        if len(tokens) > self.max_model_len or len(blocks) > self.max_blocks_per_req:
            raise BatchError("row capacity exceeded")
        if not (0 <= num_prompt <= len(tokens)) or not (0 <= num_computed <= len(tokens)):
            raise BatchError("counters outside the token history")
        self._check_blocks(blocks)
        free = [i for i, r in enumerate(self.rows) if r is None]
        if not free:
            raise BatchError("no free row")
        row = free[0]
        self.rows[row] = RowState(req_id, [int(t) for t in tokens], int(num_prompt),
                                  int(num_computed), 0, [int(b) for b in blocks],
                                  tuple(sampling))
        self.row_of[req_id] = row
        return row

    def remove_request(self, req_id: int) -> int:
        if req_id not in self.row_of:
            raise BatchError("unknown request")
        row = self.row_of.pop(req_id)
        self.rows[row] = None
        return row

    def append_blocks(self, req_id: int, ids) -> None:
        r = self.rows[self.row_of[req_id]]
        if len(r.blocks) + len(ids) > self.max_blocks_per_req:
            raise BatchError("block row full")
        self._check_blocks(ids)
        r.blocks.extend(int(b) for b in ids)

    def replace_blocks(self, req_id: int, ids) -> None:
        r = self.rows[self.row_of[req_id]]
        if len(ids) > self.max_blocks_per_req:
            raise BatchError("block row full")
        self._check_blocks(ids)
        r.blocks = [int(b) for b in ids]

    def append_blocks_group(self, req_id: int, group: int, ids) -> None:
        """Blocks of a further KV-cache group (a request owns one table per
        group, [P1 §混合 KV Cache：一条请求不止一张页表]); new rows start empty."""
        self._check_blocks(ids)
        self.rows[self.row_of[req_id]].group_blocks.setdefault(group, []).extend(int(b) for b in ids)

    def replace_blocks_group(self, req_id: int, group: int, ids) -> None:
        self._check_blocks(ids)
        self.rows[self.row_of[req_id]].group_blocks[group] = [int(b) for b in ids]

    def append_tokens(self, req_id: int, ids) -> None:
        r = self.rows[self.row_of[req_id]]
        if len(r.tokens) + len(ids) > self.max_model_len:
            raise BatchError("token row full")
        r.tokens.extend(int(t) for t in ids)

    def truncate_tokens(self, req_id: int, num_tokens: int) -> None:
        """Keep the first num_tokens of the history: drafts that verification
        rejected leave it, since only the verified prefix is committed
        ([P1 §投机解码：一条请求一轮可能产生多个决策位置]).  The prompt stays."""
        r = self.rows[self.row_of[req_id]]
        if num_tokens < r.num_prompt or num_tokens > len(r.tokens):
            raise BatchError("truncation outside [num_prompt, num_tokens]")
        del r.tokens[num_tokens:]

    def condense_pairs(self) -> List[Tuple[int, int]]:
        """(hole, source) pairs: k-th lowest hole <- k-th highest live row,
        while the hole is below the row."""
        used = self.num_used_rows()
        holes = [i for i in range(used) if self.rows[i] is None]
        live = [i for i in range(used - 1, -1, -1) if self.rows[i] is not None]
        pairs = []
        for h, l in zip(holes, live):
            if h >= l:
                break
            pairs.append((h, l))
        return pairs

    def condense(self) -> List[Tuple[int, int]]:
        pairs = self.condense_pairs()
        for h, l in pairs:
            self.rows[h] = self.rows[l]
            self.rows[l] = None
            self.row_of[self.rows[h].req_id] = h
        return pairs

    def schedule(self, num_computed, num_scheduled) -> None:
        R = len(num_scheduled)
        if self.num_live() != R or self.num_used_rows() != R:
            raise BatchError("live rows are not exactly [0, R)")
        for i in range(R):
            self.rows[i].num_computed = int(num_computed[i])
            self.rows[i].num_scheduled = int(num_scheduled[i])

    # -- views -----------------------------------------------------------
    def step_rows(self):
        """Rows 0..R-1 as objects with the attributes ``step.compile_step`` reads."""
        out = []
        for r in self.rows[:self.num_used_rows()]:
            out.append(_StepRow(r.num_computed, r.num_scheduled, r.num_prompt,
                                np.asarray(r.tokens, dtype=np.int64),
                                np.asarray(r.blocks, dtype=np.int64)))
        return out


@dataclass
class _StepRow:
    num_computed: int
    num_scheduled: int
    num_prompt: int
    tokens: np.ndarray
    blocks: np.ndarray
