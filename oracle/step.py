"""Plain per-token definition of one step's compile, K/V write and gather.

Test infrastructure only (see the package docstring).  Pure Python loops, one
token at a time, written so each line can be checked against the pages:

* query_start_loc is the running total of the per-request scheduled counts
  ([P1 §第一步：从每请求 token 数得到边界]; [P3 §布局与元数据]).
* token j of request i sits at model position c_i + j
  ([P1 §第二步：相对位置加已计算长度得到模型位置]).
* its input id is entry c_i + j of row i of the token table
  ([P1 §第三步：从二维 token 历史抽取本轮切片]).
* its K/V slot is block_table[i][p // B] * B + p % B
  ([P1 §Block table 是逐请求的页表], worked out in [P1 §3. 物理 KV 槽位]).
* seq_lens_i = c_i + q_i; logits index = last flat token of the request
  ([P1 §第四步：只在必要位置计算 logits]; [P2 §8.6.3]).
* a chunk that has not reached the end of the prompt is discarded
  ([P1 §Chunked Prefill：query 很长，但仍只是一段区间]); the compacted list
  keeps only requests that may sample ([P3 §练习 1. 元数据推导]).
* padding to a captured size: pseudo-requests get empty intervals and padded
  tokens go to the reserved null block ([P1 §固定地址与动态有效长度如何共存];
  [P4 §5. 关键细节与坑]).
* the t-th new K/V row is written to slot_mapping[t] with no request id
  involved ([P1 §3. 物理 KV 槽位]; [P3 §实现]).

Readings where the pages leave a value open:

* pad token t in [N, N_pad): input_id 0, position 0, req_index -1,
  slot null_block * B.
* pseudo-request i in [R, max_num_reqs): query_start_loc[i+1] = N,
  seq_len 0, logits index -1, discard 1, sample index -1.
* discard_i = (c_i + q_i < P_i), with P_i the prompt length.
"""
from __future__ import annotations

from typing import Dict, List, Sequence


class StepError(ValueError):
    """A precondition of the step does not hold."""


def padded_size(capture_sizes: Sequence[int], num_tokens: int) -> int:
    """Smallest captured size >= num_tokens; num_tokens itself above the
    largest one (the step then runs unpadded).
    [P2 §8.5.0.5 pad_for_cudagraph 的实现]; [P4 §3. 原理演示：向上取整的图派发]."""
    for s in sorted(capture_sizes):
        if s >= num_tokens:
            return s
    return num_tokens


def compile_step(rows, *, block_size: int, max_num_reqs: int, max_model_len: int,
                 max_num_batched_tokens: int, num_kv_blocks: int, n_pad: int,
                 null_block: int = 0, check_unique_slots: bool = True) -> Dict:
    """Compile the condensed rows 0..R-1 into the flat token stream.

    ``rows[i]`` has ``num_computed`` (c), ``num_scheduled`` (q), ``num_prompt``
    (P), ``tokens`` (the history, length T) and ``blocks`` (physical ids).
    Returns a dict of lists; per-request lists have ``max_num_reqs`` entries
    (query_start_loc has one more), per-token lists ``n_pad``.
    """
    R = len(rows)
    B = block_size
    if R > max_num_reqs:
        raise StepError("more requests than rows")
    for i, r in enumerate(rows):
        c, q, T = r.num_computed, r.num_scheduled, len(r.tokens)
        if q < 1:
            raise StepError(f"request {i}: nothing scheduled")
        if c < 0 or c + q > T:
            raise StepError(f"request {i}: scheduled range outside the token history")
        if T > max_model_len:
            raise StepError(f"request {i}: history longer than max_model_len")
        last_block = (c + q - 1) // B
        if last_block >= len(r.blocks):
            raise StepError(f"request {i}: too few blocks for position {c + q - 1}")
        for b in r.blocks[:last_block + 1]:
            if not (0 <= b < num_kv_blocks) or b == null_block:
                raise StepError(f"request {i}: block id {b} not a usable block")

    # query_start_loc: running total of the scheduled counts.
    qsl = [0]
    for r in rows:
        qsl.append(qsl[-1] + r.num_scheduled)
    N = qsl[R]
    if N > n_pad:
        raise StepError("padded size below the real token count")
    if n_pad > max_num_batched_tokens:
        raise StepError("padded size above the token budget")
    for _ in range(R, max_num_reqs):
        qsl.append(N)

    # Every flat token t in [0, N): its request owns the interval
    # [qsl[i], qsl[i+1]) that holds t; its offset inside that interval, added
    # to the request's cached length, is its model position; the position
    # picks the history entry and, split into a block index and an offset
    # inside the block, the physical K/V slot.
    input_ids: List[int] = []
    positions: List[int] = []
    req_indices: List[int] = []
    slot_mapping: List[int] = []
    owner = 0
    for t in range(N):
        while qsl[owner + 1] <= t:          # intervals are visited in order
            owner += 1
        r = rows[owner]
        pos = r.num_computed + (t - qsl[owner])
        block_index, within = divmod(pos, B)
        req_indices.append(owner)
        positions.append(pos)
        input_ids.append(int(r.tokens[pos]))
        slot_mapping.append(int(r.blocks[block_index]) * B + within)
    for _ in range(N, n_pad):
        input_ids.append(0)
        positions.append(0)
        req_indices.append(-1)
        slot_mapping.append(null_block * B)

    if check_unique_slots and len(set(slot_mapping[:N])) != N:
        raise StepError("two real tokens map to the same K/V slot")

    seq_lens, logits_indices, discard = [], [], []
    for i, r in enumerate(rows):
        seq_lens.append(r.num_computed + r.num_scheduled)
        logits_indices.append(qsl[i + 1] - 1)
        discard.append(1 if r.num_computed + r.num_scheduled < r.num_prompt else 0)
    sample_indices = [logits_indices[i] for i in range(R) if not discard[i]]
    num_sampled = len(sample_indices)
    for _ in range(R, max_num_reqs):
        seq_lens.append(0)
        logits_indices.append(-1)
        discard.append(1)
    sample_indices += [-1] * (max_num_reqs - num_sampled)

    # Key-side boundaries for a varlen attention call: running total of the
    # sequence lengths ([P5 prepare_prefill], Q&A item 8); pseudo-requests add 0.
    cu_seqlens_k = [0]
    for i in range(max_num_reqs):
        cu_seqlens_k.append(cu_seqlens_k[-1] + seq_lens[i])

    return dict(
        query_start_loc=qsl, seq_lens=seq_lens, cu_seqlens_k=cu_seqlens_k, logits_indices=logits_indices,
        discard=discard, sample_indices=sample_indices, num_sampled=num_sampled,
        input_ids=input_ids, positions=positions, req_indices=req_indices,
        slot_mapping=slot_mapping, num_reqs=R, num_actual_tokens=N, num_tokens_padded=n_pad,
        max_query_len=max((r.num_scheduled for r in rows), default=0),
        max_seq_len=max((r.num_computed + r.num_scheduled for r in rows), default=0),
    )


def reshape_and_cache(k_rows, v_rows, k_cache, v_cache, slot_mapping) -> None:
    """Copy K row t and V row t into cache row slot_mapping[t], one token at a
    time.  Rows are opaque byte strings (indexable objects whose items can be
    assigned).  [P1 §3. 物理 KV 槽位]; [P3 §实现] (kv.write before attention)."""
    for t, s in enumerate(slot_mapping):
        k_cache[s] = k_rows[t]
        v_cache[s] = v_rows[t]


def spec_decode_metadata(query_start_loc, input_ids, num_draft_tokens):
    """Logits positions when requests carry draft tokens.

    A request verifying d draft tokens needs logits at its last d + 1 flat
    positions: the rows at its first d of them check the drafts, the last one
    gives the bonus token; the drafts themselves are its last d input ids
    ([P1 §投机解码：一条请求一轮可能产生多个决策位置]; [P2 §8.6.3]).  With no
    drafts this is query_start_loc[1:] - 1.  Returns a dict of lists; indices
    into the logits rows are "target" (one per draft) and "bonus" (one per
    request)."""
    logits, cu, target, bonus, drafts = [], [0], [], [], []
    for i, d in enumerate(num_draft_tokens):
        end = query_start_loc[i + 1]
        for k in range(d + 1):
            logits.append(end - (d + 1) + k)
        for k in range(d):
            target.append(cu[-1] + k)
            drafts.append(int(input_ids[end - d + k]))
        cu.append(cu[-1] + d + 1)
        bonus.append(cu[-1] - 1)
    return dict(logits_indices=logits, cu_num_logits=cu, target_logits_indices=target,
                bonus_logits_indices=bonus, draft_token_ids=drafts)


def expand_kernel_blocks(manager_ids, ratio: int):
    """A manager block of ratio * Bk tokens over a kernel of block size Bk:
    manager id m stands for kernel ids m*ratio .. m*ratio + ratio - 1, in
    order ([P1 §混合 KV Cache：一条请求不止一张页表])."""
    out = []
    for m in manager_ids:
        for j in range(ratio):
            out.append(int(m) * ratio + j)
    return out


def padded_block_table(rows, width: int, fill: int = -1, ratio: int = 1, blocks_of=None):
    """Rows 0..R-1 of a block table (expanded to kernel blocks when ratio > 1)
    cut or padded to ``width`` entries with ``fill`` past each row's own
    blocks (nano-vllm's prepare_block_tables pads with -1 to the longest row)
    [P5 prepare_block_tables].  ``blocks_of(i, row)`` picks another group's
    block list (default: the row's own ``blocks``)."""
    out = []
    for i, r in enumerate(rows):
        ids = expand_kernel_blocks(r.blocks if blocks_of is None else blocks_of(i, r), ratio)
        out.append([ids[j] if j < len(ids) else fill for j in range(width)])
    return out


def group_slot_mapping(positions, req_indices, group_blocks, block_size: int, null_block: int = 0):
    """Slots of one further KV-cache group: the same token positions through
    that group's own block table and block size
    ([P1 §混合 KV Cache：一条请求不止一张页表]); padded tokens (req index -1)
    go to the group's null slot."""
    out = []
    for p, r in zip(positions, req_indices):
        if r < 0:
            out.append(null_block * block_size)
        else:
            out.append(int(group_blocks[r][p // block_size]) * block_size + p % block_size)
    return out


def append_sampled(rows_tokens, rows, src_index, sampled):
    """Append one sampled token per listed row: row rows[k] gets
    sampled[src_index[k]] at the end of its history (the async-scheduling
    input path keeps last step's sampled ids on the device and places them
    through a current-row -> previous-position map, [P1 §先拷 block table，再做 CPU 索引])."""
    for k, row in enumerate(rows):
        rows_tokens[row].append(int(sampled[src_index[k] if src_index is not None else k]))


def correct_computed(num_computed, rows_tokens, rows, prev_index, num_draft, num_accepted, sampled=None):
    """Correct optimistically advanced computed counts (asynchronous
    speculative decoding, [P1 §投机解码：一条请求一轮可能产生多个决策位置]).

    Last step row ``rows[k]`` fed its last token plus d = num_draft[k] drafts
    and was then scheduled again as if all d had been accepted, i.e. with its
    computed count advanced by d + 1.  The sampler, at position
    p = prev_index[k] of its output, kept v = num_accepted[p] tokens: the
    accepted drafts and one token of its own.  Only the first v of the d + 1
    fed positions hold K/V that stays valid, so the count drops by d + 1 - v.
    With ``sampled`` (one token list per sampler position), the last kept
    token sampled[p][v - 1] is written into the row's history at the
    corrected count: it is the row's first input of the new step.  A count v
    outside [1, d + 1] leaves the row unchanged; the number of such rows is
    returned.  ``num_computed`` and ``rows_tokens`` are indexed by row and
    updated in place."""
    bad = 0
    for k, row in enumerate(rows):
        p = prev_index[k]
        d = num_draft[k]
        v = int(num_accepted[p])
        if v < 1 or v > d + 1:
            bad += 1
            continue
        num_computed[row] -= d + 1 - v
        if sampled is not None:
            rows_tokens[row][num_computed[row]] = int(sampled[p][v - 1])
    return bad


def gather_rows(src_rows, indices, count: int, zero_row):
    """out[m] = src[indices[m]] for m < count; a negative index yields the zero
    row.  [P2 §8.7 execute_model：完整主流程] (hidden_states[logits_indices]);
    [P4 §4.1]."""
    out = []
    for m in range(count):
        idx = indices[m]
        out.append(zero_row if idx < 0 else src_rows[idx])
    return out
