/*
 * ric.h - ragged input compilation for one step of a continuous-batching LLM
 * runner, on AMD Instinct MI355X (gfx950).
 *
 * One step: a persistent, row-compacted request batch (a device-resident column
 * store) is compiled into a flat 1-D token stream plus its attention metadata;
 * the step's new K/V rows are then written into a paged cache through the slot
 * mapping, and hidden states are gathered at the rows that produce logits.
 *
 * Sources, cited by page title and section:
 *   [P1] "vLLM 源码完全拆解（五）：GPUModelRunner 如何把动态请求拼成一次 GPU 前向"
 *   [P2] "第8章 ModelRunner：从 SchedulerOutput 到 GPU Kernel"
 *   [P3] "变长批处理与一次混合前向"
 *   [P4] "04 · 模型执行与 CUDA Graph"
 *   [P5] "Nano-VLLM全代码解析笔记(4)-model_runner"
 *
 * Conventions for every call:
 *   - Return value: RIC_OK (0) or a negative RIC_E* code.  On error nothing
 *     has changed (no host state, no device work enqueued) and
 *     ric_last_error() holds a message for the calling thread; the one
 *     exception is RIC_EHIP, a failure reported by the HIP runtime, which may
 *     come after part of a call's device work was enqueued.
 *   - "device" pointers are HIP device addresses (e.g. torch tensor
 *     data_ptr()); "host" pointers are ordinary host memory.  Host input arrays
 *     are read (and copied into pinned staging where needed) before the call
 *     returns, so the caller may reuse them at once.
 *   - Device work is enqueued on a HIP stream and is asynchronous.  No call on
 *     the step path (schedule, compile, reshape_and_cache, gather) waits for
 *     the device or copies device data to the host.
 *   - Integer values are int32; byte offsets are computed in 64 bits.
 *   - A handle belongs to the device that was current at ric_create; calls on
 *     it make that device current for their duration and restore the
 *     caller's.  Calls without a handle (ric_reshape_and_cache,
 *     ric_gather_rows) run on the current device, whose stream they take.
 *   - A handle is not thread-safe: one thread at a time per handle.
 */
#ifndef RIC_H
#define RIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RIC_OK      0
#define RIC_EINVAL (-1)  /* an argument or a step precondition is invalid      */
#define RIC_ENOMEM (-2)  /* device or pinned host allocation failed            */
#define RIC_EFULL  (-3)  /* no free row, or a row's token / block capacity     */
#define RIC_ENOENT (-4)  /* unknown request id                                 */
#define RIC_EEXIST (-5)  /* request id already live                            */
#define RIC_ERANGE (-6)  /* a value is outside the configured capacity         */
#define RIC_EHIP   (-7)  /* a HIP runtime call failed                          */
#define RIC_ESTATE (-8)  /* call order: e.g. compile without a fresh schedule  */

typedef struct ric_batch ric_batch;   /* opaque handle: column store + step buffers */

/* Capacities, fixed at creation. */
typedef struct {
    int32_t max_num_reqs;            /* rows of the persistent batch (<= 8000)            */
    int32_t max_model_len;           /* token-history capacity per row                    */
    int32_t block_size;              /* tokens per K/V block, B >= 1                      */
    int32_t max_blocks_per_req;      /* block-table capacity per row                      */
    int32_t max_num_batched_tokens;  /* capacity of the per-token outputs (padded count)  */
    int32_t num_kv_blocks;           /* physical blocks in the cache; num_kv_blocks*B < 2^31 */
    int32_t null_block;              /* reserved block for padded tokens (usually 0)      */
    int32_t staging_bytes;           /* pinned delta-staging capacity; 0 = default (4 MiB, more
                                        for large batches); at least 96*max_num_reqs + 64 KiB */
    /* KV-cache groups ([P1 §混合 KV Cache：一条请求不止一张页表]): a request can
     * own one block table per group (full attention, sliding window,
     * recurrent state...).  Group 0 is described by the fields above; groups
     * 1..num_kv_groups-1 by these arrays (index g).  Entry 0 of each array is
     * ignored. */
    int32_t num_kv_groups;           /* 1..4; 0 means 1 */
    int32_t group_block_size[4];     /* block size of group g; its table holds
                                        ceil(max_model_len / block size) entries */
    int32_t group_num_kv_blocks[4];  /* pool size of group g (0: num_kv_blocks); block
                                        null_block is reserved in every pool      */
    int32_t group_slot_mode[4];      /* RIC_SLOTS_PER_TOKEN: compile emits slots for
                                        group g; RIC_SLOTS_NONE: no slots (e.g. a
                                        recurrent-state group, SlotMappingMode.NONE) */
} ric_config;

#define RIC_MAX_KV_GROUPS   4
#define RIC_SLOTS_PER_TOKEN 0
#define RIC_SLOTS_NONE      1

/* Per-request sampling values.  They live in the column store and move with
 * their row; sampling itself is not part of this library.  [P2 §8.2.1]. */
typedef struct {
    float temperature;
    float top_p;
    float repetition_penalty;
    int32_t top_k;
} ric_sampling;

/* Outputs of ric_compile.  The device pointers are owned by the handle, keep
 * the same address for the handle's lifetime and are rewritten by every
 * compile (fixed-address buffers with a valid prefix, [P1 §固定地址与动态有效长度如何共存]).
 * Per-token arrays hold max_num_batched_tokens entries, of which the first
 * num_tokens_padded are written; per-request arrays hold max_num_reqs entries
 * (query_start_loc one more), all written. */
typedef struct {
    int32_t* input_ids;        /* [t] token id at position positions[t] of request req_indices[t]; pad: 0 */
    int32_t* positions;        /* [t] c_r + (t - qsl[r]); pad: 0                                */
    int32_t* req_indices;      /* [t] row r owning token t; pad: -1                              */
    int32_t* slot_mapping;     /* [t] block_table[r][p/B]*B + p%B; pad: null_block*B             */
    int32_t* query_start_loc;  /* [i] exclusive prefix sum of q; entries past R hold N           */
    int32_t* seq_lens;         /* [i] c_i + q_i; 0 past R                                        */
    int32_t* logits_indices;   /* [i] qsl[i+1]-1; -1 past R                                      */
    uint8_t* discard;          /* [i] 1 if c_i + q_i < prompt_i (partial prefill); 1 past R      */
    int32_t* sample_indices;   /* logits_indices of the rows with discard == 0, in row order; -1 after */
    int32_t* dev_scalars;      /* [8] device: R, N, N_pad, max_query_len, max_seq_len, num_sampled,
                                  [6] tokens whose column data was out of range since creation
                                  (always 0 unless device memory was corrupted), [7] sampled
                                  tokens whose source index was out of range since creation */
    int32_t* cu_seqlens_k;     /* [i] running total of seq_lens: key-side boundaries of a varlen
                                  attention call ([P5 prepare_prefill], Q&A item 8); entries past R
                                  hold the total.  [max_num_reqs + 1]                              */
    int32_t* group_slot_mapping[4]; /* [g] slots of KV-cache group g through its own table and
                                  block size (pad: null_block * its block size); [0] is
                                  slot_mapping; NULL for RIC_SLOTS_NONE groups and g >= groups */
    /* host values of this step (from the host mirror of the counters) */
    int32_t num_reqs;          /* R */
    int32_t num_actual_tokens; /* N = sum of q */
    int32_t num_tokens_padded; /* N_pad */
    int32_t max_query_len;
    int32_t max_seq_len;
    int32_t num_sampled;
    int32_t kv_path;           /* which launches this call made: 0 the compile only (ric_compile),
                                  1 the compile and the K/V write in one kernel, 2 the compile
                                  kernel followed by the K/V kernel (ric_compile_and_cache) */
} ric_step;

/* Device views of the column store (for inspection and tests).  Row r of the
 * token table starts at tokens + r*token_stride; of the block table at
 * blocks + r*block_stride.  Scalar columns hold max_num_reqs entries each. */
typedef struct {
    int32_t* tokens;           /* [max_num_reqs][token_stride] int32 */
    int32_t* blocks;           /* [max_num_reqs][block_stride] int32 */
    int64_t token_stride;
    int64_t block_stride;
    int32_t* num_tokens;       /* T_r: valid history length       */
    int32_t* num_prompt;       /* P_r                              */
    int32_t* num_computed;     /* c_r (from the last schedule)     */
    int32_t* num_scheduled;    /* q_r (from the last schedule)     */
    int32_t* num_blocks;       /* valid block-table entries        */
    int32_t* top_k;
    float* temperature;
    float* top_p;
    float* repetition_penalty;
    /* KV-cache groups: [g] block table, its row stride and its per-row valid
     * count; [0] repeats blocks / block_stride / num_blocks; NULL and 0 for
     * g >= num_kv_groups. */
    int32_t* group_blocks[4];
    int64_t group_block_stride[4];
    int32_t* group_num_blocks[4];
} ric_columns;

/* ---- handle -------------------------------------------------------------- */

/* Device bytes a handle needs for `cfg` (column store + step outputs + staging). */
size_t ric_workspace_bytes(const ric_config* cfg);

/* Create a handle.  `stream` (hipStream_t, may be NULL for the default stream)
 * orders all of the handle's device work.  `workspace` is a device buffer of at
 * least ric_workspace_bytes(cfg) bytes owned by the caller (e.g. a torch
 * tensor), or NULL for the library to allocate its own.  The pinned host
 * staging is always allocated by the library.  Errors: EINVAL (capacities),
 * ENOMEM, EHIP. */
int ric_create(const ric_config* cfg, void* stream, void* workspace, size_t workspace_bytes,
               ric_batch** out);

/* Wait for the handle's stream, free what the library allocated.  A NULL
 * handle is accepted. */
int ric_destroy(ric_batch* b);

/* Change the stream later calls enqueue on.  Waits first for the work already
 * enqueued on the previous stream, so nothing later can overtake it. */
int ric_set_stream(ric_batch* b, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* ric_last_error(void);

/* ---- column-store deltas ([P1 §新请求建立完整状态], [P1 §驻留请求只合并差量],
 *      [P2 §8.2.2 三种变更操作]).  Each call updates the host mirror at once and
 *      stages its payload; staged payloads reach the device column store at
 *      the next flush (explicit ric_flush, ric_condense or ric_compile, or when
 *      staging fills) through one scatter kernel, which reads a log of up to
 *      64 KiB straight from the pinned host staging and a larger one after
 *      one copy into device staging. */

/* Install a new request in the lowest free row: token history tokens[0,T),
 * prompt length, computed count, block ids blocks[0,nb) (each in
 * [0, num_kv_blocks) and not the null block), sampling values (NULL: 1,1,1,0).
 * A request aborted and resubmitted under the same id must be removed first
 * ([P2 §8.2.2.6]).  Errors: EEXIST, EFULL (no free row), ERANGE (T >
 * max_model_len, nb > max_blocks_per_req, counts outside [0,T], bad block id). */
int ric_add_request(ric_batch* b, uint64_t req_id, const int32_t* tokens, int32_t num_tokens,
                    int32_t num_prompt, int32_t num_computed, const int32_t* blocks,
                    int32_t num_blocks, const ric_sampling* sampling, int32_t* out_row);

/* Remove a request (finished, or unscheduled/preempted): its row becomes a
 * hole until ric_condense or a later add fills it.  Errors: ENOENT. */
int ric_remove_request(ric_batch* b, uint64_t req_id, int32_t* out_row);

/* Append new token ids to the request's history.  Errors: ENOENT, EFULL. */
int ric_append_tokens(ric_batch* b, uint64_t req_id, const int32_t* ids, int32_t n);

/* Keep the first num_tokens of the request's history, dropping the rest
 * (drafts that verification rejected: only the verified prefix is committed,
 * [P1 §投机解码：一条请求一轮可能产生多个决策位置]).  Only the count changes;
 * the dropped entries are overwritten by later appends.  Errors: ENOENT,
 * ERANGE (num_tokens below the prompt length or above the history). */
int ric_truncate_tokens(ric_batch* b, uint64_t req_id, int32_t num_tokens);

/* Append newly allocated block ids to the request's block-table row.
 * Errors: ENOENT, EFULL, ERANGE (bad block id). */
int ric_append_blocks(ric_batch* b, uint64_t req_id, const int32_t* ids, int32_t n);

/* Replace the whole block-table row (a request resumed after preemption: its
 * old ids are no longer valid, [P1 §驻留请求只合并差量]).  Errors as append. */
int ric_replace_blocks(ric_batch* b, uint64_t req_id, const int32_t* ids, int32_t n);

/* The same two calls for KV-cache group `group` (0 is the calls above).  A new
 * request's rows in groups >= 1 start empty.  Errors as above, plus EINVAL for
 * a group outside [0, num_kv_groups). */
int ric_append_blocks_group(ric_batch* b, uint64_t req_id, int32_t group, const int32_t* ids, int32_t n);
int ric_replace_blocks_group(ric_batch* b, uint64_t req_id, int32_t group, const int32_t* ids, int32_t n);

/* Fill holes so the live rows are exactly [0, R): the k-th lowest hole
 * receives the k-th highest live row while the hole lies below it, and every
 * column of a moved row moves with it (token history, block row, counters,
 * sampling values) in one kernel ([P1 §行号是一种短生命周期地址],
 * [P1 §为什么删除后还要压紧]).  *out_num_moved = rows moved.  Flushes staged
 * deltas first. */
int ric_condense(ric_batch* b, int32_t* out_num_moved);

/* Upload staged deltas now.  Uploads are refused with ESTATE (nothing
 * changes) while the handle's stream is being captured into a graph: every
 * call that flushes (this one, ric_condense, ric_compile, ric_append_sampled,
 * ric_spec_decode_metadata, ric_correct_computed, ric_block_table_padded)
 * must find the log empty during a capture, so flush before capturing. */
int ric_flush(ric_batch* b);

/* Append one token per listed row from a DEVICE array: last step's sampled ids
 * stay on the GPU instead of travelling to the host and back; rows are matched
 * to sample positions by a current-row -> previous-position map
 * ([P1 §先拷 block table，再做 CPU 索引], the async-scheduling input path).
 *   rows       HOST int32[n]: live rows receiving a token, each at most once
 *   src_index  HOST int32[n]: row rows[k] takes dev_tokens[src_index[k]]
 *              (NULL: dev_tokens[k])
 *   dev_tokens DEVICE int32[dev_tokens_len], ready on the handle's stream
 * Each listed row's token count grows by one at once on the host; the values
 * are written on the device (this call flushes staged deltas).  Errors: EINVAL
 * (row not live or repeated, index out of range), EFULL (history full). */
int ric_append_sampled(ric_batch* b, int32_t n, const int32_t* rows, const int32_t* src_index,
                       const int32_t* dev_tokens, int32_t dev_tokens_len);

/* Logits positions when requests carry draft tokens (speculative decoding,
 * [P1 §投机解码：一条请求一轮可能产生多个决策位置], [P2 §8.6.3]).  Row i verifies
 * d_i = num_draft_tokens[i] drafts, which are its last d_i scheduled tokens
 * (d_i + 1 <= q_i).  Its logits are needed at its last d_i + 1 flat
 * positions: the first d_i of those rows check the drafts, the last gives the
 * bonus token.  All arrays are device, owned by the handle, stable:
 *   logits_indices[num_logits]        flat positions, request by request
 *   cu_num_logits[R+1]                running total of (d_i + 1)
 *   target_logits_indices[num_draft]  logits row that checks each draft
 *   bonus_logits_indices[R]           logits row of each request's bonus token
 *   draft_token_ids[num_draft]        the draft ids (from input_ids)
 * With all d_i = 0 logits_indices equals ric_step.logits_indices[0..R). */
typedef struct {
    int32_t* logits_indices;
    int32_t* cu_num_logits;
    int32_t* target_logits_indices;
    int32_t* bonus_logits_indices;
    int32_t* draft_token_ids;
    int32_t num_logits;        /* sum of (d_i + 1) */
    int32_t num_draft_tokens;  /* sum of d_i */
} ric_spec_decode;

/* Build the speculative-decoding indices for the last compiled step from HOST
 * draft counts num_draft_tokens[R].  Errors: ESTATE (no compile of the current
 * schedule), EINVAL (d_i < 0 or d_i + 1 > q_i). */
int ric_spec_decode_metadata(ric_batch* b, const int32_t* num_draft_tokens, ric_spec_decode* out);

/* Correct this step's computed counts on the device when they were scheduled
 * optimistically (asynchronous speculative decoding, [P1 §投机解码：一条请求一轮
 * 可能产生多个决策位置]).  Last step row rows[k] fed its last token plus
 * d = num_draft[k] drafts, and ric_schedule was given its count advanced by
 * d + 1, as if every draft had been accepted.  The sampler kept
 * v = dev_num_accepted[p] tokens for it (the accepted drafts plus one of its
 * own), p = prev_index[k] being the row's position in the sampler's output, so
 * only v of those d + 1 positions hold valid K/V.  On the device, before the
 * compile reads it:
 *     c <- c - (d + 1 - v)
 * and, when dev_sampled is given, dev_sampled[p * sampled_stride + v - 1] (the
 * last kept token, the row's first input of this step) is written into the
 * row's token history at the corrected c.  The host never sees v: positions,
 * seq_lens, slot mappings, discard, cu_seqlens_k and the device scalars of the
 * next ric_compile follow the corrected counts with no device-to-host copy.
 *   rows, prev_index, num_draft  HOST int32[n]; rows distinct, in [0, R)
 *   dev_num_accepted  DEVICE int32[prev_len], ready on the handle's stream
 *   dev_sampled       DEVICE int32[prev_len][sampled_stride] or NULL;
 *                     sampled_stride >= d + 1 for every listed row
 *   dev_status        optional DEVICE int32: incremented once per row whose v
 *                     lies outside [1, d + 1]; that row keeps its count and
 *                     gets no token
 * Call it after ric_schedule and before ric_compile, at most once per
 * schedule.  The host mirror keeps the scheduled counts: every check made on
 * them still holds for the lower corrected counts, and ric_step's host
 * max_seq_len and num_sampled are computed from them (an upper bound, and the
 * count before correction); dev_scalars hold the corrected values.  The
 * caller passes the corrected counts to its next ric_schedule once it knows
 * them.  Errors: ESTATE (no schedule, already compiled or corrected), EINVAL
 * (row not scheduled or repeated, position outside [0, prev_len), d < 0 or
 * d above the row's scheduled count, sampled_stride too small). */
int ric_correct_computed(ric_batch* b, int32_t n, const int32_t* rows, const int32_t* prev_index,
                         const int32_t* num_draft, const int32_t* dev_num_accepted, int32_t prev_len,
                         const int32_t* dev_sampled, int64_t sampled_stride, int32_t* dev_status);

/* Dense block table of KV-cache group `group` for an attention call that
 * wants one: rows 0..R-1 of the scheduled batch, `width` entries each.
 * With kernel_blocks_per_block = k > 1 every stored id m is expanded to the k
 * kernel block ids m*k .. m*k+k-1 (a manager block of k*Bk tokens over a
 * kernel of block size Bk, [P1 §混合 KV Cache]: [0,1,2] -> [0..5] for k = 2).
 * Entries past a row's own (expanded) blocks are set to `fill` (nano-vllm pads
 * with -1, [P5 prepare_block_tables]).  dst: DEVICE int32[R][width],
 * width <= k * the group's table capacity, and k * the group's pool size must
 * stay below 2^31 (expanded ids are int32).  The persistent tables themselves
 * (ric_get_columns: group_blocks[g]) can be used directly when stale entries
 * past each row's count are acceptable.  Errors: ESTATE (no schedule since the
 * last row change), EINVAL. */
int ric_block_table_padded(ric_batch* b, int32_t group, int32_t kernel_blocks_per_block, int32_t width,
                           int32_t fill, int32_t* dst);

/* Number of live requests; row of a request (or RIC_ENOENT); request at a row
 * (RIC_ENOENT for a hole). */
int32_t ric_num_reqs(const ric_batch* b);
int32_t ric_row_of(const ric_batch* b, uint64_t req_id);
int ric_req_at(const ric_batch* b, int32_t row, uint64_t* out_req_id);

/* Device views of the columns. */
int ric_get_columns(const ric_batch* b, ric_columns* out);

/* Wait until the handle's stream is idle (tests, teardown; not a step call). */
int ric_sync(ric_batch* b);

/* Inspection (tests, debugging; not a step call): wait for the device, then
 * copy `bytes` from a DEVICE address to HOST memory.  Errors: EINVAL, EHIP. */
int ric_read_device(void* host_dst, const void* dev_src, size_t bytes);

/* ---- step ---------------------------------------------------------------- */

/* This step's counts for rows 0..R-1 (host arrays of R entries): cached
 * length c_i and scheduled count q_i ([P1 §第一步], [P1 §第二步]).  Checked
 * in O(R) against the host mirror: live rows are exactly [0,R) (condensed),
 * q_i >= 1, c_i >= 0, c_i + q_i <= T_i, ceil((c_i+q_i)/B) <= blocks of row i,
 * sum q_i <= max_num_batched_tokens.  Errors: EINVAL, ESTATE (holes). */
int ric_schedule(ric_batch* b, int32_t num_reqs, const int32_t* num_computed,
                 const int32_t* num_scheduled);

/* Compile the scheduled batch into the flat token stream and its metadata in
 * one kernel: query_start_loc, req_indices, positions, input_ids, slot_mapping,
 * seq_lens, logits_indices, discard, sample_indices and the device scalars
 * ([P1 §第一步..第四步], [P1 §Block table 是逐请求的页表], [P3 §布局与元数据]).
 * Tokens [N, num_tokens_padded) are padding: they map to the null block
 * ([P1 §固定地址与动态有效长度如何共存], [P4 §5]).  Requires a ric_schedule
 * since the last row-changing call.  A compile captured into a graph replays
 * the R and num_tokens_padded it was captured with (the counts themselves are
 * read from the device columns at replay), and needs an empty delta log at
 * capture (see ric_flush).  Errors: ESTATE, EINVAL (N > N_pad or
 * N_pad > max_num_batched_tokens). */
int ric_compile(ric_batch* b, int32_t num_tokens_padded, ric_step* out);

/* ric_compile followed by ric_reshape_and_cache of the step's group-0 slot
 * mapping over all num_tokens_padded tokens, on the handle's stream, with
 * the same outputs and cache contents as those two calls
 * ([P1 §3. 物理 KV 槽位], [P3 §实现]: each token's K/V row goes to the slot the
 * compile gives it).  For rows of 128 B, 256 B, 512 B, 1, 2, 3, 4, 6 or 8 KiB the compile and
 * the K/V write of up to 32 layers are one kernel: each workgroup derives its
 * own tokens' slots and copies their rows, so there is no second launch to
 * wait for.  flags picks the path: 0 lets the library choose (the single
 * kernel, except for steps with rows of 1 KiB or more whose scheduled tokens
 * average 1024 or more per request: those long contiguous runs go through
 * the compile kernel and the K/V kernel, which measured faster whenever
 * other kernels ran just before), RIC_FUSE_ALWAYS asks for the single kernel
 * (with a tile shape of its own for such long runs, faster only in calls
 * made back to back), RIC_FUSE_NEVER for the two kernels; any other bit is
 * EINVAL.  Other row sizes and layers past 32 use the separate K/V kernel
 * after the compile.  The other
 * K/V arguments are those of ric_reshape_and_cache (k, v, k_cache, v_cache:
 * host arrays of num_layers device pointers; src_row_stride 0 = row_bytes;
 * dev_status optional; num_slots the cache rows, a slot outside [0,
 * num_slots) skips its row and counts in *dev_status).  Each source holds
 * num_tokens_padded rows and must be ready on the handle's stream when the
 * call is made: the single kernel reads the rows while it compiles.  Padded
 * tokens write their rows into the null block, as ric_reshape_and_cache does
 * with the padded slot mapping.  Errors: those of ric_compile and of
 * ric_reshape_and_cache; on an argument error nothing is enqueued. */
#define RIC_FUSE_ALWAYS 1u
#define RIC_FUSE_NEVER  2u
int ric_compile_and_cache(ric_batch* b, int32_t num_tokens_padded, const void* const* k, const void* const* v,
                          void* const* k_cache, void* const* v_cache, int32_t num_layers, int64_t src_row_stride,
                          int32_t row_bytes, int64_t num_slots, int32_t* dev_status, uint32_t flags,
                          ric_step* out);

/* Write the step's new K/V rows into paged caches through a slot mapping
 * ([P1 §3. 物理 KV 槽位], [P3 §实现]: the t-th row goes to slot_mapping[t]).
 *   k[l], v[l]        host arrays of num_layers DEVICE pointers: source row t
 *                     starts at k[l] + t*src_row_stride (bytes; 0 = row_bytes)
 *   k_cache[l], v_cache[l]  host arrays of DEVICE pointers: cache row s starts
 *                     at k_cache[l] + s*row_bytes; s < num_slots
 *                     (layout [num_blocks, B, kv_heads, head_dim])
 *   slot_mapping      DEVICE int32[num_tokens]
 *   row_bytes         bytes of one token's K (or V) row; multiple of 16;
 *                     src_row_stride and every pointer 16-byte aligned
 *   dev_status        optional DEVICE int32: incremented once per row whose
 *                     slot is outside [0, num_slots) (that row is not written)
 *   flags             reserved for launch hints; pass 0 (anything else is
 *                     EINVAL)
 * Up to 32 layers are written by one launch (more layers: one launch per 32).
 * num_tokens <= 2^24 per call.
 * Errors: EINVAL (alignment, counts, unknown flags), EHIP. */
int ric_reshape_and_cache(const void* const* k, const void* const* v, void* const* k_cache,
                          void* const* v_cache, int32_t num_layers, const int32_t* slot_mapping,
                          int32_t num_tokens, int64_t src_row_stride, int32_t row_bytes,
                          int64_t num_slots, int32_t* dev_status, uint32_t flags, void* stream);

/* Gather rows: dst[m] = src[idx[m]] for m < count, where count = *dev_count
 * (DEVICE int32, e.g. ric_step.dev_scalars + 5 for the compacted list) or
 * max_rows when dev_count is NULL.  A negative index yields a zero row; an
 * index >= src_rows yields a zero row and bumps *dev_status if given.  Rows
 * m in [count, max_rows) of dst are left untouched.  Used for hidden states at
 * logits_indices / sample_indices ([P2 §8.7], [P4 §4.1]).  Pointers and
 * strides 16-byte aligned, row_bytes a multiple of 16, max_rows <= 2^24.
 * Errors: EINVAL, EHIP. */
int ric_gather_rows(const void* src, int64_t src_row_stride, int64_t src_rows,
                    const int32_t* idx, const int32_t* dev_count, int32_t max_rows,
                    int32_t row_bytes, void* dst, int64_t dst_row_stride, int32_t* dev_status,
                    void* stream);

/* Slot-collision check of a step's slot mapping (a debugging aid, not a step
 * call).  Every real token must own its cache slot: two tokens writing one
 * slot would leave a K/V row that depends on the order of the writes (each
 * block has a single owner, [P1 §八条必须成立的不变量], item 7).  For the first n slots, n =
 * num_tokens, or min(num_tokens, *dev_num_tokens) when dev_num_tokens (a
 * DEVICE int32, e.g. ric_step.dev_scalars + 1 for N) is given:
 *   dev_result[0] += tokens whose slot an earlier-checked token of the same
 *                    call also holds (k tokens on one slot add k - 1)
 *   dev_result[1] += slots outside [0, num_slots)
 * dev_result is a DEVICE int32[2] the caller zeroes.  Pass the real token
 * count N, not the padded one: padded tokens all share the null block.
 *   workspace  DEVICE buffer of at least ric_check_slots_workspace_bytes(
 *              num_slots) bytes (a bitmap of one bit per slot), 4-byte
 *              aligned, owned by the caller, cleared by the call itself
 * Two launches on `stream`; nothing is read back.  Errors: EINVAL (counts,
 * NULL or misaligned pointers, workspace too small), EHIP. */
size_t ric_check_slots_workspace_bytes(int64_t num_slots);   /* 0 if num_slots outside [1, 2^31] */
int ric_check_slots(const int32_t* slot_mapping, int32_t num_tokens, const int32_t* dev_num_tokens,
                    int64_t num_slots, void* workspace, size_t workspace_bytes, int32_t* dev_result,
                    void* stream);

/* ric_check_slots for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same check and counts, with the bitmap in a static device array of the
 * library (4 MiB on each GPU it runs on, held until the process ends) instead
 * of a workspace.  Runs on the current device.  Calls no allocator.  Every
 * call on one GPU shares that GPU's bitmap, which each call clears (with a
 * kernel) before use: calls that overlap on one GPU, on different streams or
 * threads, race and must be serialised by the caller.
 * Errors: ERANGE (num_slots above RIC_CHECK_SLOTS_NOALLOC_MAX_SLOTS), EINVAL,
 * EHIP. */
#define RIC_CHECK_SLOTS_NOALLOC_MAX_SLOTS (1LL << 25)
int ric_check_slots_noalloc(const int32_t* slot_mapping, int32_t num_tokens, const int32_t* dev_num_tokens,
                            int64_t num_slots, int32_t* dev_result, void* stream);

/* ---- host-only helpers (no device work) ----------------------------------- */

/* Smallest of the n capture sizes >= num_tokens; num_tokens itself when it
 * exceeds them all ([P2 §8.5.0.5], [P4 §3]).  Sizes need not be sorted.
 * Returns RIC_EINVAL for num_tokens < 0 or n < 0. */
int32_t ric_padded_size(const int32_t* capture_sizes, int32_t n, int32_t num_tokens);

/* Condense plan for a row-occupancy mask live[0..num_rows): writes the
 * (hole, source) pairs the handle would use and returns their count. */
int32_t ric_condense_plan(const uint8_t* live, int32_t num_rows, int32_t* holes,
                          int32_t* sources);

/* Check a step against the rules of ric_schedule/ric_compile from host
 * counters of rows 0..R-1 (c, q, prompt P, history T, blocks nb) and fill the
 * host scalars of *out (device pointers left NULL).  Returns RIC_OK or the
 * error the handle would return. */
int ric_check_step(const ric_config* cfg, int32_t num_reqs, const int32_t* num_computed,
                   const int32_t* num_scheduled, const int32_t* num_prompt,
                   const int32_t* num_tokens, const int32_t* num_blocks,
                   int32_t num_tokens_padded, ric_step* out);

#ifdef __cplusplus
}
#endif

#endif /* RIC_H */
