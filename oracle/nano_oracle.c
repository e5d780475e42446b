/*
 * Plain C oracle: the step compile written the way the nano-vllm runner builds
 * its prefill inputs, plus a row-by-row K/V scatter.
 *
 * TEST INFRASTRUCTURE ONLY: called from the tests and from the benchmark's
 * CPU-baseline leg, never from the product library.  Single-threaded scalar
 * loops; shares nothing with the HIP code.
 *
 * Sources:
 *   [P5] "Nano-VLLM全代码解析笔记(4)-model_runner": the prefill inputs cover
 *        each sequence from its cached length to cached + scheduled, with
 *        running totals of query and key lengths (cu_seqlens_q / _k), and the
 *        K/V slots come one physical block at a time as contiguous ranges
 *        (prepare_prefill; Q&A item 14 works such ranges by hand).  Written
 *        here as the intersection of each request's position interval with
 *        each block's interval.
 *   [P1] "vLLM 源码完全拆解（五）…" §第四步 (logits index = last token of each
 *        request) and §Chunked Prefill (partial prompts are discarded).
 *   [P3] "变长批处理与一次混合前向" §练习 1 (compacted logits list).
 * Pad-tail values follow the same readings as the Python oracle.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int32_t num_reqs;
    int32_t block_size;
    int32_t max_num_reqs;
    int32_t n_pad;
    int32_t null_block;
    int64_t tok_stride;        /* elements between token-table rows  */
    int64_t blk_stride;        /* elements between block-table rows  */
    const int32_t* num_computed;
    const int32_t* num_scheduled;
    const int32_t* num_prompt;
    const int32_t* tokens;     /* [num_reqs][tok_stride] */
    const int32_t* blocks;     /* [num_reqs][blk_stride] */
} nano_in;

typedef struct {
    int32_t* input_ids;        /* [n_pad] */
    int32_t* positions;        /* [n_pad] */
    int32_t* req_indices;      /* [n_pad] */
    int32_t* slot_mapping;     /* [n_pad] */
    int32_t* query_start_loc;  /* [max_num_reqs + 1] */
    int32_t* cu_seqlens_k;     /* [max_num_reqs + 1] */
    int32_t* seq_lens;         /* [max_num_reqs] */
    int32_t* logits_indices;   /* [max_num_reqs] */
    uint8_t* discard;          /* [max_num_reqs] */
    int32_t* sample_indices;   /* [max_num_reqs] */
    int32_t num_sampled;
    int32_t num_actual_tokens;
    int32_t max_seqlen_q;
    int32_t max_seqlen_k;
} nano_out;

/* Returns 0, or -1 when the padded size cannot hold the real tokens. */
int nano_compile(const nano_in* in, nano_out* out)
{
    const int32_t B = in->block_size;
    int32_t n = 0;                 /* tokens emitted so far */
    int32_t max_q = 0, max_k = 0;
    int32_t i, k;

    out->query_start_loc[0] = 0;
    out->cu_seqlens_k[0] = 0;
    for (i = 0; i < in->num_reqs; ++i) {
        const int32_t cached = in->num_computed[i];
        const int32_t fresh = in->num_scheduled[i];
        const int32_t total = cached + fresh;           /* key length after this step */
        const int32_t* history = in->tokens + (int64_t)i * in->tok_stride;
        const int32_t* owned = in->blocks + (int64_t)i * in->blk_stride;
        int32_t b;

        if (fresh > in->n_pad - n)
            return -1;
        out->query_start_loc[i + 1] = out->query_start_loc[i] + fresh;
        out->cu_seqlens_k[i + 1] = out->cu_seqlens_k[i] + total;
        out->seq_lens[i] = total;
        max_q = fresh > max_q ? fresh : max_q;
        max_k = total > max_k ? total : max_k;

        /* The new tokens are positions [cached, total) of the history. */
        for (k = 0; k < fresh; ++k) {
            out->input_ids[n + k] = history[cached + k];
            out->positions[n + k] = cached + k;
            out->req_indices[n + k] = i;
        }

        /* Their K/V slots, one physical block at a time: logical block b
         * covers positions [b*B, (b+1)*B); the part of [cached, total) that
         * falls inside it maps to consecutive slots of physical block
         * owned[b], at the same offsets within the block. */
        for (b = cached / B; b * B < total; ++b) {
            const int32_t lo = cached > b * B ? cached : b * B;
            const int32_t hi = total < (b + 1) * B ? total : (b + 1) * B;
            int32_t p;
            for (p = lo; p < hi; ++p)
                out->slot_mapping[n + (p - cached)] = owned[b] * B + (p - b * B);
        }
        n += fresh;

        out->logits_indices[i] = out->query_start_loc[i + 1] - 1;
        out->discard[i] = (uint8_t)(total < in->num_prompt[i] ? 1 : 0);
    }
    out->num_actual_tokens = n;
    out->max_seqlen_q = max_q;
    out->max_seqlen_k = max_k;

    /* Pseudo-requests past the real ones: empty query intervals. */
    for (i = in->num_reqs; i < in->max_num_reqs; ++i) {
        out->query_start_loc[i + 1] = n;
        out->cu_seqlens_k[i + 1] = out->cu_seqlens_k[in->num_reqs];
        out->seq_lens[i] = 0;
        out->logits_indices[i] = -1;
        out->discard[i] = 1;
    }
    /* Padded tokens: null block, neutral values. */
    for (k = n; k < in->n_pad; ++k) {
        out->input_ids[k] = 0;
        out->positions[k] = 0;
        out->req_indices[k] = -1;
        out->slot_mapping[k] = in->null_block * B;
    }
    /* Compacted list of the requests that may sample this step. */
    out->num_sampled = 0;
    for (i = 0; i < in->num_reqs; ++i)
        if (!out->discard[i])
            out->sample_indices[out->num_sampled++] = out->logits_indices[i];
    for (i = out->num_sampled; i < in->max_num_reqs; ++i)
        out->sample_indices[i] = -1;
    return 0;
}

/* K/V write: row t of each source goes to cache row slot[t]. */
void nano_kv_scatter(const uint8_t* k, const uint8_t* v, uint8_t* k_cache, uint8_t* v_cache,
                     const int32_t* slot, int32_t n, int64_t row_bytes)
{
    int32_t t;
    for (t = 0; t < n; ++t) {
        memcpy(k_cache + (int64_t)slot[t] * row_bytes, k + (int64_t)t * row_bytes, (size_t)row_bytes);
        memcpy(v_cache + (int64_t)slot[t] * row_bytes, v + (int64_t)t * row_bytes, (size_t)row_bytes);
    }
}

/* Hidden-state gather: out[m] = src[idx[m]], zero row for a negative index. */
void nano_gather(const uint8_t* src, int64_t row_bytes, const int32_t* idx, int32_t count,
                 uint8_t* out)
{
    int32_t m;
    for (m = 0; m < count; ++m) {
        if (idx[m] < 0)
            memset(out + (int64_t)m * row_bytes, 0, (size_t)row_bytes);
        else
            memcpy(out + (int64_t)m * row_bytes, src + (int64_t)idx[m] * row_bytes, (size_t)row_bytes);
    }
}
