/* One step through the C ABI from plain C (no C++, no Python): the worked
 * example of the first page ("vLLM 源码完全拆解（五）…", sections 1-5: three
 * requests, block size 4), compiled and its K/V rows written (by the two
 * separate calls, then again by ric_compile_and_cache), outputs printed
 * as one JSON object for the test that runs this program to compare with the
 * page's values.  Device memory for the K/V sources and caches comes from the
 * HIP runtime's C API; everything else goes through ric.h. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ric.h"

#define ROW2 128   /* rows the single compile + K/V kernel takes */

#define CHECK(x)                                                                     \
    do {                                                                             \
        int rc_ = (x);                                                               \
        if (rc_ != 0) {                                                              \
            fprintf(stderr, "%s failed: %d %s\n", #x, rc_, ric_last_error());        \
            exit(1);                                                                 \
        }                                                                            \
    } while (0)

static void print_array(const char* name, const int32_t* dev, int n, int last) {
    int32_t host[64];
    CHECK(ric_read_device(host, dev, (size_t)n * 4));
    printf("\"%s\": [", name);
    for (int i = 0; i < n; ++i) printf("%s%d", i ? ", " : "", host[i]);
    printf("]%s\n", last ? "" : ",");
}

int main(void) {
    enum { B = 4, R = 3, NPAD = 8, ROW = 64, SLOTS = 16 * B };
    ric_config cfg;
    memset(&cfg, 0, sizeof cfg);
    cfg.max_num_reqs = 4;
    cfg.max_model_len = 16;
    cfg.block_size = B;
    cfg.max_blocks_per_req = 4;
    cfg.max_num_batched_tokens = NPAD;
    cfg.num_kv_blocks = 16;
    cfg.null_block = 0;
    cfg.num_kv_groups = 1;

    ric_batch* b = NULL;
    CHECK(ric_create(&cfg, NULL, NULL, 0, &b));

    /* A: 5 cached + 1 decode; B: a 3-token prompt chunk of a longer prompt;
     * C: 8 cached + 2 new.  Token p of request k is 1000*(k+1) + p. */
    const int32_t c[R] = {5, 0, 8}, q[R] = {1, 3, 2}, P[R] = {4, 5, 10};
    const int32_t blocks[R][3] = {{7, 2, 0}, {5, 0, 0}, {8, 9, 4}};
    const int32_t nblocks[R] = {2, 1, 3};
    for (int k = 0; k < R; ++k) {
        int32_t tokens[16];
        const int32_t T = P[k] > c[k] + q[k] ? P[k] : c[k] + q[k];
        for (int p = 0; p < T; ++p) tokens[p] = 1000 * (k + 1) + p;
        int32_t row = -1;
        CHECK(ric_add_request(b, (uint64_t)(k + 1), tokens, T, P[k], c[k], blocks[k], nblocks[k], NULL, &row));
        if (row != k) {
            fprintf(stderr, "request %d landed in row %d\n", k, row);
            return 1;
        }
    }
    CHECK(ric_schedule(b, R, c, q));
    ric_step s;
    CHECK(ric_compile(b, NPAD, &s));

    /* K/V: one layer, 64-byte rows; source row t holds bytes equal to t + 1. */
    void *k_src, *v_src, *k_cache, *v_cache;
    if (hipMalloc(&k_src, NPAD * ROW) || hipMalloc(&v_src, NPAD * ROW) || hipMalloc(&k_cache, SLOTS * ROW) ||
        hipMalloc(&v_cache, SLOTS * ROW)) {
        fprintf(stderr, "hipMalloc failed\n");
        return 1;
    }
    uint8_t host[NPAD * ROW];
    for (int t = 0; t < NPAD; ++t) memset(host + t * ROW, t + 1, ROW);
    if (hipMemcpy(k_src, host, sizeof host, hipMemcpyHostToDevice) ||
        hipMemcpy(v_src, host, sizeof host, hipMemcpyHostToDevice) || hipMemset(k_cache, 0, SLOTS * ROW) ||
        hipMemset(v_cache, 0, SLOTS * ROW)) {
        fprintf(stderr, "hipMemcpy failed\n");
        return 1;
    }
    const void* ks[1] = {k_src};
    const void* vs[1] = {v_src};
    void* kc[1] = {k_cache};
    void* vc[1] = {v_cache};
    CHECK(ric_reshape_and_cache(ks, vs, kc, vc, 1, s.slot_mapping, NPAD, 0, ROW, SLOTS, NULL, 0, NULL));

    /* First byte of every cache row: 0 if untouched, else 1 + the source token. */
    uint8_t cache_host[SLOTS * ROW];
    CHECK(ric_read_device(cache_host, k_cache, sizeof cache_host));

    /* The same step again through ric_compile_and_cache, with 128-byte rows
     * (compile and K/V write in one kernel), into caches of their own. */
    void *k2_src, *v2_src, *k2_cache, *v2_cache;
    if (hipMalloc(&k2_src, NPAD * ROW2) || hipMalloc(&v2_src, NPAD * ROW2) || hipMalloc(&k2_cache, SLOTS * ROW2) ||
        hipMalloc(&v2_cache, SLOTS * ROW2)) {
        fprintf(stderr, "hipMalloc failed\n");
        return 1;
    }
    uint8_t host2[NPAD * ROW2];
    for (int t = 0; t < NPAD; ++t) memset(host2 + t * ROW2, t + 1, ROW2);
    if (hipMemcpy(k2_src, host2, sizeof host2, hipMemcpyHostToDevice) ||
        hipMemcpy(v2_src, host2, sizeof host2, hipMemcpyHostToDevice) || hipMemset(k2_cache, 0, SLOTS * ROW2) ||
        hipMemset(v2_cache, 0, SLOTS * ROW2)) {
        fprintf(stderr, "hipMemcpy failed\n");
        return 1;
    }
    const void* ks2[1] = {k2_src};
    const void* vs2[1] = {v2_src};
    void* kc2[1] = {k2_cache};
    void* vc2[1] = {v2_cache};
    CHECK(ric_schedule(b, R, c, q));
    ric_step s2;
    CHECK(ric_compile_and_cache(b, NPAD, ks2, vs2, kc2, vc2, 1, 0, ROW2, SLOTS, NULL, 0, &s2));
    uint8_t cache2_host[SLOTS * ROW2];
    CHECK(ric_read_device(cache2_host, v2_cache, sizeof cache2_host));

    printf("{\n\"num_reqs\": %d, \"num_actual_tokens\": %d, \"num_tokens_padded\": %d,\n", s.num_reqs,
           s.num_actual_tokens, s.num_tokens_padded);
    printf("\"max_query_len\": %d, \"max_seq_len\": %d, \"num_sampled\": %d,\n", s.max_query_len, s.max_seq_len,
           s.num_sampled);
    print_array("query_start_loc", s.query_start_loc, R + 1, 0);
    print_array("req_indices", s.req_indices, NPAD, 0);
    print_array("positions", s.positions, NPAD, 0);
    print_array("input_ids", s.input_ids, NPAD, 0);
    print_array("slot_mapping", s.slot_mapping, NPAD, 0);
    print_array("seq_lens", s.seq_lens, R, 0);
    print_array("cu_seqlens_k", s.cu_seqlens_k, R + 1, 0);
    print_array("logits_indices", s.logits_indices, R, 0);
    print_array("sample_indices", s.sample_indices, R, 0);
    printf("\"k_cache_first_byte\": [");
    for (int i = 0; i < SLOTS; ++i) printf("%s%d", i ? ", " : "", cache_host[i * ROW]);
    printf("],\n");
    print_array("fused_slot_mapping", s2.slot_mapping, NPAD, 0);
    printf("\"fused_v_cache_first_byte\": [");
    for (int i = 0; i < SLOTS; ++i) printf("%s%d", i ? ", " : "", cache2_host[i * ROW2]);
    printf("]\n}\n");

    hipFree(k_src);
    hipFree(v_src);
    hipFree(k_cache);
    hipFree(v_cache);
    hipFree(k2_src);
    hipFree(v2_src);
    hipFree(k2_cache);
    hipFree(v2_cache);
    CHECK(ric_destroy(b));
    return 0;
}
