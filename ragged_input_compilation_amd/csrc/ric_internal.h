// Internal declarations shared by the host control plane and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ric {

// Per-row scalar columns of the column store, in this order in one
// [kNumScalarCols][max_num_reqs] int32 region (float columns hold their bits).
enum ScalarCol : int {
    kNumTokens = 0,
    kNumPrompt = 1,
    kNumComputed = 2,
    kNumScheduled = 3,
    kNumBlocks = 4,
    kTopK = 5,
    kTemperature = 6,
    kTopP = 7,
    kRepPenalty = 8,
    kNumBlocksG1 = 9,             // block counts of KV-cache groups 1..3
    kNumBlocksG2 = 10,
    kNumBlocksG3 = 11,
    kNumScalarCols = 12
};

constexpr int kMaxGroups = 4;             // KV-cache groups per handle
__host__ __device__ inline int blocks_col(int g) { return g == 0 ? kNumBlocks : kNumBlocksG1 + g - 1; }

constexpr int kMaxReqsLimit = 8000;       // compile LDS: 2R + 21 int32 (+ up to 128 slots) < 64 KiB
constexpr int kMaxLayersPerLaunch = 32;   // K/V pointer sets passed by value
constexpr int kNumDevScalars = 8;

// One staged copy: n_words 32-bit words from the staging payload to dst.
struct DeltaOp {
    uint64_t dst;
    uint32_t src_word;
    uint32_t n_words;
};

struct CompileParams {
    const int32_t* scal;          // [kNumScalarCols][max_num_reqs]
    const int32_t* tokens;        // [max_num_reqs][tok_stride]
    const int32_t* blocks;        // [max_num_reqs][blk_stride]
    int64_t tok_stride;
    int64_t blk_stride;
    int32_t max_num_reqs;
    int32_t num_reqs;
    int32_t n_pad;
    int32_t block_size;
    int32_t block_shift;          // log2(block_size) when a power of two, else -1
    int32_t null_slot;            // null_block * block_size
    int32_t num_token_tiles;
    int32_t* input_ids;
    int32_t* positions;
    int32_t* req_indices;
    int32_t* slot_mapping;
    int32_t* query_start_loc;
    int32_t* seq_lens;
    int32_t* logits_indices;
    uint8_t* discard;
    int32_t* sample_indices;
    int32_t* dev_scalars;
    int32_t* cu_seqlens_k;
    // further KV-cache groups that get per-token slots (group 0 is the one above)
    int32_t num_extra_groups;
    const int32_t* xblocks[kMaxGroups - 1];
    int64_t xblk_stride[kMaxGroups - 1];
    int32_t xblock_size[kMaxGroups - 1];
    int32_t xblock_shift[kMaxGroups - 1];
    int32_t xnull_slot[kMaxGroups - 1];
    int32_t* xslot_mapping[kMaxGroups - 1];
};

struct SpecParams {
    const int32_t* qsl;           // compile output [R + 1]
    const int32_t* input_ids;     // compile output
    const int32_t* num_draft;     // [R] uploaded draft counts
    int32_t num_reqs;
    int32_t num_logits;           // sum of (d + 1)
    int32_t num_tiles;
    int32_t* logits_indices;      // [num_logits]
    int32_t* cu_num_logits;       // [R + 1]
    int32_t* target;              // [sum d]
    int32_t* bonus;               // [R]
    int32_t* draft_ids;           // [sum d]
};

struct PaddedTableParams {
    const int32_t* blocks;        // [max_num_reqs][blk_stride]
    const int32_t* num_blocks;    // device column
    int32_t* dst;                 // [rows][width]
    int64_t blk_stride;
    int32_t rows;
    int32_t width;
    int32_t fill;
    int32_t ratio;                // kernel blocks per table block (1: ids as stored)
};

struct KVParams {
    const uint8_t* k[kMaxLayersPerLaunch];
    const uint8_t* v[kMaxLayersPerLaunch];
    uint8_t* kc[kMaxLayersPerLaunch];
    uint8_t* vc[kMaxLayersPerLaunch];
    const int32_t* slot;
    int64_t src_stride;
    int64_t num_slots;
    int32_t* status;
    int32_t num_tokens;
    int32_t row_bytes;
    int32_t chunk_shift;          // log2(row_bytes / 16) when a power of two, else -1
    int32_t rows_per_wg;
};

struct GatherParams {
    const uint8_t* src;
    int64_t src_stride;
    int64_t src_rows;
    const int32_t* idx;
    const int32_t* dev_count;
    uint8_t* dst;
    int64_t dst_stride;
    int32_t* status;
    int32_t max_rows;
    int32_t row_bytes;
};

struct MoveParams {
    const int32_t* pairs;         // [num_pairs][2] = (destination hole, source row)
    int32_t* tokens;
    int32_t* blocks[kMaxGroups];  // per group [max_num_reqs][blk_stride[g]]
    int64_t blk_stride[kMaxGroups];
    int32_t* scal;
    int64_t tok_stride;
    int32_t num_groups;
    int32_t max_num_reqs;
    int32_t num_pairs;
    int32_t chunk_vec4;           // 16-byte units of token history per workgroup
};

struct CorrectParams {
    int32_t* computed;            // device num_computed column
    int32_t* tokens;              // [max_num_reqs][tok_stride]
    int64_t tok_stride;
    const int32_t* rows;          // [n] uploaded: corrected rows
    const int32_t* prev;          // [n] uploaded: sampler position of each
    const int32_t* draft;         // [n] uploaded: drafts each verified
    const int32_t* accepted;      // caller's device array [prev_len]
    const int32_t* sampled;       // caller's device array [prev_len][sampled_stride], or null
    int64_t sampled_stride;
    int32_t* status;              // caller's device counter of out-of-range counts, or null
    int32_t n;
};

// Launchers (enqueue only; return the launch status).
hipError_t launch_compile(const CompileParams& p, hipStream_t s);
hipError_t launch_kv_scatter(const KVParams& p, int num_layers, hipStream_t s);
hipError_t launch_gather(const GatherParams& p, hipStream_t s);
hipError_t launch_move_rows(const MoveParams& p, int max_token_chunks, hipStream_t s);
hipError_t launch_apply_deltas(const uint32_t* payload, const DeltaOp* ops, int n_ops, hipStream_t s);
hipError_t launch_padded_table(const PaddedTableParams& p, hipStream_t s);
hipError_t launch_spec_decode(const SpecParams& p, hipStream_t s);
hipError_t launch_correct_computed(const CorrectParams& p, hipStream_t s);
// dst_off[k] (int64, in int32 elements of the token table) <- src[src_idx[k]]
hipError_t launch_append_sampled(int32_t* tokens, const int64_t* dst_off, const int32_t* src_idx,
                                 const int32_t* src, int32_t src_len, int32_t n, int32_t* err, hipStream_t s);

// Compile plus the K/V write of `num_layers` (<= kMaxLayersPerLaunch) layers
// through the group-0 slots in one launch; only for rows the fused kernel
// handles (fused_kv_supported).  `long_runs`: the step is mostly long
// per-request runs (picks the tile shape).  p.num_token_tiles is set by the
// launcher.
bool fused_kv_supported(int row_bytes);
hipError_t launch_compile_kv(const CompileParams& p, const KVParams& kv, int num_layers, bool long_runs,
                             hipStream_t s);

// Clears ceil(num_slots / 32) bitmap words, then counts, for the first
// min(n, *dev_n) slots (n when dev_n is null), collisions in result[0] and
// slots outside [0, num_slots) in result[1].
hipError_t launch_check_slots(const int32_t* slot, int32_t n, const int32_t* dev_n, int64_t num_slots,
                              uint32_t* bits, int32_t* result, hipStream_t s);

// The allocation-free check keeps its bitmap in a static device array of
// kCheckScratchWords words (4 MiB: up to 2^25 slots) on each GPU.
constexpr int64_t kCheckScratchWords = int64_t(1) << 20;
constexpr int kMaxScratchDevices = 64;
// Device address of that array on the current device (looked up once per
// device, then cached).
hipError_t check_scratch_for_current_device(uint32_t** out);

// Token tile of one compile workgroup.
constexpr int kCompileThreads = 256;
constexpr int kCompileTokensPerThread = 1;
constexpr int kCompileTile = kCompileThreads * kCompileTokensPerThread;

}  // namespace ric
