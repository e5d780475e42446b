// Host control plane and C ABI of libric: the persistent batch's row maps and
// counters (host mirror), validation, delta staging, and the launches.
//
// Sources (page title, section):
//   [P1] "vLLM 源码完全拆解（五）：GPUModelRunner 如何把动态请求拼成一次 GPU 前向"
//   [P2] "第8章 ModelRunner：从 SchedulerOutput 到 GPU Kernel"
//   [P4] "04 · 模型执行与 CUDA Graph"
//
// The device holds the column store; the host keeps only what validation and
// row bookkeeping need (row <-> request maps and the per-row scalar columns).
// Token and block payloads never live on the host beyond the pinned staging:
// each mutation appends its payload to a pinned log, and a flush scatters the
// whole log with one kernel (which reads a small log in place from the pinned
// memory and a large one after one copy into device staging), instead of one
// small copy per request.  Two pinned logs alternate, each guarded by an event
// so the host never overwrites a log that the device may still be reading
// ([P1 §为什么 CPU 侧同时要 tensor 和 NumPy view]: producer/consumer ordering
// of pinned buffers).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/ric.h"
#include "ric_internal.h"

using namespace ric;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

#define HIP_TRY(expr)                                                                   \
    do {                                                                                \
        hipError_t e_ = (expr);                                                         \
        if (e_ != hipSuccess) return fail(RIC_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

constexpr size_t kAlign = 256;
constexpr int32_t kMaxRowsPerLaunch = 1 << 24;   // rows * 256 lanes must fit a 32-bit work-item count
constexpr uint32_t kMaxWordsPerOp = 8192;   // split big payloads so ops spread over workgroups
// A flush whose log (payload + ops) fits in kDirectLogBytes and whose ops are
// at most kDirectMaxOpWords long is applied by the scatter kernel reading the
// pinned log in place; larger ones are first copied into device staging.
constexpr size_t kDirectLogBytes = 65536;
constexpr uint32_t kDirectMaxOpWords = 2048;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round4(int64_t x) { return (x + 3) / 4 * 4; }

int ilog2_exact(int64_t x) {
    if (x <= 0 || (x & (x - 1)) != 0) return -1;
    int s = 0;
    while ((int64_t(1) << s) < x) ++s;
    return s;
}

struct Layout {
    int64_t tok_stride, blk_stride;
    size_t off_tok, off_blk, off_scal, off_ids, off_pos, off_req, off_slot, off_qsl, off_seq,
        off_logits, off_sample, off_discard, off_dscal, off_pairs, off_cuk, off_samp_off, off_samp_idx,
        off_spec_logits, off_spec_target, off_spec_draft, off_spec_cu, off_spec_bonus, off_spec_d,
        off_corr, off_staging, total;
    size_t staging_bytes;
    // KV-cache groups 1..groups-1 (index g): block tables and slot outputs
    int groups;
    int64_t xblk_stride[kMaxGroups];
    size_t off_xblk[kMaxGroups], off_xslot[kMaxGroups];
};

int num_groups_of(const ric_config& c) { return c.num_kv_groups <= 0 ? 1 : c.num_kv_groups; }
int32_t group_B(const ric_config& c, int g) { return g == 0 ? c.block_size : c.group_block_size[g]; }
int32_t group_pool(const ric_config& c, int g) {
    return (g == 0 || c.group_num_kv_blocks[g] <= 0) ? c.num_kv_blocks : c.group_num_kv_blocks[g];
}
int32_t group_cap(const ric_config& c, int g) {
    return g == 0 ? c.max_blocks_per_req : (c.max_model_len + c.group_block_size[g] - 1) / c.group_block_size[g];
}
bool group_slots(const ric_config& c, int g) { return g == 0 || c.group_slot_mode[g] == RIC_SLOTS_PER_TOKEN; }

size_t default_staging(const ric_config& c) {
    const size_t scal_reserve = (size_t)kNumScalarCols * (size_t)c.max_num_reqs * 4 + 64 * 16;
    return std::max<size_t>(4u << 20, 4 * scal_reserve);
}

// Smallest staging that always makes progress: room for a full scalar-column
// refresh (reserved by every flush) plus 64 KiB of payload and ops.
size_t min_staging(const ric_config& c) {
    return 2 * (size_t)kNumScalarCols * (size_t)c.max_num_reqs * 4 + (64u << 10);
}

Layout layout_of(const ric_config& c) {
    Layout L{};
    L.tok_stride = round4(c.max_model_len);
    L.blk_stride = round4(c.max_blocks_per_req);
    L.staging_bytes = c.staging_bytes > 0 ? (size_t)c.staging_bytes : default_staging(c);
    const size_t R = (size_t)c.max_num_reqs, NT = (size_t)c.max_num_batched_tokens;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes, kAlign);
        return at;
    };
    L.off_tok = take(R * (size_t)L.tok_stride * 4);
    L.off_blk = take(R * (size_t)L.blk_stride * 4);
    L.off_scal = take((size_t)kNumScalarCols * R * 4);
    L.off_ids = take(NT * 4);
    L.off_pos = take(NT * 4);
    L.off_req = take(NT * 4);
    L.off_slot = take(NT * 4);
    L.off_qsl = take((R + 1) * 4);
    L.off_seq = take(R * 4);
    L.off_logits = take(R * 4);
    L.off_sample = take(R * 4);
    L.off_discard = take(R);
    L.off_dscal = take(kNumDevScalars * 4);
    L.off_pairs = take(R * 2 * 4);
    L.off_cuk = take((R + 1) * 4);
    L.off_samp_off = take(R * 8);
    L.off_samp_idx = take(R * 4);
    L.off_spec_logits = take(NT * 4);
    L.off_spec_target = take(NT * 4);
    L.off_spec_draft = take(NT * 4);
    L.off_spec_cu = take((R + 1) * 4);
    L.off_spec_bonus = take(R * 4);
    L.off_spec_d = take(R * 4);
    L.off_corr = take(R * 3 * 4);
    L.groups = num_groups_of(c);
    for (int g = 1; g < L.groups; ++g) {
        L.xblk_stride[g] = round4(group_cap(c, g));
        L.off_xblk[g] = take(R * (size_t)L.xblk_stride[g] * 4);
        L.off_xslot[g] = group_slots(c, g) ? take(NT * 4) : 0;
    }
    L.off_staging = take(L.staging_bytes);
    L.total = o;
    return L;
}

int check_config(const ric_config* c) {
    if (!c) return fail(RIC_EINVAL, "config is NULL");
    if (c->max_num_reqs < 1 || c->max_num_reqs > kMaxReqsLimit)
        return fail(RIC_EINVAL, "max_num_reqs must be in [1, %d]", kMaxReqsLimit);
    if (c->max_model_len < 1 || c->block_size < 1 || c->max_blocks_per_req < 1 ||
        c->max_num_batched_tokens < 1 || c->num_kv_blocks < 1)
        return fail(RIC_EINVAL, "capacities must be positive");
    if (c->null_block < 0 || c->null_block >= c->num_kv_blocks)
        return fail(RIC_EINVAL, "null_block outside [0, num_kv_blocks)");
    if ((int64_t)c->num_kv_blocks * c->block_size >= (int64_t(1) << 31))
        return fail(RIC_EINVAL, "num_kv_blocks * block_size must stay below 2^31 (int32 slots)");
    if (c->num_kv_groups < 0 || c->num_kv_groups > kMaxGroups)
        return fail(RIC_EINVAL, "num_kv_groups %d outside [0, %d]", c->num_kv_groups, kMaxGroups);
    for (int g = 1; g < num_groups_of(*c); ++g) {
        if (c->group_block_size[g] < 1) return fail(RIC_EINVAL, "group %d: block size must be positive", g);
        if (c->group_num_kv_blocks[g] < 0) return fail(RIC_EINVAL, "group %d: negative pool size", g);
        if (c->group_slot_mode[g] != RIC_SLOTS_PER_TOKEN && c->group_slot_mode[g] != RIC_SLOTS_NONE)
            return fail(RIC_EINVAL, "group %d: unknown slot mode %d", g, c->group_slot_mode[g]);
        if (c->null_block >= group_pool(*c, g)) return fail(RIC_EINVAL, "group %d: null_block outside its pool", g);
        if ((int64_t)group_pool(*c, g) * c->group_block_size[g] >= (int64_t(1) << 31))
            return fail(RIC_EINVAL, "group %d: pool * block size must stay below 2^31", g);
    }
    if (c->staging_bytes < 0) return fail(RIC_EINVAL, "staging_bytes negative");
    if (c->staging_bytes > 0 && (size_t)c->staging_bytes < min_staging(*c))
        return fail(RIC_EINVAL, "staging_bytes %d below the minimum %zu (twice the scalar columns + 64 KiB)",
                    c->staging_bytes, min_staging(*c));
    return RIC_OK;
}

}  // namespace

struct ric_batch {
    ric_config cfg{};
    Layout L{};
    hipStream_t stream = nullptr;
    int device = 0;
    bool own_ws = false;
    uint8_t* ws = nullptr;

    // device regions
    int32_t *d_tok = nullptr, *d_blk = nullptr, *d_scal = nullptr;
    int32_t* d_xblk[kMaxGroups] = {nullptr, nullptr, nullptr, nullptr};    // groups 1..
    int32_t* d_xslot[kMaxGroups] = {nullptr, nullptr, nullptr, nullptr};
    int32_t *d_ids = nullptr, *d_pos = nullptr, *d_req = nullptr, *d_slot = nullptr;
    int32_t *d_qsl = nullptr, *d_seq = nullptr, *d_logits = nullptr, *d_sample = nullptr;
    uint8_t* d_discard = nullptr;
    int32_t *d_dscal = nullptr, *d_pairs = nullptr, *d_cuk = nullptr, *d_samp_idx = nullptr;
    int64_t* d_samp_off = nullptr;
    int32_t *d_spec_logits = nullptr, *d_spec_target = nullptr, *d_spec_draft = nullptr,
            *d_spec_cu = nullptr, *d_spec_bonus = nullptr, *d_spec_d = nullptr;
    int32_t* d_corr = nullptr;       // [3][max_num_reqs]: rows, sampler positions, draft counts
    uint8_t* d_staging = nullptr;

    // pinned delta logs
    uint8_t* h_log[2] = {nullptr, nullptr};
    uint8_t* d_log[2] = {nullptr, nullptr};  // device addresses of the same pinned logs
    hipEvent_t ev[2] = {nullptr, nullptr};
    bool ev_pending[2] = {false, false};
    int cur = 0;
    bool cur_ready = false;          // h_log[cur] is known free to write
    uint32_t payload_words = 0;
    std::vector<DeltaOp> ops;
    uint32_t epoch = 1;

    // host mirror
    std::vector<int32_t> scal;       // [kNumScalarCols][max_num_reqs]
    int32_t dirty_lo[kNumScalarCols], dirty_hi[kNumScalarCols];
    std::vector<uint64_t> req_at;
    std::vector<uint8_t> live;
    std::vector<uint32_t> pending_epoch;
    std::unordered_map<uint64_t, int32_t> row_of;
    int32_t num_live = 0;

    // schedule state
    bool scheduled = false;
    bool compiled = false;           // a compile ran since the last schedule
    bool corrected = false;          // ric_correct_computed ran since the last schedule
    int32_t sched_R = 0, sched_N = 0, sched_max_q = 0, sched_max_seq = 0, sched_sampled = 0;

    int32_t& S(int col, int row) { return scal[(size_t)col * cfg.max_num_reqs + row]; }
    int32_t* dcol(int col) { return d_scal + (size_t)col * cfg.max_num_reqs; }

    void mark(int col, int row) {
        dirty_lo[col] = std::min(dirty_lo[col], row);
        dirty_hi[col] = std::max(dirty_hi[col], row + 1);
    }
    void clear_dirty() {
        for (int c = 0; c < kNumScalarCols; ++c) {
            dirty_lo[c] = cfg.max_num_reqs;
            dirty_hi[c] = 0;
        }
    }
    int32_t used_rows() const {
        for (int32_t r = cfg.max_num_reqs - 1; r >= 0; --r)
            if (live[r]) return r + 1;
        return 0;
    }
    // block table of KV-cache group g
    int32_t* blk(int g) const { return g == 0 ? d_blk : d_xblk[g]; }
    int64_t bstride(int g) const { return g == 0 ? L.blk_stride : L.xblk_stride[g]; }
};

namespace {

// Makes the handle's device current for one call (and restores the caller's),
// so a process that drives handles on several GPUs needs no device switching
// of its own around library calls.
struct DeviceScope {
    int prev = -1;
    explicit DeviceScope(const ric_batch* b) {
        int cur = -1;
        if (hipGetDevice(&cur) == hipSuccess && cur != b->device && hipSetDevice(b->device) == hipSuccess) prev = cur;
    }
    ~DeviceScope() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
    DeviceScope(const DeviceScope&) = delete;
    DeviceScope& operator=(const DeviceScope&) = delete;
};

// Bytes the log needs for everything staged so far plus `extra_words` more
// payload in one more op, plus the scalar columns a flush appends.
size_t log_need(const ric_batch* b, size_t extra_words, size_t extra_ops) {
    const size_t scal_words = (size_t)kNumScalarCols * b->cfg.max_num_reqs;
    return align_up(((size_t)b->payload_words + extra_words + scal_words) * 4, 16) +
           (b->ops.size() + extra_ops + kNumScalarCols) * sizeof(DeltaOp);
}

int ensure_log_writable(ric_batch* b) {
    if (b->cur_ready) return RIC_OK;
    if (b->ev_pending[b->cur]) {
        HIP_TRY(hipEventSynchronize(b->ev[b->cur]));
        b->ev_pending[b->cur] = false;
    }
    b->cur_ready = true;
    return RIC_OK;
}

uint32_t* log_payload(ric_batch* b) { return reinterpret_cast<uint32_t*>(b->h_log[b->cur]); }

int flush(ric_batch* b);

// Stage `n` words for device address `dst`, splitting across ops and flushes.
int stage(ric_batch* b, void* dst, const void* src, size_t n) {
    const uint8_t* s = static_cast<const uint8_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    while (n > 0) {
        size_t take = std::min<size_t>(n, kMaxWordsPerOp);
        if (log_need(b, take, 1) > b->L.staging_bytes) {
            // shrink to what fits, or flush if nothing does
            size_t lo = 0, hi = take;
            while (lo < hi) {
                const size_t mid = (lo + hi + 1) / 2;
                if (log_need(b, mid, 1) <= b->L.staging_bytes) lo = mid; else hi = mid - 1;
            }
            take = lo;
            if (take == 0) {
                int rc = flush(b);
                if (rc) return rc;
                continue;
            }
        }
        int rc = ensure_log_writable(b);
        if (rc) return rc;
        memcpy(log_payload(b) + b->payload_words, s, take * 4);
        b->ops.push_back(DeltaOp{reinterpret_cast<uint64_t>(d), b->payload_words, (uint32_t)take});
        b->payload_words += (uint32_t)take;
        s += take * 4;
        d += take * 4;
        n -= take;
    }
    return RIC_OK;
}

// A graph captured during an upload would record a read of a pinned log that
// later flushes rewrite (in place, or through a copy), and an apply kernel
// whose op count and offsets belong to that one flush: a replay would scatter
// whatever the log then holds.  Uploads therefore happen outside capture only; calls that stage and
// upload in one go check this before they stage anything.
int refuse_if_capturing(ric_batch* b) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(b->stream, &cap));
    if (cap != hipStreamCaptureStatusNone)
        return fail(RIC_ESTATE, "staged deltas cannot be uploaded while the handle's stream is being captured: "
                                "flush (ric_flush, or an eager step) before the capture begins");
    return RIC_OK;
}

int flush(ric_batch* b) {
    bool any_dirty = false;
    for (int c = 0; c < kNumScalarCols; ++c) any_dirty |= b->dirty_lo[c] < b->dirty_hi[c];
    if (b->ops.empty() && !any_dirty) return RIC_OK;
    int rc = refuse_if_capturing(b);
    if (rc) return rc;
    rc = ensure_log_writable(b);
    if (rc) return rc;
    // Scalar columns: copy the dirty row range of each column from the mirror.
    // (Room for them is always reserved by log_need.)
    for (int c = 0; c < kNumScalarCols; ++c) {
        if (b->dirty_lo[c] >= b->dirty_hi[c]) continue;
        const int32_t lo = b->dirty_lo[c], n = b->dirty_hi[c] - lo;
        memcpy(log_payload(b) + b->payload_words, &b->S(c, lo), (size_t)n * 4);
        b->ops.push_back(DeltaOp{reinterpret_cast<uint64_t>(b->dcol(c) + lo), b->payload_words, (uint32_t)n});
        b->payload_words += (uint32_t)n;
    }
    const size_t ops_off = align_up((size_t)b->payload_words * 4, 16);
    const size_t ops_bytes = b->ops.size() * sizeof(DeltaOp);
    if (ops_off + ops_bytes > b->L.staging_bytes) return fail(RIC_EHIP, "internal: delta log overflow");
    memcpy(b->h_log[b->cur] + ops_off, b->ops.data(), ops_bytes);
    // A step's usual log (counts, appended tokens, new block ids: a few KB)
    // is read by the scatter kernel straight from the pinned log, which saves
    // the copy's own launch: about 2 us of device time and 2.5 us of host
    // time per flush on MI355X.  Reading across the host link takes one
    // round trip per pass, so large logs (whole prompts at admission) are
    // copied into device staging first.
    uint32_t max_words = 0;
    for (const DeltaOp& op : b->ops) max_words = std::max(max_words, op.n_words);
    const uint8_t* src = b->d_staging;
    if (ops_off + ops_bytes <= kDirectLogBytes && max_words <= kDirectMaxOpWords) {
        src = b->d_log[b->cur];
    } else {
        HIP_TRY(hipMemcpyAsync(b->d_staging, b->h_log[b->cur], ops_off + ops_bytes, hipMemcpyHostToDevice,
                               b->stream));
    }
    HIP_TRY(launch_apply_deltas(reinterpret_cast<const uint32_t*>(src),
                                reinterpret_cast<const DeltaOp*>(src + ops_off), (int)b->ops.size(), b->stream));
    HIP_TRY(hipEventRecord(b->ev[b->cur], b->stream));
    b->ev_pending[b->cur] = true;
    b->cur ^= 1;
    b->cur_ready = false;
    b->payload_words = 0;
    b->ops.clear();
    b->clear_dirty();
    ++b->epoch;
    return RIC_OK;
}

// Flush first when a new whole-row write could overlap a staged write to the
// same row (ops of one flush are applied in parallel).
int before_row_overwrite(ric_batch* b, int32_t row) {
    if (b->pending_epoch[row] == b->epoch) return flush(b);
    return RIC_OK;
}

int check_blocks(const ric_batch* b, int g, const int32_t* ids, int32_t n) {
    const int32_t pool = group_pool(b->cfg, g);
    for (int32_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= pool || ids[i] == b->cfg.null_block)
            return fail(RIC_ERANGE, "group %d: block id %d at index %d is not a usable block", g, ids[i], i);
    return RIC_OK;
}

int find(const ric_batch* b, uint64_t req_id, int32_t* row) {
    auto it = b->row_of.find(req_id);
    if (it == b->row_of.end()) return fail(RIC_ENOENT, "unknown request id %llu", (unsigned long long)req_id);
    *row = it->second;
    return RIC_OK;
}

int32_t as_bits(float f) {
    int32_t i;
    memcpy(&i, &f, 4);
    return i;
}

// Validation shared by ric_schedule and ric_check_step.
int check_step_rows(const ric_config& cfg, int32_t R, const int32_t* c, const int32_t* q,
                    const int32_t* P, const int32_t* T, const int32_t* nb, int32_t* N_out,
                    int32_t* maxq_out, int32_t* maxseq_out, int32_t* sampled_out) {
    if (R < 0 || R > cfg.max_num_reqs) return fail(RIC_EINVAL, "num_reqs %d outside [0, max_num_reqs]", R);
    if (R > 0 && (!c || !q)) return fail(RIC_EINVAL, "count arrays are NULL");
    int64_t N = 0;
    int32_t maxq = 0, maxseq = 0, sampled = 0;
    for (int32_t i = 0; i < R; ++i) {
        if (q[i] < 1) return fail(RIC_EINVAL, "row %d: num_scheduled %d < 1", i, q[i]);
        if (c[i] < 0) return fail(RIC_EINVAL, "row %d: num_computed %d < 0", i, c[i]);
        const int64_t end = (int64_t)c[i] + q[i];
        if (end > T[i]) return fail(RIC_EINVAL, "row %d: c+q = %lld exceeds the %d-token history", i, (long long)end, T[i]);
        if ((end + cfg.block_size - 1) / cfg.block_size > nb[i])
            return fail(RIC_EINVAL, "row %d: %d blocks cannot hold position %lld", i, nb[i], (long long)(end - 1));
        N += q[i];
        maxq = std::max(maxq, q[i]);
        maxseq = std::max<int32_t>(maxseq, (int32_t)end);
        sampled += (end >= P[i]) ? 1 : 0;
    }
    if (N > cfg.max_num_batched_tokens)
        return fail(RIC_EINVAL, "%lld scheduled tokens exceed max_num_batched_tokens %d", (long long)N, cfg.max_num_batched_tokens);
    *N_out = (int32_t)N;
    *maxq_out = maxq;
    *maxseq_out = maxseq;
    *sampled_out = sampled;
    return RIC_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

const char* ric_last_error(void) { return g_err.c_str(); }

size_t ric_workspace_bytes(const ric_config* cfg) {
    if (check_config(cfg)) return 0;
    return layout_of(*cfg).total;
}

int ric_create(const ric_config* cfg, void* stream, void* workspace, size_t workspace_bytes, ric_batch** out) {
    if (!out) return fail(RIC_EINVAL, "out is NULL");
    int rc = check_config(cfg);
    if (rc) return rc;
    ric_batch* b = new (std::nothrow) ric_batch();
    if (!b) return fail(RIC_ENOMEM, "host allocation failed");
    b->cfg = *cfg;
    b->L = layout_of(*cfg);
    b->stream = static_cast<hipStream_t>(stream);
    auto bail = [&](int code) {
        ric_destroy(b);
        return code;
    };
    if (hipGetDevice(&b->device) != hipSuccess) return bail(fail(RIC_EHIP, "no HIP device"));
    if (workspace) {
        if (workspace_bytes < b->L.total)
            return bail(fail(RIC_EINVAL, "workspace of %zu bytes, %zu needed", workspace_bytes, b->L.total));
        if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
            return bail(fail(RIC_EINVAL, "workspace must be %zu-byte aligned", kAlign));
        b->ws = static_cast<uint8_t*>(workspace);
    } else {
        if (hipMalloc(&b->ws, b->L.total) != hipSuccess) {
            b->ws = nullptr;
            return bail(fail(RIC_ENOMEM, "hipMalloc of %zu bytes failed", b->L.total));
        }
        b->own_ws = true;
    }
    const Layout& L = b->L;
    b->d_tok = reinterpret_cast<int32_t*>(b->ws + L.off_tok);
    b->d_blk = reinterpret_cast<int32_t*>(b->ws + L.off_blk);
    for (int g = 1; g < L.groups; ++g) {
        b->d_xblk[g] = reinterpret_cast<int32_t*>(b->ws + L.off_xblk[g]);
        if (group_slots(*cfg, g)) b->d_xslot[g] = reinterpret_cast<int32_t*>(b->ws + L.off_xslot[g]);
    }
    b->d_scal = reinterpret_cast<int32_t*>(b->ws + L.off_scal);
    b->d_ids = reinterpret_cast<int32_t*>(b->ws + L.off_ids);
    b->d_pos = reinterpret_cast<int32_t*>(b->ws + L.off_pos);
    b->d_req = reinterpret_cast<int32_t*>(b->ws + L.off_req);
    b->d_slot = reinterpret_cast<int32_t*>(b->ws + L.off_slot);
    b->d_qsl = reinterpret_cast<int32_t*>(b->ws + L.off_qsl);
    b->d_seq = reinterpret_cast<int32_t*>(b->ws + L.off_seq);
    b->d_logits = reinterpret_cast<int32_t*>(b->ws + L.off_logits);
    b->d_sample = reinterpret_cast<int32_t*>(b->ws + L.off_sample);
    b->d_discard = b->ws + L.off_discard;
    b->d_dscal = reinterpret_cast<int32_t*>(b->ws + L.off_dscal);
    b->d_pairs = reinterpret_cast<int32_t*>(b->ws + L.off_pairs);
    b->d_cuk = reinterpret_cast<int32_t*>(b->ws + L.off_cuk);
    b->d_samp_off = reinterpret_cast<int64_t*>(b->ws + L.off_samp_off);
    b->d_samp_idx = reinterpret_cast<int32_t*>(b->ws + L.off_samp_idx);
    b->d_spec_logits = reinterpret_cast<int32_t*>(b->ws + L.off_spec_logits);
    b->d_spec_target = reinterpret_cast<int32_t*>(b->ws + L.off_spec_target);
    b->d_spec_draft = reinterpret_cast<int32_t*>(b->ws + L.off_spec_draft);
    b->d_spec_cu = reinterpret_cast<int32_t*>(b->ws + L.off_spec_cu);
    b->d_spec_bonus = reinterpret_cast<int32_t*>(b->ws + L.off_spec_bonus);
    b->d_spec_d = reinterpret_cast<int32_t*>(b->ws + L.off_spec_d);
    b->d_corr = reinterpret_cast<int32_t*>(b->ws + L.off_corr);
    b->d_staging = b->ws + L.off_staging;
    for (int i = 0; i < 2; ++i) {
        void* p = nullptr;
        // Coherent: the scatter kernel may read the log in place, and must see
        // what the host wrote before the launch, not a cached older copy.
        if (hipHostMalloc(&p, L.staging_bytes, hipHostMallocCoherent) != hipSuccess)
            return bail(fail(RIC_ENOMEM, "pinned staging allocation failed"));
        b->h_log[i] = static_cast<uint8_t*>(p);
        void* dp = nullptr;
        if (hipHostGetDevicePointer(&dp, p, 0) != hipSuccess)
            return bail(fail(RIC_EHIP, "pinned staging has no device address"));
        b->d_log[i] = static_cast<uint8_t*>(dp);
        // These events only tell the host when the device has finished
        // reading a log; no device write needs to become visible to the host, so
        // they skip the system-scope fence (an L2 write-back and invalidate
        // on every flush otherwise).
        if (hipEventCreateWithFlags(&b->ev[i], hipEventDisableTiming | hipEventDisableSystemFence) != hipSuccess)
            return bail(fail(RIC_EHIP, "event creation failed"));
    }
    const int MR = cfg->max_num_reqs;
    b->scal.assign((size_t)kNumScalarCols * MR, 0);
    b->req_at.assign(MR, 0);
    b->live.assign(MR, 0);
    b->pending_epoch.assign(MR, 0);
    b->clear_dirty();
    // Scalar columns start at zero on the device too (the whole region).
    for (int c = 0; c < kNumScalarCols; ++c) {
        b->dirty_lo[c] = 0;
        b->dirty_hi[c] = MR;
    }
    // Device scalars: [6] counts tokens whose row data was out of range (sticky).
    const int32_t zeros[kNumDevScalars] = {0, 0, 0, 0, 0, 0, 0, 0};
    rc = stage(b, b->d_dscal, zeros, kNumDevScalars);
    if (rc) return bail(rc);
    rc = flush(b);
    if (rc) return bail(rc);
    *out = b;
    return RIC_OK;
}

int ric_destroy(ric_batch* b) {
    if (!b) return RIC_OK;
    DeviceScope ds(b);
    if (b->ws) (void)hipStreamSynchronize(b->stream);
    for (int i = 0; i < 2; ++i) {
        if (b->ev[i]) (void)hipEventDestroy(b->ev[i]);
        if (b->h_log[i]) (void)hipHostFree(b->h_log[i]);
    }
    if (b->own_ws && b->ws) (void)hipFree(b->ws);
    delete b;
    return RIC_OK;
}

int ric_set_stream(ric_batch* b, void* stream) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    HIP_TRY(hipStreamSynchronize(b->stream));
    b->stream = static_cast<hipStream_t>(stream);
    return RIC_OK;
}

int ric_add_request(ric_batch* b, uint64_t req_id, const int32_t* tokens, int32_t num_tokens,
                    int32_t num_prompt, int32_t num_computed, const int32_t* blocks, int32_t num_blocks,
                    const ric_sampling* sampling, int32_t* out_row) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    if (b->row_of.count(req_id)) return fail(RIC_EEXIST, "request id %llu is live", (unsigned long long)req_id);
    if (num_tokens < 0 || num_tokens > b->cfg.max_model_len)
        return fail(RIC_ERANGE, "num_tokens %d outside [0, max_model_len %d]", num_tokens, b->cfg.max_model_len);
    if (num_blocks < 0 || num_blocks > b->cfg.max_blocks_per_req)
        return fail(RIC_ERANGE, "num_blocks %d outside [0, max_blocks_per_req %d]", num_blocks, b->cfg.max_blocks_per_req);
    if (num_prompt < 0 || num_prompt > num_tokens || num_computed < 0 || num_computed > num_tokens)
        return fail(RIC_ERANGE, "num_prompt %d / num_computed %d outside [0, %d]", num_prompt, num_computed, num_tokens);
    if ((num_tokens > 0 && !tokens) || (num_blocks > 0 && !blocks)) return fail(RIC_EINVAL, "payload is NULL");
    int rc = check_blocks(b, 0, blocks, num_blocks);
    if (rc) return rc;
    int32_t row = -1;
    for (int32_t r = 0; r < b->cfg.max_num_reqs; ++r)
        if (!b->live[r]) {
            row = r;
            break;
        }
    if (row < 0) return fail(RIC_EFULL, "no free row (max_num_reqs %d)", b->cfg.max_num_reqs);
    rc = before_row_overwrite(b, row);
    if (rc) return rc;
    rc = stage(b, b->d_tok + (int64_t)row * b->L.tok_stride, tokens, (size_t)num_tokens);
    if (rc) return rc;
    rc = stage(b, b->d_blk + (int64_t)row * b->L.blk_stride, blocks, (size_t)num_blocks);
    if (rc) return rc;
    const ric_sampling sp = sampling ? *sampling : ric_sampling{1.f, 1.f, 1.f, 0};
    // the remaining columns (block counts of groups 1..) start at zero
    const int32_t vals[kNumScalarCols] = {num_tokens, num_prompt, num_computed, 0, num_blocks, sp.top_k,
                                          as_bits(sp.temperature), as_bits(sp.top_p),
                                          as_bits(sp.repetition_penalty)};
    for (int c = 0; c < kNumScalarCols; ++c) {
        b->S(c, row) = vals[c];
        b->mark(c, row);
    }
    b->live[row] = 1;
    b->req_at[row] = req_id;
    b->row_of[req_id] = row;
    b->pending_epoch[row] = b->epoch;
    ++b->num_live;
    b->scheduled = false;
    if (out_row) *out_row = row;
    return RIC_OK;
}

int ric_remove_request(ric_batch* b, uint64_t req_id, int32_t* out_row) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    int32_t row;
    int rc = find(b, req_id, &row);
    if (rc) return rc;
    b->row_of.erase(req_id);
    b->live[row] = 0;
    --b->num_live;
    b->scheduled = false;
    if (out_row) *out_row = row;
    return RIC_OK;
}

int ric_append_tokens(ric_batch* b, uint64_t req_id, const int32_t* ids, int32_t n) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    int32_t row;
    int rc = find(b, req_id, &row);
    if (rc) return rc;
    const int32_t T = b->S(kNumTokens, row);
    if (n < 0 || (int64_t)T + n > b->cfg.max_model_len)
        return fail(RIC_EFULL, "row %d: %d + %d tokens exceed max_model_len %d", row, T, n, b->cfg.max_model_len);
    if (n > 0 && !ids) return fail(RIC_EINVAL, "ids is NULL");
    rc = stage(b, b->d_tok + (int64_t)row * b->L.tok_stride + T, ids, (size_t)n);
    if (rc) return rc;
    b->S(kNumTokens, row) = T + n;
    b->mark(kNumTokens, row);
    b->pending_epoch[row] = b->epoch;
    b->scheduled = false;
    return RIC_OK;
}

int ric_truncate_tokens(ric_batch* b, uint64_t req_id, int32_t num_tokens) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    int32_t row;
    int rc = find(b, req_id, &row);
    if (rc) return rc;
    const int32_t T = b->S(kNumTokens, row), P = b->S(kNumPrompt, row);
    if (num_tokens < P || num_tokens > T)
        return fail(RIC_ERANGE, "row %d: %d tokens outside [prompt %d, history %d]", row, num_tokens, P, T);
    // A later append lands where a still-staged one may write; the ops of one
    // flush run in parallel, so the staged writes go first.
    if (num_tokens < T) {
        rc = before_row_overwrite(b, row);
        if (rc) return rc;
    }
    b->S(kNumTokens, row) = num_tokens;
    b->mark(kNumTokens, row);
    b->scheduled = false;
    return RIC_OK;
}

static int set_blocks(ric_batch* b, uint64_t req_id, int32_t g, const int32_t* ids, int32_t n, bool replace) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    if (g < 0 || g >= b->L.groups) return fail(RIC_EINVAL, "group %d outside [0, %d)", g, b->L.groups);
    int32_t row;
    int rc = find(b, req_id, &row);
    if (rc) return rc;
    const int col = blocks_col(g);
    const int32_t cap = group_cap(b->cfg, g);
    const int32_t nb = replace ? 0 : b->S(col, row);
    if (n < 0 || (int64_t)nb + n > cap)
        return fail(RIC_EFULL, "row %d group %d: %d + %d blocks exceed the table capacity %d", row, g, nb, n, cap);
    if (n > 0 && !ids) return fail(RIC_EINVAL, "ids is NULL");
    rc = check_blocks(b, g, ids, n);
    if (rc) return rc;
    if (replace) {
        rc = before_row_overwrite(b, row);
        if (rc) return rc;
    }
    rc = stage(b, b->blk(g) + (int64_t)row * b->bstride(g) + nb, ids, (size_t)n);
    if (rc) return rc;
    b->S(col, row) = nb + n;
    b->mark(col, row);
    b->pending_epoch[row] = b->epoch;
    b->scheduled = false;
    return RIC_OK;
}

int ric_append_blocks(ric_batch* b, uint64_t req_id, const int32_t* ids, int32_t n) {
    return set_blocks(b, req_id, 0, ids, n, false);
}

int ric_replace_blocks(ric_batch* b, uint64_t req_id, const int32_t* ids, int32_t n) {
    return set_blocks(b, req_id, 0, ids, n, true);
}

int ric_append_blocks_group(ric_batch* b, uint64_t req_id, int32_t group, const int32_t* ids, int32_t n) {
    return set_blocks(b, req_id, group, ids, n, false);
}

int ric_replace_blocks_group(ric_batch* b, uint64_t req_id, int32_t group, const int32_t* ids, int32_t n) {
    return set_blocks(b, req_id, group, ids, n, true);
}

int32_t ric_condense_plan(const uint8_t* live, int32_t num_rows, int32_t* holes, int32_t* sources) {
    if (!live || num_rows < 0) return RIC_EINVAL;
    int32_t lo = 0, hi = num_rows - 1, k = 0;
    for (;;) {
        while (lo < num_rows && live[lo]) ++lo;     // next hole from the bottom
        while (hi >= 0 && !live[hi]) --hi;          // next live row from the top
        if (lo >= num_rows || hi < 0 || lo >= hi) break;
        if (holes) holes[k] = lo;
        if (sources) sources[k] = hi;
        ++k;
        ++lo;
        --hi;
    }
    return k;
}

int ric_condense(ric_batch* b, int32_t* out_num_moved) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    const int MR = b->cfg.max_num_reqs;
    std::vector<int32_t> holes(MR), srcs(MR);
    const int32_t np = ric_condense_plan(b->live.data(), MR, holes.data(), srcs.data());
    if (np > 0) {
        int rc = refuse_if_capturing(b);
        if (rc) return rc;
        // The pair list rides in the log with any staged deltas; the flush
        // applies them all before the move kernel runs on the same stream.
        std::vector<int32_t> pairs(2 * (size_t)np);
        int32_t max_T = 0;
        for (int32_t k = 0; k < np; ++k) {
            pairs[2 * k] = holes[k];
            pairs[2 * k + 1] = srcs[k];
            max_T = std::max(max_T, b->S(kNumTokens, srcs[k]));
        }
        rc = stage(b, b->d_pairs, pairs.data(), pairs.size());
        if (rc) return rc;
        rc = flush(b);
        if (rc) return rc;
        MoveParams mp{};
        mp.pairs = b->d_pairs;
        mp.tokens = b->d_tok;
        for (int g = 0; g < b->L.groups; ++g) {
            mp.blocks[g] = b->blk(g);
            mp.blk_stride[g] = b->bstride(g);
        }
        mp.num_groups = b->L.groups;
        mp.scal = b->d_scal;
        mp.tok_stride = b->L.tok_stride;
        mp.max_num_reqs = MR;
        mp.num_pairs = np;
        mp.chunk_vec4 = 1024;  // 16 KiB of history per workgroup
        const int chunks = (int)(((int64_t)max_T + 4 * mp.chunk_vec4 - 1) / (4 * mp.chunk_vec4));
        HIP_TRY(launch_move_rows(mp, chunks, b->stream));
        for (int32_t k = 0; k < np; ++k) {
            const int32_t h = holes[k], s = srcs[k];
            for (int c = 0; c < kNumScalarCols; ++c) b->S(c, h) = b->S(c, s);
            b->live[h] = 1;
            b->live[s] = 0;
            b->req_at[h] = b->req_at[s];
            b->row_of[b->req_at[h]] = h;
        }
    }
    b->scheduled = false;
    if (out_num_moved) *out_num_moved = np;
    return RIC_OK;
}

int ric_append_sampled(ric_batch* b, int32_t n, const int32_t* rows, const int32_t* src_index,
                       const int32_t* dev_tokens, int32_t dev_tokens_len) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    if (n < 0 || n > b->cfg.max_num_reqs) return fail(RIC_EINVAL, "n %d outside [0, max_num_reqs]", n);
    if (n == 0) return RIC_OK;
    if (!rows || !dev_tokens || dev_tokens_len <= 0) return fail(RIC_EINVAL, "NULL or empty argument");
    std::vector<uint8_t> seen(b->cfg.max_num_reqs, 0);
    std::vector<int64_t> off((size_t)n);
    std::vector<int32_t> idx((size_t)n);
    for (int32_t k = 0; k < n; ++k) {
        const int32_t r = rows[k];
        if (r < 0 || r >= b->cfg.max_num_reqs || !b->live[r]) return fail(RIC_EINVAL, "row %d is not live", r);
        if (seen[r]) return fail(RIC_EINVAL, "row %d listed twice", r);
        seen[r] = 1;
        const int32_t T = b->S(kNumTokens, r);
        if (T + 1 > b->cfg.max_model_len) return fail(RIC_EFULL, "row %d: token history full", r);
        idx[k] = src_index ? src_index[k] : k;
        if (idx[k] < 0 || idx[k] >= dev_tokens_len)
            return fail(RIC_EINVAL, "source index %d outside [0, %d)", idx[k], dev_tokens_len);
        off[k] = (int64_t)r * b->L.tok_stride + T;
    }
    int rc = refuse_if_capturing(b);
    if (rc) return rc;
    rc = stage(b, b->d_samp_off, off.data(), 2 * (size_t)n);
    if (rc) return rc;
    rc = stage(b, b->d_samp_idx, idx.data(), (size_t)n);
    if (rc) return rc;
    for (int32_t k = 0; k < n; ++k) {
        b->S(kNumTokens, rows[k]) += 1;
        b->mark(kNumTokens, rows[k]);
    }
    b->scheduled = false;
    rc = flush(b);
    if (rc) return rc;
    HIP_TRY(launch_append_sampled(b->d_tok, b->d_samp_off, b->d_samp_idx, dev_tokens, dev_tokens_len, n,
                                  b->d_dscal + 7, b->stream));
    return RIC_OK;
}

int ric_spec_decode_metadata(ric_batch* b, const int32_t* num_draft_tokens, ric_spec_decode* out) {
    if (!b || !out) return fail(RIC_EINVAL, "NULL argument");
    DeviceScope ds(b);
    if (!b->scheduled || !b->compiled) return fail(RIC_ESTATE, "needs a compile of the current schedule");
    const int32_t R = b->sched_R;
    if (R > 0 && !num_draft_tokens) return fail(RIC_EINVAL, "num_draft_tokens is NULL");
    int64_t num_logits = 0, num_draft = 0;
    for (int32_t i = 0; i < R; ++i) {
        const int32_t d = num_draft_tokens[i];
        if (d < 0 || d + 1 > b->S(kNumScheduled, i))
            return fail(RIC_EINVAL, "row %d: %d drafts need more than its %d scheduled tokens", i, d,
                        b->S(kNumScheduled, i));
        num_logits += d + 1;
        num_draft += d;
    }
    int rc = refuse_if_capturing(b);
    if (rc) return rc;
    rc = stage(b, b->d_spec_d, num_draft_tokens, (size_t)R);
    if (rc) return rc;
    rc = flush(b);
    if (rc) return rc;
    SpecParams p{};
    p.qsl = b->d_qsl;
    p.input_ids = b->d_ids;
    p.num_draft = b->d_spec_d;
    p.num_reqs = R;
    p.num_logits = (int32_t)num_logits;
    p.num_tiles = (int32_t)((num_logits + 255) / 256);
    p.logits_indices = b->d_spec_logits;
    p.cu_num_logits = b->d_spec_cu;
    p.target = b->d_spec_target;
    p.bonus = b->d_spec_bonus;
    p.draft_ids = b->d_spec_draft;
    HIP_TRY(launch_spec_decode(p, b->stream));
    out->logits_indices = b->d_spec_logits;
    out->cu_num_logits = b->d_spec_cu;
    out->target_logits_indices = b->d_spec_target;
    out->bonus_logits_indices = b->d_spec_bonus;
    out->draft_token_ids = b->d_spec_draft;
    out->num_logits = (int32_t)num_logits;
    out->num_draft_tokens = (int32_t)num_draft;
    return RIC_OK;
}

int ric_correct_computed(ric_batch* b, int32_t n, const int32_t* rows, const int32_t* prev_index,
                         const int32_t* num_draft, const int32_t* dev_num_accepted, int32_t prev_len,
                         const int32_t* dev_sampled, int64_t sampled_stride, int32_t* dev_status) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    if (!b->scheduled || b->compiled)
        return fail(RIC_ESTATE, "needs a schedule that has not been compiled yet");
    if (b->corrected) return fail(RIC_ESTATE, "this schedule's counts were corrected already");
    const int32_t R = b->sched_R;
    if (n < 0 || n > R) return fail(RIC_EINVAL, "n %d outside [0, scheduled rows %d]", n, R);
    if (n == 0) return RIC_OK;
    if (!rows || !prev_index || !num_draft || !dev_num_accepted)
        return fail(RIC_EINVAL, "NULL argument");
    if (prev_len <= 0) return fail(RIC_EINVAL, "prev_len %d must be positive", prev_len);
    std::vector<uint8_t> seen((size_t)R, 0);
    for (int32_t k = 0; k < n; ++k) {
        const int32_t r = rows[k], d = num_draft[k];
        if (r < 0 || r >= R) return fail(RIC_EINVAL, "row %d outside the scheduled rows [0, %d)", r, R);
        if (seen[r]) return fail(RIC_EINVAL, "row %d listed twice", r);
        seen[r] = 1;
        if (prev_index[k] < 0 || prev_index[k] >= prev_len)
            return fail(RIC_EINVAL, "sampler position %d outside [0, %d)", prev_index[k], prev_len);
        // the correction lowers c by at most d, so the scheduled c must hold d
        if (d < 0 || d > b->S(kNumComputed, r))
            return fail(RIC_EINVAL, "row %d: %d drafts, but its scheduled count is %d", r, d,
                        b->S(kNumComputed, r));
        if (dev_sampled && sampled_stride < (int64_t)d + 1)
            return fail(RIC_EINVAL, "sampled_stride %lld cannot hold the %d tokens of row %d", (long long)sampled_stride,
                        d + 1, r);
    }
    const int MR = b->cfg.max_num_reqs;
    int rc = refuse_if_capturing(b);
    if (rc) return rc;
    rc = stage(b, b->d_corr, rows, (size_t)n);
    if (rc) return rc;
    rc = stage(b, b->d_corr + MR, prev_index, (size_t)n);
    if (rc) return rc;
    rc = stage(b, b->d_corr + 2 * (size_t)MR, num_draft, (size_t)n);
    if (rc) return rc;
    rc = flush(b);    // the schedule's counts and these arrays land before the kernel reads them
    if (rc) return rc;
    CorrectParams p{};
    p.computed = b->dcol(kNumComputed);
    p.tokens = b->d_tok;
    p.tok_stride = b->L.tok_stride;
    p.rows = b->d_corr;
    p.prev = b->d_corr + MR;
    p.draft = b->d_corr + 2 * (size_t)MR;
    p.accepted = dev_num_accepted;
    p.sampled = dev_sampled;
    p.sampled_stride = sampled_stride;
    p.status = dev_status;
    p.n = n;
    HIP_TRY(launch_correct_computed(p, b->stream));
    b->corrected = true;
    return RIC_OK;
}

int ric_block_table_padded(ric_batch* b, int32_t group, int32_t ratio, int32_t width, int32_t fill, int32_t* dst) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    if (!b->scheduled) return fail(RIC_ESTATE, "ric_schedule must follow the last row change");
    if (group < 0 || group >= b->L.groups) return fail(RIC_EINVAL, "group %d outside [0, %d)", group, b->L.groups);
    if (ratio < 1) return fail(RIC_EINVAL, "kernel_blocks_per_block %d < 1", ratio);
    if ((int64_t)group_pool(b->cfg, group) * ratio >= (int64_t(1) << 31))
        return fail(RIC_EINVAL, "kernel_blocks_per_block %d: expanded block ids would not fit in int32", ratio);
    const int64_t cap = (int64_t)ratio * group_cap(b->cfg, group);
    if (width < 0 || width > cap) return fail(RIC_EINVAL, "width %d outside [0, %lld]", width, (long long)cap);
    if (width > 0 && b->sched_R > 0 && !dst) return fail(RIC_EINVAL, "dst is NULL");
    int rc = flush(b);
    if (rc) return rc;
    PaddedTableParams p{};
    p.blocks = b->blk(group);
    p.num_blocks = b->dcol(blocks_col(group));
    p.dst = dst;
    p.blk_stride = b->bstride(group);
    p.rows = b->sched_R;
    p.width = width;
    p.fill = fill;
    p.ratio = ratio;
    HIP_TRY(launch_padded_table(p, b->stream));
    return RIC_OK;
}

int ric_flush(ric_batch* b) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    return flush(b);
}

int32_t ric_num_reqs(const ric_batch* b) { return b ? b->num_live : RIC_EINVAL; }

int32_t ric_row_of(const ric_batch* b, uint64_t req_id) {
    if (!b) return RIC_EINVAL;
    auto it = b->row_of.find(req_id);
    return it == b->row_of.end() ? RIC_ENOENT : it->second;
}

int ric_req_at(const ric_batch* b, int32_t row, uint64_t* out_req_id) {
    if (!b || !out_req_id) return fail(RIC_EINVAL, "NULL argument");
    if (row < 0 || row >= b->cfg.max_num_reqs) return fail(RIC_ERANGE, "row %d out of range", row);
    if (!b->live[row]) return RIC_ENOENT;
    *out_req_id = b->req_at[row];
    return RIC_OK;
}

int ric_get_columns(const ric_batch* b, ric_columns* o) {
    if (!b || !o) return fail(RIC_EINVAL, "NULL argument");
    ric_batch* m = const_cast<ric_batch*>(b);
    o->tokens = m->d_tok;
    o->blocks = m->d_blk;
    o->token_stride = b->L.tok_stride;
    o->block_stride = b->L.blk_stride;
    o->num_tokens = m->dcol(kNumTokens);
    o->num_prompt = m->dcol(kNumPrompt);
    o->num_computed = m->dcol(kNumComputed);
    o->num_scheduled = m->dcol(kNumScheduled);
    o->num_blocks = m->dcol(kNumBlocks);
    o->top_k = m->dcol(kTopK);
    o->temperature = reinterpret_cast<float*>(m->dcol(kTemperature));
    o->top_p = reinterpret_cast<float*>(m->dcol(kTopP));
    o->repetition_penalty = reinterpret_cast<float*>(m->dcol(kRepPenalty));
    for (int g = 0; g < RIC_MAX_KV_GROUPS; ++g) {
        const bool on = g < b->L.groups;
        o->group_blocks[g] = on ? m->blk(g) : nullptr;
        o->group_block_stride[g] = on ? m->bstride(g) : 0;
        o->group_num_blocks[g] = on ? m->dcol(blocks_col(g)) : nullptr;
    }
    return RIC_OK;
}

int ric_sync(ric_batch* b) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    HIP_TRY(hipStreamSynchronize(b->stream));
    return RIC_OK;
}

int ric_read_device(void* host_dst, const void* dev_src, size_t bytes) {
    if (bytes == 0) return RIC_OK;
    if (!host_dst || !dev_src) return fail(RIC_EINVAL, "NULL pointer argument");
    HIP_TRY(hipDeviceSynchronize());
    HIP_TRY(hipMemcpy(host_dst, dev_src, bytes, hipMemcpyDeviceToHost));
    return RIC_OK;
}

int ric_check_step(const ric_config* cfg, int32_t R, const int32_t* c, const int32_t* q, const int32_t* P,
                   const int32_t* T, const int32_t* nb, int32_t n_pad, ric_step* out) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (R > 0 && (!P || !T || !nb)) return fail(RIC_EINVAL, "row arrays are NULL");
    int32_t N, mq, ms, ns;
    rc = check_step_rows(*cfg, R, c, q, P, T, nb, &N, &mq, &ms, &ns);
    if (rc) return rc;
    if (n_pad < N || n_pad > cfg->max_num_batched_tokens)
        return fail(RIC_EINVAL, "num_tokens_padded %d outside [N=%d, max_num_batched_tokens=%d]", n_pad, N,
                    cfg->max_num_batched_tokens);
    if (out) {
        memset(out, 0, sizeof *out);
        out->num_reqs = R;
        out->num_actual_tokens = N;
        out->num_tokens_padded = n_pad;
        out->max_query_len = mq;
        out->max_seq_len = ms;
        out->num_sampled = ns;
    }
    return RIC_OK;
}

int ric_schedule(ric_batch* b, int32_t R, const int32_t* c, const int32_t* q) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    if (R != b->num_live) return fail(RIC_EINVAL, "num_reqs %d but %d requests are live", R, b->num_live);
    if (b->used_rows() != R) return fail(RIC_ESTATE, "rows are not condensed: live rows must be [0, %d)", R);
    const int MR = b->cfg.max_num_reqs;
    int32_t N, mq, ms, ns;
    int rc = check_step_rows(b->cfg, R, c, q, &b->scal[(size_t)kNumPrompt * MR], &b->scal[(size_t)kNumTokens * MR],
                             &b->scal[(size_t)kNumBlocks * MR], &N, &mq, &ms, &ns);
    if (rc) return rc;
    // further groups with per-token slots must also cover every scheduled position
    for (int g = 1; g < b->L.groups; ++g) {
        if (!group_slots(b->cfg, g)) continue;
        const int64_t B = group_B(b->cfg, g);
        for (int32_t i = 0; i < R; ++i)
            if (((int64_t)c[i] + q[i] + B - 1) / B > b->S(blocks_col(g), i))
                return fail(RIC_EINVAL, "row %d group %d: %d blocks cannot hold position %lld", i, g,
                            b->S(blocks_col(g), i), (long long)c[i] + q[i] - 1);
    }
    for (int32_t i = 0; i < R; ++i) {
        b->S(kNumComputed, i) = c[i];
        b->S(kNumScheduled, i) = q[i];
    }
    if (R > 0) {
        b->mark(kNumComputed, 0);
        b->mark(kNumComputed, R - 1);
        b->mark(kNumScheduled, 0);
        b->mark(kNumScheduled, R - 1);
    }
    b->scheduled = true;
    b->compiled = false;
    b->corrected = false;
    b->sched_R = R;
    b->sched_N = N;
    b->sched_max_q = mq;
    b->sched_max_seq = ms;
    b->sched_sampled = ns;
    return RIC_OK;
}

}  // extern "C"

namespace {

CompileParams compile_params(ric_batch* b, int32_t n_pad) {
    CompileParams p{};
    p.scal = b->d_scal;
    p.tokens = b->d_tok;
    p.blocks = b->d_blk;
    p.tok_stride = b->L.tok_stride;
    p.blk_stride = b->L.blk_stride;
    p.max_num_reqs = b->cfg.max_num_reqs;
    p.num_reqs = b->sched_R;
    p.n_pad = n_pad;
    p.block_size = b->cfg.block_size;
    p.block_shift = ilog2_exact(b->cfg.block_size);
    p.null_slot = b->cfg.null_block * b->cfg.block_size;
    p.num_token_tiles = (n_pad + kCompileTile - 1) / kCompileTile;
    p.input_ids = b->d_ids;
    p.positions = b->d_pos;
    p.req_indices = b->d_req;
    p.slot_mapping = b->d_slot;
    p.query_start_loc = b->d_qsl;
    p.seq_lens = b->d_seq;
    p.logits_indices = b->d_logits;
    p.discard = b->d_discard;
    p.sample_indices = b->d_sample;
    p.dev_scalars = b->d_dscal;
    p.cu_seqlens_k = b->d_cuk;
    p.num_extra_groups = 0;
    for (int g = 1; g < b->L.groups; ++g) {
        if (!group_slots(b->cfg, g)) continue;
        const int x = p.num_extra_groups++;
        const int32_t B = group_B(b->cfg, g);
        p.xblocks[x] = b->blk(g);
        p.xblk_stride[x] = b->bstride(g);
        p.xblock_size[x] = B;
        p.xblock_shift[x] = ilog2_exact(B);
        p.xnull_slot[x] = b->cfg.null_block * B;
        p.xslot_mapping[x] = b->d_xslot[g];
    }
    return p;
}

void fill_step(const ric_batch* b, int32_t n_pad, ric_step* out) {
    if (!out) return;
    out->input_ids = b->d_ids;
    out->positions = b->d_pos;
    out->req_indices = b->d_req;
    out->slot_mapping = b->d_slot;
    out->query_start_loc = b->d_qsl;
    out->seq_lens = b->d_seq;
    out->logits_indices = b->d_logits;
    out->discard = b->d_discard;
    out->sample_indices = b->d_sample;
    out->dev_scalars = b->d_dscal;
    out->cu_seqlens_k = b->d_cuk;
    for (int g = 0; g < RIC_MAX_KV_GROUPS; ++g)
        out->group_slot_mapping[g] = (g == 0) ? b->d_slot : (g < b->L.groups ? b->d_xslot[g] : nullptr);
    out->num_reqs = b->sched_R;
    out->num_actual_tokens = b->sched_N;
    out->num_tokens_padded = n_pad;
    out->max_query_len = b->sched_max_q;
    out->max_seq_len = b->sched_max_seq;
    out->num_sampled = b->sched_sampled;
    out->kv_path = 0;
}

int check_compile_args(const ric_batch* b, int32_t n_pad) {
    if (!b->scheduled) return fail(RIC_ESTATE, "ric_schedule must follow the last row change");
    if (n_pad < b->sched_N || n_pad > b->cfg.max_num_batched_tokens)
        return fail(RIC_EINVAL, "num_tokens_padded %d outside [N=%d, max_num_batched_tokens=%d]", n_pad,
                    b->sched_N, b->cfg.max_num_batched_tokens);
    return RIC_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Argument checks shared by the K/V-writing calls; fills the launch
// parameters that do not depend on the layer range.
int kv_params(const void* const* k, const void* const* v, void* const* k_cache, void* const* v_cache,
              int32_t num_layers, int32_t num_tokens, int64_t src_row_stride, int32_t row_bytes, int64_t num_slots,
              int32_t* dev_status, uint32_t flags, KVParams* p) {
    if (num_layers < 0 || num_tokens < 0) return fail(RIC_EINVAL, "negative count");
    if (flags != 0) return fail(RIC_EINVAL, "flags 0x%x: no flag is defined (pass 0)", flags);
    if (num_tokens > kMaxRowsPerLaunch)
        return fail(RIC_EINVAL, "num_tokens %d above %d per call (the grid counts work-items in 32 bits)",
                    num_tokens, kMaxRowsPerLaunch);
    if (num_layers > 0 && (!k || !v || !k_cache || !v_cache)) return fail(RIC_EINVAL, "NULL pointer argument");
    if (row_bytes <= 0 || row_bytes % 16 != 0) return fail(RIC_EINVAL, "row_bytes %d not a positive multiple of 16", row_bytes);
    if (src_row_stride == 0) src_row_stride = row_bytes;
    if (src_row_stride < row_bytes || src_row_stride % 16 != 0)
        return fail(RIC_EINVAL, "src_row_stride %lld must be a multiple of 16 and >= row_bytes", (long long)src_row_stride);
    if (num_slots <= 0) return fail(RIC_EINVAL, "num_slots must be positive");
    for (int32_t l = 0; l < num_layers; ++l)
        if (!k[l] || !v[l] || !k_cache[l] || !v_cache[l] || !aligned16(k[l]) || !aligned16(v[l]) ||
            !aligned16(k_cache[l]) || !aligned16(v_cache[l]))
            return fail(RIC_EINVAL, "layer %d: NULL or misaligned pointer", l);
    *p = KVParams{};
    p->src_stride = src_row_stride;
    p->num_slots = num_slots;
    p->status = dev_status;
    p->num_tokens = num_tokens;
    p->row_bytes = row_bytes;
    p->chunk_shift = ilog2_exact(row_bytes / 16);
    p->rows_per_wg = 0;
    return RIC_OK;
}

void set_layers(KVParams* p, const void* const* k, const void* const* v, void* const* k_cache, void* const* v_cache,
                int32_t l0, int nl) {
    for (int i = 0; i < nl; ++i) {
        p->k[i] = static_cast<const uint8_t*>(k[l0 + i]);
        p->v[i] = static_cast<const uint8_t*>(v[l0 + i]);
        p->kc[i] = static_cast<uint8_t*>(k_cache[l0 + i]);
        p->vc[i] = static_cast<uint8_t*>(v_cache[l0 + i]);
    }
}

}  // namespace

extern "C" {

int ric_compile(ric_batch* b, int32_t n_pad, ric_step* out) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    int rc = check_compile_args(b, n_pad);
    if (rc) return rc;
    rc = flush(b);
    if (rc) return rc;
    HIP_TRY(launch_compile(compile_params(b, n_pad), b->stream));
    b->compiled = true;
    fill_step(b, n_pad, out);
    return RIC_OK;
}

int ric_compile_and_cache(ric_batch* b, int32_t n_pad, const void* const* k, const void* const* v,
                          void* const* k_cache, void* const* v_cache, int32_t num_layers, int64_t src_row_stride,
                          int32_t row_bytes, int64_t num_slots, int32_t* dev_status, uint32_t flags,
                          ric_step* out) {
    if (!b) return fail(RIC_EINVAL, "handle is NULL");
    DeviceScope ds(b);
    int rc = check_compile_args(b, n_pad);
    if (rc) return rc;
    const uint32_t path = flags & 3u;
    if (path == 3u) return fail(RIC_EINVAL, "flags 0x%x: RIC_FUSE_ALWAYS and RIC_FUSE_NEVER together", flags);
    KVParams kv{};
    rc = kv_params(k, v, k_cache, v_cache, num_layers, n_pad, src_row_stride, row_bytes, num_slots, dev_status,
                   flags & ~3u, &kv);
    if (rc) return rc;
    rc = flush(b);
    if (rc) return rc;
    const CompileParams p = compile_params(b, n_pad);
    kv.slot = b->d_slot;
    // A step whose scheduled tokens average 1024 or more per request is mostly
    // long contiguous runs.  With rows of 1 KiB or more the library's own
    // choice keeps those on the compile kernel followed by the K/V kernel's
    // small streaming tiles: the single kernel's tile shape for them is
    // faster only when it runs right after itself (long-context 46.7 against
    // 50.3 us) and slower after any other kernel (55-57 us after a read, a
    // matrix product or an idle gap, 70 us after a large write), while the
    // two kernels take 51 us in every case.  With narrower rows (a tensor-
    // parallel shard's heads) the compile is a larger share of the step and
    // the single kernel stays ahead after other kernels too (long-context,
    // 256 B rows: 9.8 against 14.8 us after matrix products), so every step
    // takes it; so do all other steps.
    const bool long_runs = (int64_t)b->sched_N >= (int64_t)1024 * std::max<int32_t>(b->sched_R, 1);
    const bool own_choice_fuses = !long_runs || row_bytes < 1024;
    const bool fuse = (path == RIC_FUSE_ALWAYS || (path == 0 && own_choice_fuses)) && num_layers > 0 && n_pad > 0 &&
                      fused_kv_supported(row_bytes);
    int32_t done = 0;
    if (fuse) {
        done = std::min<int32_t>(kMaxLayersPerLaunch, num_layers);
        set_layers(&kv, k, v, k_cache, v_cache, 0, done);
        HIP_TRY(launch_compile_kv(p, kv, done, long_runs, b->stream));
    } else {
        HIP_TRY(launch_compile(p, b->stream));
    }
    // Layers past the first launch, or rows the fused kernel does not take:
    // the K/V kernels through the slot mapping just written.
    for (int32_t l0 = done; l0 < num_layers && n_pad > 0; l0 += kMaxLayersPerLaunch) {
        const int nl = std::min<int>(kMaxLayersPerLaunch, num_layers - l0);
        set_layers(&kv, k, v, k_cache, v_cache, l0, nl);
        HIP_TRY(launch_kv_scatter(kv, nl, b->stream));
    }
    b->compiled = true;
    fill_step(b, n_pad, out);
    if (out) out->kv_path = fuse ? 1 : 2;
    return RIC_OK;
}

int ric_reshape_and_cache(const void* const* k, const void* const* v, void* const* k_cache, void* const* v_cache,
                          int32_t num_layers, const int32_t* slot_mapping, int32_t num_tokens,
                          int64_t src_row_stride, int32_t row_bytes, int64_t num_slots, int32_t* dev_status,
                          uint32_t flags, void* stream) {
    if (num_layers < 0 || num_tokens < 0) return fail(RIC_EINVAL, "negative count");
    if (flags != 0) return fail(RIC_EINVAL, "flags 0x%x: no flag is defined (pass 0)", flags);
    if (num_layers == 0 || num_tokens == 0) return RIC_OK;
    if (!slot_mapping) return fail(RIC_EINVAL, "NULL pointer argument");
    KVParams p{};
    int rc = kv_params(k, v, k_cache, v_cache, num_layers, num_tokens, src_row_stride, row_bytes, num_slots,
                       dev_status, flags, &p);
    if (rc) return rc;
    p.slot = slot_mapping;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t l0 = 0; l0 < num_layers; l0 += kMaxLayersPerLaunch) {
        const int nl = std::min<int>(kMaxLayersPerLaunch, num_layers - l0);
        set_layers(&p, k, v, k_cache, v_cache, l0, nl);
        HIP_TRY(launch_kv_scatter(p, nl, s));
    }
    return RIC_OK;
}

int ric_gather_rows(const void* src, int64_t src_row_stride, int64_t src_rows, const int32_t* idx,
                    const int32_t* dev_count, int32_t max_rows, int32_t row_bytes, void* dst,
                    int64_t dst_row_stride, int32_t* dev_status, void* stream) {
    if (max_rows < 0) return fail(RIC_EINVAL, "max_rows negative");
    if (max_rows == 0) return RIC_OK;
    if (max_rows > kMaxRowsPerLaunch)
        return fail(RIC_EINVAL, "max_rows %d above %d per call (the grid counts work-items in 32 bits)", max_rows,
                    kMaxRowsPerLaunch);
    if (!src || !idx || !dst) return fail(RIC_EINVAL, "NULL pointer argument");
    if (row_bytes <= 0 || row_bytes % 16 != 0) return fail(RIC_EINVAL, "row_bytes %d not a positive multiple of 16", row_bytes);
    if (src_row_stride == 0) src_row_stride = row_bytes;
    if (dst_row_stride == 0) dst_row_stride = row_bytes;
    if (src_row_stride < row_bytes || dst_row_stride < row_bytes || src_row_stride % 16 || dst_row_stride % 16)
        return fail(RIC_EINVAL, "strides must be multiples of 16 and >= row_bytes");
    if (!aligned16(src) || !aligned16(dst)) return fail(RIC_EINVAL, "src/dst must be 16-byte aligned");
    if (src_rows < 0) return fail(RIC_EINVAL, "src_rows negative");
    GatherParams p{};
    p.src = static_cast<const uint8_t*>(src);
    p.src_stride = src_row_stride;
    p.src_rows = src_rows;
    p.idx = idx;
    p.dev_count = dev_count;
    p.dst = static_cast<uint8_t*>(dst);
    p.dst_stride = dst_row_stride;
    p.status = dev_status;
    p.max_rows = max_rows;
    p.row_bytes = row_bytes;
    HIP_TRY(launch_gather(p, static_cast<hipStream_t>(stream)));
    return RIC_OK;
}

size_t ric_check_slots_workspace_bytes(int64_t num_slots) {
    if (num_slots <= 0 || num_slots > (int64_t(1) << 31)) return 0;
    return align_up((size_t)((num_slots + 31) / 32) * 4, kAlign);
}

int ric_check_slots(const int32_t* slot_mapping, int32_t num_tokens, const int32_t* dev_num_tokens,
                    int64_t num_slots, void* workspace, size_t workspace_bytes, int32_t* dev_result,
                    void* stream) {
    if (num_tokens < 0 || num_tokens > kMaxRowsPerLaunch)
        return fail(RIC_EINVAL, "num_tokens %d outside [0, %d]", num_tokens, kMaxRowsPerLaunch);
    if (num_slots <= 0 || num_slots > (int64_t(1) << 31))
        return fail(RIC_EINVAL, "num_slots %lld outside [1, 2^31]", (long long)num_slots);
    if (!dev_result || (num_tokens > 0 && !slot_mapping)) return fail(RIC_EINVAL, "NULL pointer argument");
    if (!workspace || reinterpret_cast<uintptr_t>(workspace) % 4 != 0)
        return fail(RIC_EINVAL, "workspace is NULL or not 4-byte aligned");
    const size_t need = (size_t)((num_slots + 31) / 32) * 4;
    if (workspace_bytes < need)
        return fail(RIC_EINVAL, "workspace of %zu bytes, %zu needed for %lld slots", workspace_bytes, need,
                    (long long)num_slots);
    HIP_TRY(launch_check_slots(slot_mapping, num_tokens, dev_num_tokens, num_slots,
                               static_cast<uint32_t*>(workspace), dev_result, static_cast<hipStream_t>(stream)));
    return RIC_OK;
}

int ric_check_slots_noalloc(const int32_t* slot_mapping, int32_t num_tokens, const int32_t* dev_num_tokens,
                            int64_t num_slots, int32_t* dev_result, void* stream) {
    if (num_tokens < 0 || num_tokens > kMaxRowsPerLaunch)
        return fail(RIC_EINVAL, "num_tokens %d outside [0, %d]", num_tokens, kMaxRowsPerLaunch);
    if (num_slots <= 0) return fail(RIC_EINVAL, "num_slots %lld must be positive", (long long)num_slots);
    if (num_slots > kCheckScratchWords * 32)
        return fail(RIC_ERANGE, "num_slots %lld above the %lld slots the library's static bitmap holds "
                                "(use ric_check_slots with a workspace)", (long long)num_slots,
                    (long long)(kCheckScratchWords * 32));
    if (!dev_result || (num_tokens > 0 && !slot_mapping)) return fail(RIC_EINVAL, "NULL pointer argument");
    uint32_t* bits = nullptr;
    HIP_TRY(check_scratch_for_current_device(&bits));
    HIP_TRY(launch_check_slots(slot_mapping, num_tokens, dev_num_tokens, num_slots, bits, dev_result,
                               static_cast<hipStream_t>(stream)));
    return RIC_OK;
}

int32_t ric_padded_size(const int32_t* sizes, int32_t n, int32_t num_tokens) {
    if (num_tokens < 0 || n < 0 || (n > 0 && !sizes)) return RIC_EINVAL;
    int32_t best = -1;
    for (int32_t i = 0; i < n; ++i)
        if (sizes[i] >= num_tokens && (best < 0 || sizes[i] < best)) best = sizes[i];
    return best < 0 ? num_tokens : best;
}

}  // extern "C"
