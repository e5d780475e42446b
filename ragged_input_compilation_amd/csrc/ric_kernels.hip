// HIP kernels for gfx950 (CDNA4, wave64): step compile, paged K/V write, the
// two in one kernel, row gather, condense row move, staged-delta apply, the
// slot-collision check, and the small kernels of the next rows (padded
// tables, speculative-decoding indices, sampled-token append, correction of
// optimistic computed counts).
//
// Sources (page title, section):
//   [P1] "vLLM 源码完全拆解（五）：GPUModelRunner 如何把动态请求拼成一次 GPU 前向"
//   [P3] "变长批处理与一次混合前向"
//   [P4] "04 · 模型执行与 CUDA Graph"
//
// Nothing here is a contraction, so no MFMA: the compile is a few integer
// operations per token behind two dependent loads, and the K/V write and the
// gather are indexed copies bound by HBM bandwidth.  The copies move 16-byte
// vectors per lane, use non-temporal accesses where a byte is touched once per
// step and the measurements favour them, and compute byte offsets in 64 bits.
#include <algorithm>
#include <mutex>

#include "ric_internal.h"

namespace ric {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kWave = 64;

// Scans across a 64-lane wave with DPP (data-parallel lane moves between
// registers, no LDS traffic): row shifts by 1, 2, 4 and 8 scan each row of 16
// lanes, then lane 15 is broadcast into rows 1 and 3 and lane 31 into rows 2
// and 3, which carries the row totals across the wave.  A lane whose source
// lies outside its row, or whose row the mask leaves out, keeps `identity`.
// All 64 lanes must be active: callers reach these with every thread of a
// full-wave workgroup.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_move(int identity, int x) {
    return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROW_MASK, 0xf, false);
}

__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += dpp_move<kDppRowShr1, 0xf>(0, x);
    x += dpp_move<kDppRowShr2, 0xf>(0, x);
    x += dpp_move<kDppRowShr4, 0xf>(0, x);
    x += dpp_move<kDppRowShr8, 0xf>(0, x);
    x += dpp_move<kDppRowBcast15, 0xa>(0, x);
    x += dpp_move<kDppRowBcast31, 0xc>(0, x);
    return x;
}

// Running maximum over lanes 0..l; lane 63 holds the wave's maximum.
__device__ __forceinline__ int wave_inclusive_max(int x) {
    constexpr int lo = -2147483647 - 1;
    x = max(x, dpp_move<kDppRowShr1, 0xf>(lo, x));
    x = max(x, dpp_move<kDppRowShr2, 0xf>(lo, x));
    x = max(x, dpp_move<kDppRowShr4, 0xf>(lo, x));
    x = max(x, dpp_move<kDppRowShr8, 0xf>(lo, x));
    x = max(x, dpp_move<kDppRowBcast15, 0xa>(lo, x));
    x = max(x, dpp_move<kDppRowBcast31, 0xc>(lo, x));
    return x;
}

// Exclusive scan of one value per thread across the workgroup; *total gets
// the sum.  `tmp` holds one int per wave.  Contains barriers: every thread of
// the workgroup must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int x, int* tmp, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int inc = wave_inclusive_scan(x);
    if (lane == kWave - 1) tmp[wid] = inc;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        const int v = tmp[w];
        off += (w < wid) ? v : 0;
        tot += v;
    }
    __syncthreads();
    *total = tot;
    return off + inc - x;
}

// Two exclusive scans and two maxima across the workgroup with one barrier:
// a[0], a[1] are replaced by their exclusive prefix sums (totals in tot[]),
// m[0], m[1] by the workgroup maxima.  `tmp` holds 4 ints per wave and must
// not be reused by the caller afterwards.  Every thread must call it.
template <int NT>
__device__ __forceinline__ void block_scan2_max2(int a[2], int m[2], int* tmp, int tot[2]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int inc0 = wave_inclusive_scan(a[0]);
    const int inc1 = wave_inclusive_scan(a[1]);
    const int m0 = wave_inclusive_max(m[0]);   // the wave's maximum at lane 63
    const int m1 = wave_inclusive_max(m[1]);
    if (lane == kWave - 1) {
        tmp[4 * wid + 0] = inc0;
        tmp[4 * wid + 1] = inc1;
        tmp[4 * wid + 2] = m0;
        tmp[4 * wid + 3] = m1;
    }
    __syncthreads();
    int off0 = 0, off1 = 0, t0 = 0, t1 = 0, mx0 = tmp[2], mx1 = tmp[3];
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) {
        const int v0 = tmp[4 * w + 0];
        const int v1 = tmp[4 * w + 1];
        off0 += (w < wid) ? v0 : 0;
        off1 += (w < wid) ? v1 : 0;
        t0 += v0;
        t1 += v1;
        mx0 = max(mx0, tmp[4 * w + 2]);
        mx1 = max(mx1, tmp[4 * w + 3]);
    }
    a[0] = off0 + inc0 - a[0];
    a[1] = off1 + inc1 - a[1];
    tot[0] = t0;
    tot[1] = t1;
    m[0] = mx0;
    m[1] = mx1;
}

}  // namespace

// ---------------------------------------------------------------------------
// Step compile.  Workgroups 0..num_token_tiles-1 each own a tile of the flat
// token stream; the last workgroup writes the per-request outputs.  Every
// workgroup first rebuilds query_start_loc in LDS from the scheduled counts
// (R <= 8000), so one launch needs no grid-wide synchronisation.
//   query_start_loc: exclusive prefix sum of q       [P1 §第一步]
//   position of token j of request i: c_i + j        [P1 §第二步]
//   input id: token table row i at that position     [P1 §第三步]
//   slot: block_table[i][p / B] * B + p % B          [P1 §Block table 是逐请求的页表]
//   logits index: qsl[i+1] - 1; partial prefills discarded  [P1 §第四步], [P1 §Chunked Prefill]
//   padded tokens -> null block                      [P1 §固定地址与动态有效长度如何共存], [P4 §5]
// The three parts below are shared by the compile kernel and the fused
// compile + K/V kernel, so both produce the same outputs by construction.
// ---------------------------------------------------------------------------

// LDS of one compile workgroup: query_start_loc [R + 1], base [R] (c_i - qsl_i,
// so that position = base + t), one scan word per wave, four reduction words
// per wave.
struct CompileLds {
    int32_t* qsl;
    int32_t* base;
    int32_t* tmp;
    int32_t* red;
    __device__ CompileLds(int32_t* smem, int R)
        : qsl(smem), base(smem + R + 1), tmp(smem + 2 * R + 1), red(smem + 2 * R + 1 + kCompileThreads / kWave) {}
    static constexpr int extra_words = 5 * kCompileThreads / kWave;
};

// What a thread of the per-request workgroup carries from the scan to the
// per-request outputs: its contiguous run of requests [r0, r1) and their
// partial sums and maxima.
struct ReqRun {
    int r0, r1;
    int kept, max_q, max_seq, local_seq;
    uint32_t partial;   // bit k: request r0 + k has not reached the end of its prompt
};

// Rebuilds query_start_loc and the position bases in LDS; returns N.  Each
// thread owns a contiguous run of at most 32 requests (R <= 8000).  A
// request's q and c (and, in the per-request workgroup, its prompt length) are
// loaded together; up to 256 requests that is one round trip per thread.
// Above that the loop takes a thread's requests one after another: issuing
// four at a time measured the same (1024 requests), and all at once (unrolled
// and predicated: larger code) about 1 us slower per compile.  Contains
// barriers: every thread of the workgroup must call it.
__device__ __forceinline__ int scan_requests(const CompileParams& p, const CompileLds& L, bool req_wg, ReqRun& run) {
    const int R = p.num_reqs;
    const int tid = threadIdx.x;
    const int32_t* col_c = p.scal + (int64_t)kNumComputed * p.max_num_reqs;
    const int32_t* col_q = p.scal + (int64_t)kNumScheduled * p.max_num_reqs;
    const int32_t* col_P = p.scal + (int64_t)kNumPrompt * p.max_num_reqs;
    const int per = (R + kCompileThreads - 1) / kCompileThreads;
    run.r0 = min(R, tid * per);
    run.r1 = min(R, run.r0 + per);
    run.kept = 0;
    run.max_q = 0;
    run.max_seq = 0;
    run.local_seq = 0;
    run.partial = 0;
    int local = 0;
    for (int i = run.r0; i < run.r1; ++i) {
        const int q = col_q[i];
        const int c = col_c[i];
        L.qsl[i] = q;
        L.base[i] = c;
        local += q;
        if (req_wg) {
            const int seq = c + q;
            const bool part = seq < col_P[i];
            run.partial |= (part ? 1u : 0u) << (i - run.r0);
            run.kept += part ? 0 : 1;
            run.max_q = max(run.max_q, q);
            run.max_seq = max(run.max_seq, seq);
            run.local_seq += seq;
        }
    }
    int N = 0;
    int off = block_exclusive_scan<kCompileThreads>(local, L.tmp, &N);
    for (int i = run.r0; i < run.r1; ++i) {
        const int q = L.qsl[i];
        L.qsl[i] = off;
        L.base[i] -= off;
        off += q;
    }
    if (tid == 0) L.qsl[R] = N;
    __syncthreads();
    return N;
}

// Token t < n_pad: its group-0 slot; with `write`, also its per-token outputs
// (input id, position, request, slots of every slotted group).
__device__ __forceinline__ int token_outputs(const CompileParams& p, const CompileLds& L, int N, int t, bool write) {
    const int R = p.num_reqs;
    if (t >= N) {
        if (write) {
            p.input_ids[t] = 0;
            p.positions[t] = 0;
            p.req_indices[t] = -1;
            p.slot_mapping[t] = p.null_slot;
            for (int x = 0; x < p.num_extra_groups; ++x) p.xslot_mapping[x][t] = p.xnull_slot[x];
        }
        return p.null_slot;
    }
    // request r: the last one whose interval starts at or before t
    int lo = 0, hi = R - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (L.qsl[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int r = lo;
    const int pos = L.base[r] + t;
    int lb, off;
    if (p.block_shift >= 0) {
        lb = pos >> p.block_shift;
        off = pos & (p.block_size - 1);
    } else {
        lb = pos / p.block_size;
        off = pos - lb * p.block_size;
    }
    int slot;
    // The host validated c + q <= T and the block count; this guard only
    // keeps a corrupted column from turning into a wild read.
    const bool ok = pos >= 0 && pos < p.tok_stride && lb < p.blk_stride;
    if (ok) {
        slot = p.blocks[(int64_t)r * p.blk_stride + lb] * p.block_size + off;
    } else {
        slot = p.null_slot;
    }
    if (!write) return slot;
    p.positions[t] = pos;
    p.req_indices[t] = r;
    if (ok) {
        p.input_ids[t] = p.tokens[(int64_t)r * p.tok_stride + pos];
        p.slot_mapping[t] = slot;
    } else {
        p.input_ids[t] = -1;
        p.slot_mapping[t] = p.null_slot;
        atomicAdd(p.dev_scalars + 6, 1);
    }
    // Further KV-cache groups: the same position through each group's own
    // block table and block size ([P1 §混合 KV Cache：一条请求不止一张页表]).
    for (int x = 0; x < p.num_extra_groups; ++x) {
        const int B = p.xblock_size[x];
        int xlb, xoff;
        if (p.xblock_shift[x] >= 0) {
            xlb = pos >> p.xblock_shift[x];
            xoff = pos & (B - 1);
        } else {
            xlb = pos / B;
            xoff = pos - xlb * B;
        }
        if (pos >= 0 && xlb < p.xblk_stride[x]) {
            p.xslot_mapping[x][t] = p.xblocks[x][(int64_t)r * p.xblk_stride[x] + xlb] * B + xoff;
        } else {
            p.xslot_mapping[x][t] = p.xnull_slot[x];
            atomicAdd(p.dev_scalars + 6, 1);
        }
    }
    return slot;
}

// Per-request outputs, written by one workgroup: compacted-sample positions,
// and the key-side boundaries of a varlen attention call (running total of
// seq_lens), in one pass with the maxima.  Contains a barrier: every thread of
// the workgroup must call it.
__device__ __forceinline__ void request_outputs(const CompileParams& p, const ReqRun& run, const CompileLds& L, int N) {
    const int R = p.num_reqs;
    const int MR = p.max_num_reqs;
    const int tid = threadIdx.x;
    int sc[2] = {run.kept, run.local_seq}, mx[2] = {run.max_q, run.max_seq}, tot[2];
    block_scan2_max2<kCompileThreads>(sc, mx, L.red, tot);
    int slot_out = sc[0], seq_run = sc[1];
    const int num_sampled = tot[0], seq_total = tot[1];
    for (int i = run.r0; i < run.r1; ++i) {
        const int end = L.qsl[i + 1];
        const int li = end - 1;
        const int seq = L.base[i] + end;   // c_i + q_i
        const bool part = ((run.partial >> (i - run.r0)) & 1u) != 0;
        p.seq_lens[i] = seq;
        p.cu_seqlens_k[i] = seq_run;
        seq_run += seq;
        p.logits_indices[i] = li;
        p.discard[i] = part ? 1 : 0;
        if (!part) p.sample_indices[slot_out++] = li;
    }
    for (int i = tid; i <= MR; i += kCompileThreads) {
        p.query_start_loc[i] = (i <= R) ? L.qsl[i] : N;
        if (i >= R) p.cu_seqlens_k[i] = seq_total;
        if (i >= R && i < MR) {
            p.seq_lens[i] = 0;
            p.logits_indices[i] = -1;
            p.discard[i] = 1;
        }
        if (i >= num_sampled && i < MR) p.sample_indices[i] = -1;
    }
    if (tid == 0) {
        p.dev_scalars[0] = R;
        p.dev_scalars[1] = N;
        p.dev_scalars[2] = p.n_pad;
        p.dev_scalars[3] = mx[0];
        p.dev_scalars[4] = mx[1];
        p.dev_scalars[5] = num_sampled;
    }
}

__global__ __launch_bounds__(kCompileThreads) void compile_kernel(CompileParams p) {
    extern __shared__ int32_t smem[];
    const CompileLds L(smem, p.num_reqs);
    const bool req_wg = (int)blockIdx.x >= p.num_token_tiles;
    ReqRun run;
    const int N = scan_requests(p, L, req_wg, run);
    if (!req_wg) {
        const int tile0 = blockIdx.x * kCompileTile;
#pragma unroll
        for (int k = 0; k < kCompileTokensPerThread; ++k) {
            const int t = tile0 + k * kCompileThreads + threadIdx.x;
            if (t >= p.n_pad) break;
            token_outputs(p, L, N, t, true);
        }
        return;
    }
    request_outputs(p, run, L, N);
}

static size_t compile_lds_bytes(int num_reqs, int extra_words) {
    return sizeof(int32_t) * (2 * (size_t)num_reqs + 1 + CompileLds::extra_words + extra_words);
}

hipError_t launch_compile(const CompileParams& p, hipStream_t s) {
    hipLaunchKernelGGL(compile_kernel, dim3(p.num_token_tiles + 1), dim3(kCompileThreads),
                       compile_lds_bytes(p.num_reqs, 0), s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Paged K/V write: row t of every K and V source goes to cache row slot[t]
// ([P1 §3. 物理 KV 槽位]; [P3 §实现]).  Two launch shapes, chosen by size from
// measured sweeps on MI355X:
//
// * wave rows (up to 8192 tokens of 1, 2 or 4 KiB): blockIdx.y = layer; each
//   wave owns ROWS consecutive tokens and copies both the K and the V row of
//   each, so one wave-uniform (scalar) slot load serves both; 4*ROWS*CPL
//   16-byte loads per lane are in flight before any store.
// * chunk tiles (larger launches, other row sizes): blockIdx.y = 2*layer +
//   (K:0, V:1), blockIdx.x = a run of rows of about 4 KiB; lanes walk the
//   run's 16-byte chunks in order, so a source run is read contiguously and
//   each cache row is written contiguously.  More bytes in flight per lane
//   (2-4 loads before the stores, bigger tiles, a persistent grid) measured
//   slower.
//
// Both use non-temporal loads and stores: every byte is touched once, and
// streaming accesses measured as fast or faster than plain ones in nearly
// every pattern, with the sources in HBM or still in the caches.
//
// A slot outside [0, num_slots) skips that row and counts it in *status.
// ---------------------------------------------------------------------------
template <bool NT>
__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void store16(uint8_t* p, u32x4 v) {
    if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
    else *reinterpret_cast<u32x4*>(p) = v;
}

template <int U, bool NTL, bool NTS>
__global__ __launch_bounds__(256) void kv_chunk_kernel(KVParams p) {
    const int tensor = blockIdx.y;
    const int layer = tensor >> 1;
    const bool is_v = (tensor & 1) != 0;
    const uint8_t* __restrict__ src = is_v ? p.v[layer] : p.k[layer];
    uint8_t* __restrict__ dst = is_v ? p.vc[layer] : p.kc[layer];
    const int t0 = blockIdx.x * p.rows_per_wg;
    const int rows = min(p.rows_per_wg, p.num_tokens - t0);
    const int C = p.row_bytes >> 4;
    const int total = rows * C;
    for (int base = threadIdx.x; base < total; base += 256 * U) {
        u32x4 val[U];
        int64_t doff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = base + u * 256;
            doff[u] = -1;
            if (i < total) {
                const int r = (p.chunk_shift >= 0) ? (i >> p.chunk_shift) : (i / C);
                const int j = i - r * C;
                const int t = t0 + r;
                const int s = p.slot[t];
                val[u] = load16<NTL>(src + (int64_t)t * p.src_stride + ((int64_t)j << 4));
                if (s >= 0 && (int64_t)s < p.num_slots)
                    doff[u] = (int64_t)s * p.row_bytes + ((int64_t)j << 4);
                else if (j == 0 && p.status != nullptr)
                    atomicAdd(p.status, 1);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (doff[u] >= 0) store16<NTS>(dst + doff[u], val[u]);
    }
}

// CPL: 16-byte chunks per lane per row (row_bytes = 1024 * CPL).
template <int CPL, int ROWS, int WAVES, bool NTL, bool NTS>
__global__ __launch_bounds__(64 * WAVES) void kv_wave_kernel(KVParams p) {
    const int layer = blockIdx.y;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int t0 = (blockIdx.x * WAVES + wid) * ROWS;
    const uint8_t* __restrict__ ks = p.k[layer];
    const uint8_t* __restrict__ vs = p.v[layer];
    uint8_t* __restrict__ kd = p.kc[layer];
    uint8_t* __restrict__ vd = p.vc[layer];
    u32x4 a[ROWS][2 * CPL];
    int64_t off[ROWS];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int t = t0 + r;
        off[r] = -1;
        if (t < p.num_tokens) {
            const int s = p.slot[t];
            const int64_t so = (int64_t)t * p.src_stride + lane * 16;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                a[r][c] = load16<NTL>(ks + so + c * 1024);
                a[r][CPL + c] = load16<NTL>(vs + so + c * 1024);
            }
            if (s >= 0 && (int64_t)s < p.num_slots)
                off[r] = (int64_t)s * p.row_bytes + lane * 16;
            else if (lane == 0 && p.status != nullptr)
                atomicAdd(p.status, 2);
        }
    }
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        if (off[r] >= 0) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                store16<NTS>(kd + off[r] + c * 1024, a[r][c]);
                store16<NTS>(vd + off[r] + c * 1024, a[r][CPL + c]);
            }
        }
    }
}

constexpr int kKvTileBytes = 4096;        // chunk tiles: about 4 KiB per workgroup
constexpr int kKvWaveMaxTokens = 8192;    // wave rows up to this many tokens per launch
constexpr int kKvWaveRows = 4;
constexpr int kKvWaveWaves = 4;

template <int CPL>
static void launch_wave(const KVParams& p, int num_layers, hipStream_t s) {
    const int per_wg = kKvWaveRows * kKvWaveWaves;
    hipLaunchKernelGGL((kv_wave_kernel<CPL, kKvWaveRows, kKvWaveWaves, true, true>),
                       dim3((p.num_tokens + per_wg - 1) / per_wg, num_layers), dim3(64 * kKvWaveWaves), 0, s, p);
}

hipError_t launch_kv_scatter(const KVParams& p_in, int num_layers, hipStream_t s) {
    KVParams p = p_in;
    if (p.num_tokens == 0 || num_layers == 0) return hipSuccess;
    const int cpl = p.row_bytes / 1024;
    const bool wave_ok = p.row_bytes % 1024 == 0 && (cpl == 1 || cpl == 2 || cpl == 4);
    if (wave_ok && p.num_tokens <= kKvWaveMaxTokens) {
        if (cpl == 1) launch_wave<1>(p, num_layers, s);
        else if (cpl == 2) launch_wave<2>(p, num_layers, s);
        else launch_wave<4>(p, num_layers, s);
        return hipGetLastError();
    }
    p.rows_per_wg = p.rows_per_wg > 0 ? p.rows_per_wg : max(1, kKvTileBytes / p.row_bytes);
    const int gx = (p.num_tokens + p.rows_per_wg - 1) / p.rows_per_wg;
    hipLaunchKernelGGL((kv_chunk_kernel<1, true, true>), dim3(gx, 2 * num_layers), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compile and K/V write in one launch.  blockIdx.y = layer; workgroup x <
// num_token_tiles owns TT = ROWS * 4 consecutive tokens, the last one (layer 0
// only) writes the per-request outputs.  Each token workgroup issues the
// loads of the first PRE rows of each wave's K and V rows of its layer (they
// do not depend on the compile; with at most 256 requests the request
// counters are loaded just before them), rebuilds query_start_loc in LDS like the
// compile kernel, derives its tokens' slots (layer-0 workgroups also write the
// per-token outputs), loads the remaining rows and stores them all, wave by
// wave as the wave kernel does.  This saves the second launch and the drain
// between two kernels, and the first rows' loads overlap the slot work.  A
// slot outside [0, num_slots) skips its row and counts in *status, as in the
// K/V kernels.
// ---------------------------------------------------------------------------
// Steps of at most kCompileThreads requests: thread i's own request's q and c,
// which a token workgroup of the single compile + K/V kernel loads before its
// K/V rows, so that these loads are not queued behind the rows.
struct OwnCounters {
    int q, c;
};

__device__ __forceinline__ OwnCounters load_own_counters(const CompileParams& p) {
    OwnCounters oc{0, 0};
    const int i = threadIdx.x;
    if (i < p.num_reqs) {
        oc.q = p.scal[(int64_t)kNumScheduled * p.max_num_reqs + i];
        oc.c = p.scal[(int64_t)kNumComputed * p.max_num_reqs + i];
    }
    return oc;
}

// scan_requests for a token workgroup whose counters were loaded by
// load_own_counters.  Contains barriers: every thread must call it.
__device__ __forceinline__ int scan_own_counters(const CompileParams& p, const CompileLds& L, OwnCounters oc) {
    const int i = threadIdx.x;
    const int R = p.num_reqs;
    int N = 0;
    const int off = block_exclusive_scan<kCompileThreads>(i < R ? oc.q : 0, L.tmp, &N);
    if (i < R) {
        L.qsl[i] = off;
        L.base[i] = oc.c - off;
    }
    if (i == 0) L.qsl[R] = N;
    __syncthreads();
    return N;
}

template <int CPL, int ROWS, int PRE, int SUB>
__global__ __launch_bounds__(kCompileThreads) void compile_kv_kernel(CompileParams p, KVParams kv) {
    static_assert(PRE >= 0 && PRE <= ROWS, "rows loaded early must be rows of the wave");
    static_assert(SUB == 1 || CPL == 1, "rows narrower than 1 KiB take one 16-byte chunk per lane");
    constexpr int WAVES = kCompileThreads / kWave;
    constexpr int LPR = kWave / SUB;           // lanes per row: SUB rows share one wave load
    constexpr int TW = ROWS * SUB;             // tokens per wave
    constexpr int TT = TW * WAVES;
    extern __shared__ int32_t smem[];
    const CompileLds L(smem, p.num_reqs);
    int32_t* s_slot = smem + 2 * p.num_reqs + 1 + CompileLds::extra_words;   // [TT]
    const int layer = blockIdx.y;
    const bool req_wg = (int)blockIdx.x >= p.num_token_tiles;
    if (req_wg && layer != 0) return;          // whole workgroup: before any barrier
    const int lane = threadIdx.x & (kWave - 1);
    const int sub = lane / LPR;                // this lane's row within a wave load
    const int64_t lane_off = (int64_t)(lane % LPR) * 16;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tile0 = blockIdx.x * TT;
    const int t0 = tile0 + wid * TW;           // this wave's first token
    const uint8_t* __restrict__ ks = kv.k[layer];
    const uint8_t* __restrict__ vs = kv.v[layer];
    u32x4 a[ROWS][2 * CPL];
    auto load_row = [&](int r) {
        const int t = t0 + r * SUB + sub;
        if (t < p.n_pad) {
            const int64_t so = (int64_t)t * kv.src_stride + lane_off;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                a[r][c] = load16<true>(ks + so + c * 1024);
                a[r][CPL + c] = load16<true>(vs + so + c * 1024);
            }
        }
    };
    // up to kCompileThreads requests, each thread's counters go out before the rows
    const bool own = !req_wg && p.num_reqs <= kCompileThreads;
    OwnCounters oc{0, 0};
    if (own) oc = load_own_counters(p);
    if (!req_wg) {
#pragma unroll
        for (int r = 0; r < PRE; ++r) load_row(r);
    }
    ReqRun run;
    const int N = own ? scan_own_counters(p, L, oc) : scan_requests(p, L, req_wg, run);
    if (req_wg) {
        request_outputs(p, run, L, N);
        return;
    }
    if ((int)threadIdx.x < TT) {
        const int t = tile0 + threadIdx.x;
        if (t < p.n_pad) s_slot[threadIdx.x] = token_outputs(p, L, N, t, layer == 0);
    }
    __syncthreads();
#pragma unroll
    for (int r = PRE; r < ROWS; ++r) load_row(r);
    uint8_t* __restrict__ kd = kv.kc[layer];
    uint8_t* __restrict__ vd = kv.vc[layer];
#pragma unroll
    for (int r = 0; r < ROWS; ++r) {
        const int t = t0 + r * SUB + sub;
        if (t >= p.n_pad) continue;
        const int s = s_slot[wid * TW + r * SUB + sub];
        if (s >= 0 && (int64_t)s < kv.num_slots) {
            const int64_t off = (int64_t)s * kv.row_bytes + lane_off;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                store16<true>(kd + off + c * 1024, a[r][c]);
                store16<true>(vd + off + c * 1024, a[r][CPL + c]);
            }
        } else if (lane % LPR == 0 && kv.status != nullptr) {
            atomicAdd(kv.status, 2);
        }
    }
}

bool fused_kv_supported(int row_bytes) {
    switch (row_bytes) {
    case 128: case 256: case 512: case 1024: case 2048: case 3072: case 4096: case 6144: case 8192: return true;
    default: return false;
    }
}

// Tile shape.  Rows of 1 KiB or more, from sweeps on MI355X over 1/2/4/8 rows
// per wave, rows loaded before or after the prefix sum, other tile orders and
// a persistent grid: steps of long per-request runs (few requests: a short prefix sum) take two
// rows per wave and load only the first before the prefix sum: loading every
// row up front puts more reads in flight than some machines serve well
// (long-context, calls back to back: 48 us against 52 us all-first, and 50 us
// for the compile and the K/V kernel as two launches; after other kernels the
// shape takes 55-57 us, so the library's own choice gives such steps two
// launches and this shape runs only when asked for).  Other steps load every
// row first, so the longer prefix sum over many requests hides behind them
// (with at most 256 requests the counters are loaded just before those
// rows), with two rows per wave when that still gives at least 2048 token
// workgroups over the layers (eight per compute unit) and one otherwise
// (decode-heavy: 13.2 us with one row per wave, 16.5 with four).
template <int CPL, int SUB>
static void launch_fused(const CompileParams& p_in, const KVParams& kv, int num_layers, bool long_runs,
                         hipStream_t s) {
    CompileParams p = p_in;
    constexpr int WAVES = kCompileThreads / kWave;
    int rows, pre;
    if (SUB > 1) {
        // Rows narrower than 1 KiB: a workgroup moves few bytes per token, so
        // its prefix sum weighs more; every row is loaded first, two rows per
        // wave, four above 256 requests (churn's 1024: 15.3 against 16.4 us
        // with two, 512 B rows), long runs included.
        rows = p.num_reqs > kCompileThreads ? 4 : 2;
        pre = rows;
    } else {
        const bool two = long_runs || (int64_t)((p.n_pad + 2 * WAVES - 1) / (2 * WAVES)) * num_layers >= 2048;
        rows = two ? 2 : 1;
        pre = long_runs ? 1 : rows;
    }
    const int TT = rows * SUB * WAVES;
    p.num_token_tiles = (p.n_pad + TT - 1) / TT;
    const dim3 grid(p.num_token_tiles + 1, num_layers);
    const size_t lds = compile_lds_bytes(p.num_reqs, TT);
    const dim3 block(kCompileThreads);
    if constexpr (SUB > 1) {
        if (rows == 4) hipLaunchKernelGGL((compile_kv_kernel<CPL, 4, 4, SUB>), grid, block, lds, s, p, kv);
        else hipLaunchKernelGGL((compile_kv_kernel<CPL, 2, 2, SUB>), grid, block, lds, s, p, kv);
    } else {
        if (pre == 1 && rows == 2) hipLaunchKernelGGL((compile_kv_kernel<CPL, 2, 1, 1>), grid, block, lds, s, p, kv);
        else if (rows == 2) hipLaunchKernelGGL((compile_kv_kernel<CPL, 2, 2, 1>), grid, block, lds, s, p, kv);
        else hipLaunchKernelGGL((compile_kv_kernel<CPL, 1, 1, 1>), grid, block, lds, s, p, kv);
    }
}

hipError_t launch_compile_kv(const CompileParams& p, const KVParams& kv, int num_layers, bool long_runs,
                             hipStream_t s) {
    if (num_layers < 1 || !fused_kv_supported(kv.row_bytes)) return hipErrorInvalidValue;
    switch (kv.row_bytes) {
    case 128: launch_fused<1, 8>(p, kv, num_layers, long_runs, s); break;
    case 256: launch_fused<1, 4>(p, kv, num_layers, long_runs, s); break;
    case 512: launch_fused<1, 2>(p, kv, num_layers, long_runs, s); break;
    case 1024: launch_fused<1, 1>(p, kv, num_layers, long_runs, s); break;
    case 2048: launch_fused<2, 1>(p, kv, num_layers, long_runs, s); break;
    case 3072: launch_fused<3, 1>(p, kv, num_layers, long_runs, s); break;
    case 4096: launch_fused<4, 1>(p, kv, num_layers, long_runs, s); break;
    case 6144: launch_fused<6, 1>(p, kv, num_layers, long_runs, s); break;
    default: launch_fused<8, 1>(p, kv, num_layers, long_runs, s); break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row gather: dst[m] = src[idx[m]] for m < count (hidden states at the logits
// rows; [P1 §第四步]).  One workgroup per output row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_kernel(GatherParams p) {
    const int m = blockIdx.x;
    int count = p.max_rows;
    if (p.dev_count != nullptr) count = min(count, *p.dev_count);
    if (m >= count) return;
    int64_t id = p.idx[m];
    if (id >= p.src_rows) {
        if (threadIdx.x == 0 && p.status != nullptr) atomicAdd(p.status, 1);
        id = -1;
    }
    const int C = p.row_bytes >> 4;
    u32x4* out = reinterpret_cast<u32x4*>(p.dst + (int64_t)m * p.dst_stride);
    if (id < 0) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        for (int j = threadIdx.x; j < C; j += 256) out[j] = z;
        return;
    }
    const u32x4* in = reinterpret_cast<const u32x4*>(p.src + id * p.src_stride);
    constexpr int U = 4;   // loads in flight per lane before the stores
    for (int base = threadIdx.x; base < C; base += 256 * U) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * 256 < C) v[u] = __builtin_nontemporal_load(in + base + u * 256);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (base + u * 256 < C) out[base + u * 256] = v[u];
    }
}

hipError_t launch_gather(const GatherParams& p, hipStream_t s) {
    if (p.max_rows == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_kernel, dim3(p.max_rows), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Condense: move every column of source row -> destination hole for each
// pair ([P1 §行号是一种短生命周期地址]).  Holes and sources are disjoint sets,
// so all pairs move at once.  blockIdx.y = pair, blockIdx.x = chunk of the
// token history; chunk 0 also moves the block row and the scalar columns.
// Row strides are multiples of 4 words, so rows copy in 16-byte units (words
// past the valid prefix are stale in both rows).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void move_rows_kernel(MoveParams p) {
    const int pair = blockIdx.y;
    const int dst_row = p.pairs[2 * pair];
    const int src_row = p.pairs[2 * pair + 1];
    const int T = p.scal[(int64_t)kNumTokens * p.max_num_reqs + src_row];
    const int nvec = min((T + 3) >> 2, (int)(p.tok_stride >> 2));
    const int v0 = blockIdx.x * p.chunk_vec4;
    const int v1 = min(nvec, v0 + p.chunk_vec4);
    const u32x4* ts = reinterpret_cast<const u32x4*>(p.tokens + (int64_t)src_row * p.tok_stride);
    u32x4* td = reinterpret_cast<u32x4*>(p.tokens + (int64_t)dst_row * p.tok_stride);
    for (int v = v0 + threadIdx.x; v < v1; v += 256) td[v] = ts[v];
    if (blockIdx.x == 0) {
        for (int g = 0; g < p.num_groups; ++g) {
            const int nb = min(p.scal[(int64_t)blocks_col(g) * p.max_num_reqs + src_row], (int)p.blk_stride[g]);
            const u32x4* bs = reinterpret_cast<const u32x4*>(p.blocks[g] + (int64_t)src_row * p.blk_stride[g]);
            u32x4* bd = reinterpret_cast<u32x4*>(p.blocks[g] + (int64_t)dst_row * p.blk_stride[g]);
            for (int v = threadIdx.x; v < ((nb + 3) >> 2); v += 256) bd[v] = bs[v];
        }
        if (threadIdx.x < kNumScalarCols) {
            const int64_t col = (int64_t)threadIdx.x * p.max_num_reqs;
            p.scal[col + dst_row] = p.scal[col + src_row];
        }
    }
}

hipError_t launch_move_rows(const MoveParams& p, int max_token_chunks, hipStream_t s) {
    if (p.num_pairs == 0) return hipSuccess;
    hipLaunchKernelGGL(move_rows_kernel, dim3(max_token_chunks > 0 ? max_token_chunks : 1, p.num_pairs),
                       dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Staged deltas: one workgroup per op copies its words from the flush's log
// (pinned host memory read in place, or its copy in device staging) to the
// column store.  Ops of one flush never overlap.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void apply_deltas_kernel(const uint32_t* payload, const DeltaOp* ops) {
    const DeltaOp op = ops[blockIdx.x];
    uint32_t* dst = reinterpret_cast<uint32_t*>(op.dst);
    const uint32_t* src = payload + op.src_word;
    // eight loads in flight per lane: the payload may be read from pinned host
    // memory, where each pass costs a round trip over the host link
    constexpr uint32_t U = 8;
    for (uint32_t base = threadIdx.x; base < op.n_words; base += 256 * U) {
        uint32_t v[U];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u)
            if (base + u * 256 < op.n_words) v[u] = src[base + u * 256];
#pragma unroll
        for (uint32_t u = 0; u < U; ++u)
            if (base + u * 256 < op.n_words) dst[base + u * 256] = v[u];
    }
}

hipError_t launch_apply_deltas(const uint32_t* payload, const DeltaOp* ops, int n_ops, hipStream_t s) {
    if (n_ops == 0) return hipSuccess;
    hipLaunchKernelGGL(apply_deltas_kernel, dim3(n_ops), dim3(256), 0, s, payload, ops);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Speculative decoding: a request verifying d drafts needs logits at its last
// d + 1 flat positions; the first d of those rows check the drafts (target),
// the last one gives the bonus token; the drafts are its last d input ids
// ([P1 §投机解码：一条请求一轮可能产生多个决策位置]).  Every workgroup rebuilds
// the prefix sum of (d + 1) in LDS; workgroups 0..num_tiles-1 each own 256
// logits rows; the last workgroup writes cu_num_logits and the bonus rows.
// Draft offsets need no second scan: sum_{j<i} d_j = cu[i] - i.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void spec_decode_kernel(SpecParams p) {
    extern __shared__ int32_t smem[];
    const int R = p.num_reqs;
    int32_t* s_cu = smem;                 // [R + 1]
    int32_t* s_tmp = smem + R + 1;        // [4]
    const int tid = threadIdx.x;
    const int per = (R + 255) / 256;
    const int r0 = min(R, tid * per);
    const int r1 = min(R, r0 + per);
    int local = 0;
    for (int i = r0; i < r1; ++i) {
        const int n = p.num_draft[i] + 1;
        s_cu[i] = n;
        local += n;
    }
    int total = 0;
    int run = block_exclusive_scan<256>(local, s_tmp, &total);
    for (int i = r0; i < r1; ++i) {
        const int n = s_cu[i];
        s_cu[i] = run;
        run += n;
    }
    if (tid == 0) s_cu[R] = total;
    __syncthreads();

    if ((int)blockIdx.x < p.num_tiles) {
        const int m = blockIdx.x * 256 + tid;
        if (m >= p.num_logits) return;
        int lo = 0, hi = R - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_cu[mid] <= m) lo = mid; else hi = mid - 1;
        }
        const int r = lo;
        const int d = s_cu[r + 1] - s_cu[r] - 1;
        const int k = m - s_cu[r];
        const int end = p.qsl[r + 1];
        p.logits_indices[m] = end - (d + 1) + k;
        if (k < d) {
            const int j = s_cu[r] - r + k;
            p.target[j] = m;
            p.draft_ids[j] = p.input_ids[end - d + k];
        }
        return;
    }
    for (int i = tid; i <= R; i += 256) {
        p.cu_num_logits[i] = s_cu[i];
        if (i < R) p.bonus[i] = s_cu[i + 1] - 1;
    }
}

hipError_t launch_spec_decode(const SpecParams& p, hipStream_t s) {
    const size_t lds = sizeof(int32_t) * ((size_t)p.num_reqs + 1 + 4);
    hipLaunchKernelGGL(spec_decode_kernel, dim3(p.num_tiles + 1), dim3(256), lds, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block table cut or padded to a fixed width for an attention call that wants
// a dense [rows][width] table: entries past a row's own blocks get `fill`
// (nano-vllm pads with -1 to the longest row).  blockIdx.y = row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void padded_table_kernel(PaddedTableParams p) {
    const int r = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= p.width) return;
    const int nb = (int)min((int64_t)p.num_blocks[r], p.blk_stride);   // the stride fits an int
    // ratio > 1: each stored (manager) block id m stands for kernel blocks
    // m*ratio .. m*ratio + ratio-1 ([P1 §混合 KV Cache], map_to_kernel_blocks)
    const int b = j / p.ratio;
    p.dst[(int64_t)r * p.width + j] =
        (b < nb) ? p.blocks[(int64_t)r * p.blk_stride + b] * p.ratio + (j - b * p.ratio) : p.fill;
}

hipError_t launch_padded_table(const PaddedTableParams& p, hipStream_t s) {
    if (p.rows == 0 || p.width == 0) return hipSuccess;
    hipLaunchKernelGGL(padded_table_kernel, dim3((p.width + 255) / 256, p.rows), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Sampled tokens appended on the device: token table element dst_off[k]
// receives src[src_idx[k]] (last step's sampled ids stay on the GPU and are
// placed through a current-row -> sample-position map, [P1 §先拷 block table，
// 再做 CPU 索引]).  An index outside [0, src_len) writes nothing and bumps *err.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void append_sampled_kernel(int32_t* tokens, const int64_t* dst_off,
                                                             const int32_t* src_idx, const int32_t* src,
                                                             int32_t src_len, int32_t n, int32_t* err) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= n) return;
    const int i = src_idx[k];
    if (i < 0 || i >= src_len) {
        atomicAdd(err, 1);
        return;
    }
    tokens[dst_off[k]] = src[i];
}

hipError_t launch_append_sampled(int32_t* tokens, const int64_t* dst_off, const int32_t* src_idx,
                                 const int32_t* src, int32_t src_len, int32_t n, int32_t* err, hipStream_t s) {
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(append_sampled_kernel, dim3((n + 255) / 256), dim3(256), 0, s, tokens, dst_off, src_idx,
                       src, src_len, n, err);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Correction of optimistically advanced computed counts (asynchronous
// speculative decoding, [P1 §投机解码：一条请求一轮可能产生多个决策位置]).  Row
// rows[k] was scheduled as if all draft[k] drafts it verified last step were
// accepted; the sampler kept v = accepted[prev[k]] tokens, so its count drops
// by draft[k] + 1 - v, on the device, before the compile reads it.  With
// sampled tokens given, the last kept one becomes the row's token at the
// corrected count (its first input of this step).  A v outside
// [1, draft + 1], or a corrected count outside the row, changes nothing and
// bumps *status.  One thread per row; rows are distinct (checked on the host).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void correct_computed_kernel(CorrectParams p) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= p.n) return;
    const int row = p.rows[k];
    const int pos = p.prev[k];
    const int d = p.draft[k];
    const int v = p.accepted[pos];
    const int c = p.computed[row] - (d + 1 - v);
    if (v < 1 || v > d + 1 || c < 0 || c >= p.tok_stride) {
        if (p.status) atomicAdd(p.status, 1);
        return;
    }
    p.computed[row] = c;
    if (p.sampled) p.tokens[(int64_t)row * p.tok_stride + c] = p.sampled[(int64_t)pos * p.sampled_stride + v - 1];
}

hipError_t launch_correct_computed(const CorrectParams& p, hipStream_t s) {
    if (p.n == 0) return hipSuccess;
    hipLaunchKernelGGL(correct_computed_kernel, dim3((p.n + 255) / 256), dim3(256), 0, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Slot-collision check: every real token must own its cache slot, since two
// tokens writing one slot leave a result that depends on the order of the
// writes (each block has a single owner, [P1 §八条必须成立的不变量], item 7).  A bitmap of
// ceil(num_slots / 32) words is cleared, then each token sets its slot's bit;
// a token that finds the bit already set counts one collision.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* words, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) words[i] = 0u;
}

__global__ __launch_bounds__(256) void mark_slots_kernel(const int32_t* slot, int32_t n, const int32_t* dev_n,
                                                         int64_t num_slots, uint32_t* bits, int32_t* result) {
    int count = n;
    if (dev_n != nullptr) count = min(count, max(0, *dev_n));
    for (int t = blockIdx.x * 256 + threadIdx.x; t < count; t += gridDim.x * 256) {
        const int s = slot[t];
        if (s < 0 || (int64_t)s >= num_slots) {
            atomicAdd(result + 1, 1);
            continue;
        }
        const uint32_t m = 1u << (s & 31);
        if (atomicOr(bits + (s >> 5), m) & m) atomicAdd(result, 1);
    }
}

// Bitmap of the allocation-free variant: one copy per GPU, held until the
// process ends.  Host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device (the array's name is a
// host-side stand-in there, not a device address).
static __device__ __align__(256) uint32_t scratch[kCheckScratchWords];

hipError_t check_scratch_for_current_device(uint32_t** out) {
    static std::mutex mu;
    static uint32_t* ptr_of[kMaxScratchDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr_of[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        ptr_of[dev] = static_cast<uint32_t*>(ptr);
    }
    *out = ptr_of[dev];
    return hipSuccess;
}

hipError_t launch_check_slots(const int32_t* slot, int32_t n, const int32_t* dev_n, int64_t num_slots,
                              uint32_t* bits, int32_t* result, hipStream_t s) {
    const int64_t words = (num_slots + 31) / 32;
    const int gc = (int)std::min<int64_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(clear_words_kernel, dim3(gc), dim3(256), 0, s, bits, words);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n == 0) return e;
    const int gm = std::min((n + 255) / 256, 4096);
    hipLaunchKernelGGL(mark_slots_kernel, dim3(gm), dim3(256), 0, s, slot, n, dev_n, num_slots, bits, result);
    return hipGetLastError();
}

}  // namespace ric
