// Test double for the device, so that the library's host control plane
// (ric_host.cpp: row maps, validation, the pinned delta log, flushes, condense
// bookkeeping) can run on a machine without a GPU, built with AddressSanitizer
// and UndefinedBehaviorSanitizer.  Linked only into a test library; the
// product library never contains it.
//
// "Device" memory is host memory.  The HIP calls the control plane makes are
// replaced by host equivalents (allocation, copies, no-op events and
// synchronisation).  Of the kernel launchers, only those that maintain the
// column store do their work here (staged-delta apply, condense row move,
// sampled-token append, computed-count correction), so the column store can
// be compared with the reference batch; the step kernels (compile, K/V write,
// gather, spec decode, padded tables) are parity-tested on the GPU and do
// nothing here.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <vector>

#include "../../ragged_input_compilation_amd/csrc/ric_internal.h"

namespace {
void* aligned(size_t n) {
    void* p = nullptr;
    if (posix_memalign(&p, 256, n ? n : 1) != 0) return nullptr;
    std::memset(p, 0xCD, n);      // never-written bytes are recognisable, like uninitialised device memory
    return p;
}
int g_device = 0;
}  // namespace

extern "C" {
hipError_t hipMalloc(void** ptr, size_t size) {
    *ptr = aligned(size);
    return *ptr ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* ptr) {
    std::free(ptr);
    return hipSuccess;
}
hipError_t hipHostMalloc(void** ptr, size_t size, unsigned int) { return hipMalloc(ptr, size); }
hipError_t hipHostFree(void* ptr) { return hipFree(ptr); }
hipError_t hipHostGetDevicePointer(void** dptr, void* hptr, unsigned int) {
    *dptr = hptr;
    return hipSuccess;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
    std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t) {
    std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned) {
    *event = reinterpret_cast<hipEvent_t>(new int(0));
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventDestroy(hipEvent_t event) {
    delete reinterpret_cast<int*>(event);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipGetDevice(int* device) {
    *device = g_device;
    return hipSuccess;
}
hipError_t hipSetDevice(int device) {
    g_device = device;
    return hipSuccess;
}
const char* hipGetErrorString(hipError_t) { return "fake device"; }
// Stream capture is simulated: the test switches it on and off.
int g_capturing = 0;
void fake_set_capturing(int on) { g_capturing = on; }
hipError_t hipStreamIsCapturing(hipStream_t, hipStreamCaptureStatus* status) {
    *status = g_capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}
}

namespace ric {

hipError_t launch_apply_deltas(const uint32_t* payload, const DeltaOp* ops, int n_ops, hipStream_t) {
    // The device applies the ops of one flush in parallel, so no two may
    // write the same bytes: a flush that breaks this aborts the test.
    std::vector<std::pair<uint64_t, uint64_t>> spans;
    for (int i = 0; i < n_ops; ++i)
        if (ops[i].n_words) spans.emplace_back(ops[i].dst, ops[i].dst + 4 * (uint64_t)ops[i].n_words);
    std::sort(spans.begin(), spans.end());
    for (size_t i = 1; i < spans.size(); ++i)
        if (spans[i].first < spans[i - 1].second) {
            std::fprintf(stderr, "fake device: two staged writes of one flush overlap\n");
            std::abort();
        }
    for (int i = 0; i < n_ops; ++i)
        std::memcpy(reinterpret_cast<void*>(ops[i].dst), payload + ops[i].src_word, 4 * (size_t)ops[i].n_words);
    return hipSuccess;
}

hipError_t launch_move_rows(const MoveParams& p, int, hipStream_t) {
    for (int k = 0; k < p.num_pairs; ++k) {
        const int dst = p.pairs[2 * k], src = p.pairs[2 * k + 1];
        const int T = p.scal[(int64_t)kNumTokens * p.max_num_reqs + src];
        const int64_t nwords = std::min<int64_t>(((int64_t)T + 3) / 4 * 4, p.tok_stride);
        std::memcpy(p.tokens + (int64_t)dst * p.tok_stride, p.tokens + (int64_t)src * p.tok_stride, 4 * nwords);
        for (int g = 0; g < p.num_groups; ++g) {
            const int64_t nb = std::min<int64_t>(p.scal[(int64_t)blocks_col(g) * p.max_num_reqs + src], p.blk_stride[g]);
            std::memcpy(p.blocks[g] + (int64_t)dst * p.blk_stride[g], p.blocks[g] + (int64_t)src * p.blk_stride[g],
                        4 * (size_t)((nb + 3) / 4 * 4));
        }
        for (int c = 0; c < kNumScalarCols; ++c)
            p.scal[(int64_t)c * p.max_num_reqs + dst] = p.scal[(int64_t)c * p.max_num_reqs + src];
    }
    return hipSuccess;
}

hipError_t launch_append_sampled(int32_t* tokens, const int64_t* dst_off, const int32_t* src_idx, const int32_t* src,
                                 int32_t src_len, int32_t n, int32_t* err, hipStream_t) {
    for (int k = 0; k < n; ++k) {
        if (src_idx[k] < 0 || src_idx[k] >= src_len) {
            ++*err;
            continue;
        }
        tokens[dst_off[k]] = src[src_idx[k]];
    }
    return hipSuccess;
}

hipError_t launch_correct_computed(const CorrectParams& p, hipStream_t) {
    for (int k = 0; k < p.n; ++k) {
        const int row = p.rows[k], pos = p.prev[k], d = p.draft[k];
        const int v = p.accepted[pos];
        const int c = p.computed[row] - (d + 1 - v);
        if (v < 1 || v > d + 1 || c < 0 || c >= p.tok_stride) {
            if (p.status) ++*p.status;
            continue;
        }
        p.computed[row] = c;
        if (p.sampled) p.tokens[(int64_t)row * p.tok_stride + c] = p.sampled[(int64_t)pos * p.sampled_stride + v - 1];
    }
    return hipSuccess;
}

hipError_t launch_check_slots(const int32_t* slot, int32_t n, const int32_t* dev_n, int64_t num_slots,
                              uint32_t* bits, int32_t* result, hipStream_t) {
    std::memset(bits, 0, (size_t)((num_slots + 31) / 32) * 4);
    const int count = dev_n ? std::min(n, std::max(0, *dev_n)) : n;
    for (int t = 0; t < count; ++t) {
        const int s = slot[t];
        if (s < 0 || s >= num_slots) {
            ++result[1];
            continue;
        }
        const uint32_t m = 1u << (s & 31);
        if (bits[s >> 5] & m) ++result[0];
        bits[s >> 5] |= m;
    }
    return hipSuccess;
}

hipError_t check_scratch_for_current_device(uint32_t** out) {
    static std::vector<uint32_t> scratch_words((size_t)kCheckScratchWords);
    *out = scratch_words.data();
    return hipSuccess;
}

hipError_t launch_compile(const CompileParams&, hipStream_t) { return hipSuccess; }
bool fused_kv_supported(int row_bytes) {
    switch (row_bytes) {
    case 128: case 256: case 512: case 1024: case 2048: case 3072: case 4096: case 6144: case 8192: return true;
    default: return false;
    }
}
hipError_t launch_compile_kv(const CompileParams&, const KVParams&, int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_kv_scatter(const KVParams&, int, hipStream_t) { return hipSuccess; }
hipError_t launch_gather(const GatherParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_padded_table(const PaddedTableParams&, hipStream_t) { return hipSuccess; }
hipError_t launch_spec_decode(const SpecParams&, hipStream_t) { return hipSuccess; }

}  // namespace ric
