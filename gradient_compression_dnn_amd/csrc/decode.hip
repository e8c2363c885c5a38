// Decompress-and-aggregate K sparse messages into a dense update.
// "Deep Gradient Compression" (Lin et al.) App. A sums the nodes' gradients;
// AdaComp (Chen et al.) averages the learners' compressed gradients.
//
// Output-tile driven, so every dense element is written exactly once and the
// messages are added in array order (bitwise deterministic without float
// atomics):
//   index   for every message and every 4096-element chunk, the first entry
//           at or after the chunk (entries are ascending, so a chunk's entries
//           are [start[c], start[c+1]))
//   decode  one workgroup per chunk: for k = 0..K-1 scatter message k's
//           entries of the chunk into an LDS accumulator (one owner per
//           element within a message), barrier; then divide by K and write
#include <algorithm>

#include "gc_internal.hpp"

namespace gc {

namespace {

struct MsgTable {
    const uint32_t *idx[GC_MAX_MESSAGES];
    const float *val[GC_MAX_MESSAGES];
    const uint32_t *count[GC_MAX_MESSAGES];  // &seg_off[nseg]
    uint64_t cap[GC_MAX_MESSAGES];            // entries never read past cap
};

__device__ __forceinline__ uint32_t msg_count(const MsgTable &m, int k) {
    uint64_t n = *m.count[k];
    return static_cast<uint32_t>(n < m.cap[k] ? n : m.cap[k]);
}

struct DecWs {
    uint32_t *start;  // [GC_MAX_MESSAGES][ndchunk + 1]
};

DecWs dec_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    DecWs w{};
    w.start = c.take<uint32_t>(size_t(GC_MAX_MESSAGES) * (p->ndchunk + 1));
    if (bytes) *bytes = c.used + 256;
    return w;
}

// Chunk holding flat index i (clamped into the plan for malformed input).
__device__ __forceinline__ uint32_t chunk_of(const PlanDev &P, uint32_t i) {
    int lo = 0, hi = P.nseg - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (P.seg_start[mid] <= i) lo = mid;
        else hi = mid - 1;
    }
    const SegDev s = P.seg[lo];
    uint64_t rel = i >= s.off ? (i - s.off) >> kChunkLog2 : 0;
    if (rel >= s.dnchunk) rel = s.dnchunk - 1;
    return s.dchunk0 + static_cast<uint32_t>(rel);
}

__global__ __launch_bounds__(kBlock) void decode_index_kernel(PlanDev P, MsgTable m, DecWs w) {
    const int k = blockIdx.y;
    const uint32_t n = msg_count(m, k);
    const uint32_t *idx = m.idx[k];
    uint32_t *start = w.start + size_t(k) * (P.ndchunk + 1);
    for (uint32_t j = blockIdx.x * kBlock + threadIdx.x; j <= n; j += gridDim.x * kBlock) {
        uint32_t cj = j < n ? chunk_of(P, idx[j]) : P.ndchunk;
        int64_t cp = j > 0 ? int64_t(chunk_of(P, idx[j - 1])) : -1;
        for (int64_t c = cp + 1; c <= int64_t(cj); ++c) start[c] = j;
    }
}

__global__ __launch_bounds__(kBlock) void decode_kernel(PlanDev P, MsgTable m, int K, DecWs w,
                                                        float *__restrict__ dense, int avg,
                                                        int accumulate) {
    const uint32_t c = blockIdx.x;
    const uint32_t s = P.dchunk_seg[c];
    const SegDev seg = P.seg[s];
    const uint32_t pos = c - seg.dchunk0;
    const uint64_t lo = seg.off + (uint64_t(pos) << kChunkLog2);
    const uint32_t rem = seg.len - (pos << kChunkLog2);
    const uint32_t cnt = rem < uint32_t(kChunk) ? rem : uint32_t(kChunk);
    __shared__ float acc[kChunk];
    for (int e = threadIdx.x; e < kChunk; e += kBlock) acc[e] = 0.0f;
    __syncthreads();
    for (int k = 0; k < K; ++k) {
        const uint32_t n = msg_count(m, k);
        const uint32_t *st = w.start + size_t(k) * (P.ndchunk + 1);
        uint32_t a = min(st[c], n);
        uint32_t b = min(max(st[c + 1], a), n);
        const uint32_t *idx = m.idx[k];
        const float *val = m.val[k];
        for (uint32_t i = a + threadIdx.x; i < b; i += kBlock) {
            uint64_t r = uint64_t(idx[i]) - lo;
            if (idx[i] >= lo && r < cnt) acc[r] = acc[r] + val[i];
        }
        __syncthreads();
    }
    const float fk = static_cast<float>(K);
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t e = j * kBlock + threadIdx.x;
        if (e < cnt) {
            float v = acc[e];
            if (avg) v = v / fk;
            if (accumulate) v = dense[lo + e] + v;
            dense[lo + e] = v;
        }
    }
}

}  // namespace

size_t decode_workspace_bytes(const gc_plan *plan) {
    size_t b = 0;
    (void)dec_layout(plan, nullptr, &b);
    return b;
}

}  // namespace gc

using namespace gc;

extern "C" gc_status gc_decompress_accumulate(const gc_plan *plan, const gc_sparse *msgs, int K,
                                              float *dense, int mode, int accumulate, void *ws,
                                              size_t ws_bytes, hipStream_t stream) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_decompress_accumulate: plan is null");
    if (K < 1 || K > GC_MAX_MESSAGES)
        return set_error(GC_EINVAL, "gc_decompress_accumulate: K must be in [1, GC_MAX_MESSAGES]");
    if (!msgs || !dense) return set_error(GC_EINVAL, "gc_decompress_accumulate: msgs and dense must be non-null");
    if (mode != GC_SUM && mode != GC_AVG)
        return set_error(GC_EINVAL, "gc_decompress_accumulate: mode must be GC_SUM or GC_AVG");
    MsgTable m{};
    for (int k = 0; k < K; ++k) {
        if (!msgs[k].idx || !msgs[k].val || !msgs[k].seg_off)
            return set_error(GC_EINVAL, "gc_decompress_accumulate: message pointers must be non-null");
        m.idx[k] = msgs[k].idx;
        m.val[k] = msgs[k].val;
        m.count[k] = msgs[k].seg_off + plan->nseg;
        m.cap[k] = std::min<uint64_t>(msgs[k].cap, 0xFFFFFFFFull);
    }
    size_t need = decode_workspace_bytes(plan);
    if (!ws || ws_bytes < need)
        return set_error(GC_ECAPACITY,
                         "gc_decompress_accumulate: workspace smaller than gc_plan_workspace_bytes");
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return set_error(GC_EINVAL, "gc_decompress_accumulate: workspace must be 256-byte aligned");
    PlanDev P;
    gc_status st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    DecWs w = dec_layout(plan, ws, nullptr);
    uint64_t max_entries = 0;
    for (int k = 0; k < K; ++k) max_entries = std::max<uint64_t>(max_entries, msgs[k].cap);
    unsigned gx = static_cast<unsigned>(std::min<uint64_t>((max_entries + kBlock) / kBlock + 1, 1024));
    decode_index_kernel<<<dim3(gx, K), kBlock, 0, stream>>>(P, m, w);
    decode_kernel<<<plan->ndchunk, kBlock, 0, stream>>>(P, m, K, w, dense, mode == GC_AVG,
                                                        accumulate != 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_decompress_accumulate launch");
    return GC_OK;
}
