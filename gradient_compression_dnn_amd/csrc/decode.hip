// Decompress-and-aggregate K sparse messages into a dense update.
// "Deep Gradient Compression" (Lin et al.) App. A sums the nodes' gradients;
// AdaComp (Chen et al.) averages the learners' compressed gradients.
//
// Output-tile driven, so every dense element is written exactly once and the
// messages are added in array order (bitwise deterministic without float
// atomics):
//   index   for every message and every 4096-element chunk, the first entry
//           at or after the chunk, by bisection in its segment's entries
//           (entries are ascending, so a chunk's entries are
//           [start[c], start[c+1]))
//   decode  one workgroup per chunk: for k = 0..K-1 scatter message k's
//           entries of the chunk into an LDS accumulator (one owner per
//           element within a message), barrier; then divide by K and write
#include <algorithm>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

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

constexpr uint32_t kSparseChunk = 32;  // up to this many entries: no LDS accumulator

// start[k][c] = first entry of message k at or after chunk c.  Chunk c lies
// in segment s, whose entries are [seg_off[s], seg_off[s+1]) of the message,
// ascending: start is the first of them at or after the chunk's first
// element, a lower bound by bisection, and start[k][ndchunk] = count_k.  One
// thread per chunk and message; the searches of a segment share their upper
// levels in cache, and the pass reads a few lines per chunk instead of every
// entry.  For a message that breaks the layout (descending indices, offsets
// past the count) the starts are still in [0, count_k], clamped, and the
// decode pass clamps each range it reads to count_k.
__global__ __launch_bounds__(kBlock) void decode_index_kernel(PlanDev P, MsgTable m, DecWs w) {
    const int k = blockIdx.y;
    const uint32_t c = blockIdx.x * kBlock + threadIdx.x;
    if (c > P.ndchunk) return;
    const uint32_t n = msg_count(m, k);
    uint32_t *start = w.start + size_t(k) * (P.ndchunk + 1);
    if (c == P.ndchunk) {
        start[c] = n;
        return;
    }
    const ChunkRec rec = P.dchunk_rec[c];
    const uint32_t *seg_off = m.count[k] - P.nseg;
    uint32_t lo = min(seg_off[rec.z], n), hi = min(seg_off[rec.z + 1], n);
    if (hi < lo) hi = lo;
    const uint32_t *idx = m.idx[k];
    while (lo < hi) {
        const uint32_t mid = lo + (hi - lo) / 2;
        if (idx[mid] < rec.x) lo = mid + 1;
        else hi = mid;
    }
    start[c] = lo;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) { return wave_total(v); }

// One workgroup per output chunk.  Lane k (< K) of every wave loads message
// k's entry range for the chunk, so every wave sees the same entry total and
// picks the same path without a workgroup vote.  The average divides by K;
// for K a power of two that is the same real number as multiplying by 1/K,
// so the exact product is used (identical correctly rounded result).
__global__ __launch_bounds__(kBlock) void decode_kernel(PlanDev P, MsgTable m, int K, DecWs w,
                                                        float *__restrict__ dense, int avg,
                                                        int accumulate) {
    // the chunk record and the entry ranges depend on c alone: one round trip
    const uint32_t c = blockIdx.x;
    const ChunkRec rec = P.dchunk_rec[c];
    const uint64_t lo = rec.x;
    const uint32_t cnt = rec.y;
    const BufRsrc rd = chunk_buf(dense + lo, cnt);
    __shared__ float acc[kChunk];
    const int lane = lane_id();
    uint32_t a = 0, b = 0;
    if (lane < K) {
        // message lane's entries of the chunk, clamped to its count: for
        // ascending indices the index pass wrote every start within it, and
        // whatever it left for other input, no entry past the count is read
        const uint32_t *st = w.start + size_t(lane) * (P.ndchunk + 1);
        const uint32_t nk = msg_count(m, lane);
        a = min(st[c], nk);
        b = min(max(st[c + 1], a), nk);
    }
    const uint32_t total = wave_sum(b - a);  // identical in every wave
    float v[kRows][4];
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) v[j][q] = 0.0f;
    if (total != 0 && total <= kSparseChunk) {
        // few entries: lane l of every wave loads the l-th entry of the
        // chunk (messages in order, entries ascending within a message) in a
        // single round trip; then every thread walks them in that order and
        // adds those that fall on its own elements
        const uint32_t cntk = b - a;
        uint32_t pre = wave_inclusive_scan(cntk) - cntk;  // exclusive scan over the message lanes
        // message q holds chunk entries [pre_q, pre_q + cnt_q); every lane
        // takes part in the shuffles, then lanes below the total load
        int k = 0;
        uint32_t base = 0, first = 0;
        for (int q = 0; q < K; ++q) {
            const uint32_t pq = __shfl(pre, q, kWave), cq = __shfl(cntk, q, kWave);
            const uint32_t aq = __shfl(a, q, kWave);
            if (uint32_t(lane) >= pq && uint32_t(lane) < pq + cq) {
                k = q;
                base = pq;
                first = aq;
            }
        }
        uint32_t my_id = 0;
        float my_x = 0.0f;
        if (uint32_t(lane) < total) {
            const uint32_t i = first + (uint32_t(lane) - base);
            my_id = m.idx[k][i];
            my_x = m.val[k][i];
        }
        for (uint32_t l = 0; l < total; ++l) {
            const uint32_t id = __shfl(my_id, int(l), kWave);
            const float x = __shfl(my_x, int(l), kWave);
            const uint64_t r = uint64_t(id) - lo;
            if (id < lo || r >= cnt) continue;
            const uint32_t e = static_cast<uint32_t>(r);
            if (((e >> 2) & (kBlock - 1)) != threadIdx.x) continue;
            const uint32_t j = e >> 10, q = e & 3u;
#pragma unroll
            for (int jj = 0; jj < kRows; ++jj)
#pragma unroll
                for (int qq = 0; qq < 4; ++qq)
                    if (uint32_t(jj) == j && uint32_t(qq) == q) v[jj][qq] = v[jj][qq] + x;
        }
    } else if (total != 0) {
        for (int e = threadIdx.x; e < kChunk; e += kBlock) acc[e] = 0.0f;
        __syncthreads();
        // entries per thread with loads in flight together: 2048 per round
        // covers the ~1100 entries a chunk holds at AdaComp's density in one
        // round trip
        constexpr uint32_t kBatch = 8;
        for (int k = 0; k < K; ++k) {
            const uint32_t ak = __shfl(a, k, kWave), bk = __shfl(b, k, kWave);
            const uint32_t *idx = m.idx[k];
            const float *val = m.val[k];
            for (uint64_t i0 = ak; i0 < bk; i0 += kBatch * kBlock) {
                uint32_t id[kBatch];
                float x[kBatch];
#pragma unroll
                for (uint32_t u = 0; u < kBatch; ++u) {
                    const uint64_t i = uint64_t(i0) + u * kBlock + threadIdx.x;
                    const uint32_t ic = i < bk ? static_cast<uint32_t>(i) : bk - 1;
                    id[u] = idx[ic];
                    x[u] = val[ic];
                }
#pragma unroll
                for (uint32_t u = 0; u < kBatch; ++u) {
                    const uint64_t r = uint64_t(id[u]) - lo;
                    if (uint64_t(i0) + u * kBlock + threadIdx.x < bk && id[u] >= lo && r < cnt)
                        acc[r] = acc[r] + x[u];
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int j = 0; j < kRows; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) v[j][q] = acc[row_elem(j) + q];
    }
    const bool pow2 = (K & (K - 1)) == 0;
    const float fk = static_cast<float>(K);
    const float inv = 1.0f / fk;  // exact for a power of two
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        const uint32_t e0 = row_elem(j);
        if (avg && K > 1) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[j][q] = pow2 ? v[j][q] * inv : v[j][q] / fk;
        }
        if (accumulate) {
            float d[4];
            load4(rd, e0, d);
#pragma unroll
            for (int q = 0; q < 4; ++q) v[j][q] = d[q] + v[j][q];
        }
        store4(rd, e0, v[j]);
    }
}

}  // namespace

size_t decode_workspace_bytes(const gc_plan *plan) {
    size_t b = 0;
    (void)dec_layout(plan, nullptr, &b);
    return b;
}

namespace {

// Host checks shared by both decode entry points; fills the message table.
gc_status decode_args(const char *fn, const gc_plan *plan, const gc_sparse *msgs, int K, const float *dense,
                      int mode, MsgTable *m) {
    const std::string f(fn);
    if (!plan) return set_error(GC_EINVAL, f + ": plan is null");
    if (K < 1 || K > GC_MAX_MESSAGES) return set_error(GC_EINVAL, f + ": K must be in [1, GC_MAX_MESSAGES]");
    if (!msgs || !dense) return set_error(GC_EINVAL, f + ": msgs and dense must be non-null");
    if (mode != GC_SUM && mode != GC_AVG) return set_error(GC_EINVAL, f + ": mode must be GC_SUM or GC_AVG");
    for (int k = 0; k < K; ++k) {
        if (!msgs[k].idx || !msgs[k].val || !msgs[k].seg_off)
            return set_error(GC_EINVAL, f + ": message pointers must be non-null");
        m->idx[k] = msgs[k].idx;
        m->val[k] = msgs[k].val;
        m->count[k] = msgs[k].seg_off + plan->nseg;
        m->cap[k] = std::min<uint64_t>(msgs[k].cap, 0xFFFFFFFFull);
    }
    return GC_OK;
}

gc_status decode_launch(const char *fn, const gc_plan *plan, const PlanDev &P, const MsgTable &m, int K,
                        const DecWs &w, float *dense, int mode, int accumulate, hipStream_t stream) {
    GC_LAUNCH("decode_index", stream,
              decode_index_kernel<<<dim3(grid_1d(uint64_t(plan->ndchunk) + 1, kBlock), K), kBlock, 0, stream>>>(P, m, w));
    GC_LAUNCH("decode", stream, decode_kernel<<<plan->ndchunk, kBlock, 0, stream>>>(P, m, K, w, dense, mode == GC_AVG,
                                                        accumulate != 0));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, fn);
    return GC_OK;
}

}  // namespace

// ------------------------------------------------------- fixed scratch
// gc_decompress_accumulate_noalloc keeps the index pass's start table in
// this array instead of a caller workspace: K * (ndchunk + 1) u32, at most
// kScratchBytes.  Every GPU the library runs on holds its own copy from the
// code object's load until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): the device address comes from hipGetSymbolAddress, once per
// device, and is kept per device.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / sizeof(uint32_t)];

namespace {
std::mutex g_scratch_mu;
std::vector<std::pair<int, uint32_t *>> g_scratch_addr;  // (device, address of its copy)

gc_status scratch_on_current_device(uint32_t **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_error(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    for (const auto &pr : g_scratch_addr)
        if (pr.first == dev) {
            *out = pr.second;
            return GC_OK;
        }
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_error(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return set_error(GC_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_addr.emplace_back(dev, static_cast<uint32_t *>(ptr));
    *out = static_cast<uint32_t *>(ptr);
    return GC_OK;
}
}  // namespace

}  // namespace gc

using namespace gc;

extern "C" gc_status gc_decompress_accumulate(const gc_plan *plan, const gc_sparse *msgs, int K,
                                              float *dense, int mode, int accumulate, void *ws,
                                              size_t ws_bytes, hipStream_t stream) {
    clear_error();
    MsgTable m{};
    gc_status st = decode_args("gc_decompress_accumulate", plan, msgs, K, dense, mode, &m);
    if (st != GC_OK) return st;
    size_t need = decode_workspace_bytes(plan);
    if (!ws || ws_bytes < need)
        return set_error(GC_ECAPACITY,
                         "gc_decompress_accumulate: workspace smaller than gc_plan_workspace_bytes");
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return set_error(GC_EINVAL, "gc_decompress_accumulate: workspace must be 256-byte aligned");
    PlanDev P;
    st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    DecWs w = dec_layout(plan, ws, nullptr);
    return decode_launch("gc_decompress_accumulate launch", plan, P, m, K, w, dense, mode, accumulate, stream);
}

extern "C" uint64_t gc_decompress_noalloc_max_chunks(int K) {
    if (K < 1 || K > GC_MAX_MESSAGES) return 0;
    return kScratchBytes / sizeof(uint32_t) / uint64_t(K) - 1;
}

extern "C" gc_status gc_decompress_accumulate_noalloc(const gc_plan *plan, const gc_sparse *msgs, int K,
                                                      float *dense, int mode, int accumulate,
                                                      hipStream_t stream) {
    clear_error();
    MsgTable m{};
    gc_status st = decode_args("gc_decompress_accumulate_noalloc", plan, msgs, K, dense, mode, &m);
    if (st != GC_OK) return st;
    if (uint64_t(plan->ndchunk) > gc_decompress_noalloc_max_chunks(K))
        return set_error(GC_ECAPACITY,
                         "gc_decompress_accumulate_noalloc: K * (chunks + 1) start entries exceed the " +
                             std::to_string(kScratchBytes >> 20) + " MiB fixed scratch (" +
                             std::to_string(K) + " messages, " + std::to_string(plan->ndchunk) +
                             " chunks); use gc_decompress_accumulate with a workspace");
    PlanDev P;
    st = plan_device_resident(plan, &P);
    if (st != GC_OK) return st;
    uint32_t *start = nullptr;
    st = scratch_on_current_device(&start);
    if (st != GC_OK) return st;
    DecWs w{};
    w.start = start;
    return decode_launch("gc_decompress_accumulate_noalloc launch", plan, P, m, K, w, dense, mode, accumulate,
                         stream);
}
