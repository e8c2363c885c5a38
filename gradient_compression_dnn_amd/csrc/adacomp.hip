// AdaComp step on gfx950: residual accumulation, bin-local max, adaptive
// selection, sign x layer-scale quantization, new residual.
// "AdaComp: Adaptive Residual Gradient Compression for Data-Parallel
// Distributed Training" (Chen et al.), "Proposed method" and Abstract.
//
// Launch sequence:
//   zero    tickets and per-segment totals
//   pass    one workgroup per chunk of whole bins: G = R + dW, bin maxima by a
//           segmented wave reduction and LDS max, selection, R <- G for every
//           element, selected (idx, G) staged in index order at the chunk's
//           own offset, bin maxima written out
//   scale   one workgroup per segment: pairwise fp64 sum of its bin maxima ->
//           layer scale; chunk prefix sums; the last segment scans the
//           segment totals into the message's seg_off
//   emit    selected entries: q = copysign(scale, G), R <- fl(G - q), message
//           (idx, q) in index order
#include <cmath>

#include "gc_internal.hpp"

namespace gc {

namespace {

struct AdaWs {
    uint32_t *zeroed;
    size_t zero_words;
    uint32_t *ticket, *seg_total;
    float *gmax;
    uint32_t *ccount, *cpre;
    uint32_t *sidx;
    float *sval;
};

AdaWs ada_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    AdaWs w{};
    w.zero_words = 64 + size_t(p->nseg);
    w.zeroed = c.take<uint32_t>(w.zero_words);
    w.ticket = w.zeroed;
    w.seg_total = w.zeroed + 64;
    w.gmax = c.take<float>(p->total_bins);
    w.ccount = c.take<uint32_t>(p->nachunk);
    w.cpre = c.take<uint32_t>(p->nachunk);
    w.sidx = c.take<uint32_t>(p->n_total);
    w.sval = c.take<float>(p->n_total);
    if (bytes) *bytes = c.used + 256;
    return w;
}

struct AChunk {
    uint32_t s;
    SegDev seg;
    uint32_t pos;  // chunk number inside the segment
    uint64_t lo;   // first flat element
    uint32_t cnt;  // elements
};

__device__ __forceinline__ AChunk achunk_info(const PlanDev &P, uint32_t c) {
    AChunk a;
    a.s = P.achunk_seg[c];
    a.seg = P.seg[a.s];
    a.pos = c - a.seg.achunk0;
    uint32_t first = a.pos * a.seg.achunk_len;
    a.lo = a.seg.off + first;
    uint32_t rem = a.seg.len - first;
    a.cnt = rem < a.seg.achunk_len ? rem : a.seg.achunk_len;
    return a;
}

// floor(e / L) for e < 2^13, L <= 2^12, from a float reciprocal plus one
// correction step in each direction.
__device__ __forceinline__ uint32_t div_small(uint32_t e, uint32_t L, float invL) {
    uint32_t q = static_cast<uint32_t>(static_cast<float>(e) * invL);
    if (q * L > e) --q;
    if ((q + 1) * L <= e) ++q;
    return q;
}

__global__ __launch_bounds__(kBlock) void ada_pass_kernel(PlanDev P, const float *__restrict__ dW,
                                                          float *__restrict__ R, float sf,
                                                          AdaWs w) {
    const uint32_t c = blockIdx.x;
    const AChunk a = achunk_info(P, c);
    const uint32_t L = a.seg.bin_len;
    const float invL = 1.0f / static_cast<float>(L);
    const uint32_t nb = (a.cnt + L - 1) / L;
    __shared__ uint32_t gm[kChunk];
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gm[b] = 0u;
    float g[kEPT];
    uint32_t bin[kEPT];
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t e = j * kBlock + threadIdx.x;
        float r = 0.0f, d = 0.0f;
        if (e < a.cnt) {
            r = R[a.lo + e];
            d = dW[a.lo + e];
        }
        g[j] = r + d;
        bin[j] = div_small(e, L, invL);
    }
    __syncthreads();
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t e = j * kBlock + threadIdx.x;
        uint32_t row0 = e - lane;  // element of lane 0 in this wave row
        uint32_t v = e < a.cnt ? (dev_f2u(g[j]) & 0x7FFFFFFFu) : 0u;
        // last lane of this wave row that lies in the same bin
        uint32_t bin_last = (bin[j] + 1) * L - 1;
        uint32_t run_last = bin_last - row0 < uint32_t(kWave) ? bin_last - row0 : uint32_t(kWave - 1);
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            uint32_t o = __shfl_down(v, d, kWave);
            if (uint32_t(lane + d) <= run_last) v = v > o ? v : o;
        }
        bool head = lane == 0 || e == bin[j] * L;
        if (head && e < a.cnt) atomicMax(&gm[bin[j]], v);
    }
    __syncthreads();
    bool flag[kEPT];
    uint32_t pos[kEPT];
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t e = j * kBlock + threadIdx.x;
        float gmx = dev_u2f(gm[bin[j] < nb ? bin[j] : 0]);
        float t = sf * fabsf(g[j]);
        flag[j] = e < a.cnt && gmx > 0.0f && t >= gmx;
        if (e < a.cnt) R[a.lo + e] = g[j];
    }
    uint32_t total = block_compact<kEPT>(flag, pos);
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        if (flag[j]) {
            uint32_t e = j * kBlock + threadIdx.x;
            w.sidx[a.lo + pos[j]] = static_cast<uint32_t>(a.lo + e);
            w.sval[a.lo + pos[j]] = g[j];
        }
    }
    float *gout = w.gmax + a.seg.bin0 + a.pos * (a.seg.achunk_len / L);
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gout[b] = dev_u2f(gm[b]);
    if (threadIdx.x == 0) w.ccount[c] = total;
}

__global__ __launch_bounds__(kBlock) void ada_scale_kernel(PlanDev P, AdaWs w,
                                                           uint32_t *__restrict__ seg_off,
                                                           float *__restrict__ seg_scale) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    const float *gm = w.gmax + seg.bin0;
    double S = block_pairwise_sum(seg.nbins, [&](uint64_t b) { return static_cast<double>(gm[b]); });
    if (threadIdx.x == 0) seg_scale[s] = static_cast<float>(S / static_cast<double>(seg.nbins));
    uint32_t before = 0;
    for (uint32_t r = 0; r < seg.anchunk; r += kBlock) {
        bool in = r + threadIdx.x < seg.anchunk;
        uint32_t cc = seg.achunk0 + r + threadIdx.x;
        uint32_t v = in ? w.ccount[cc] : 0u;
        uint32_t tot;
        uint32_t pre = block_exclusive_scan(v, &tot);
        if (in) w.cpre[cc] = before + pre;
        before += tot;
    }
    if (threadIdx.x == 0) w.seg_total[s] = before;
    if (block_arrive_last(&w.ticket[0], static_cast<uint32_t>(P.nseg))) {
        uint32_t run = 0;
        for (int r = 0; r < P.nseg; r += kBlock) {
            bool in = r + int(threadIdx.x) < P.nseg;
            uint32_t v = in ? load_coherent(w.seg_total + r + threadIdx.x) : 0u;
            uint32_t tot;
            uint32_t pre = block_exclusive_scan(v, &tot);
            if (in) seg_off[r + threadIdx.x] = run + pre;
            run += tot;
        }
        if (threadIdx.x == 0) seg_off[P.nseg] = run;
    }
}

__global__ __launch_bounds__(kBlock) void ada_emit_kernel(PlanDev P, float *__restrict__ R, AdaWs w,
                                                          const uint32_t *__restrict__ seg_off,
                                                          const float *__restrict__ seg_scale,
                                                          uint32_t *__restrict__ out_idx,
                                                          float *__restrict__ out_val) {
    const uint32_t c = blockIdx.x;
    const AChunk a = achunk_info(P, c);
    const uint32_t n = w.ccount[c];
    if (n == 0) return;
    const float scale = seg_scale[a.s];
    const uint32_t base = seg_off[a.s] + w.cpre[c];
    for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
        uint32_t id = w.sidx[a.lo + i];
        float g = w.sval[a.lo + i];
        float q = copysignf(scale, g);
        R[id] = g - q;
        out_idx[base + i] = id;
        out_val[base + i] = q;
    }
}

}  // namespace

size_t adacomp_workspace_bytes(const gc_plan *plan) {
    size_t b = 0;
    (void)ada_layout(plan, nullptr, &b);
    return b;
}

}  // namespace gc

using namespace gc;

extern "C" gc_status gc_adacomp_compress(const gc_plan *plan, const float *dW, float *R,
                                         float scale_factor, gc_sparse *out, void *ws,
                                         size_t ws_bytes, hipStream_t stream) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_adacomp_compress: plan is null");
    if (!dW || !R) return set_error(GC_EINVAL, "gc_adacomp_compress: dW and R must be non-null");
    if (!out || !out->idx || !out->val || !out->seg_off || !out->seg_scale)
        return set_error(GC_EINVAL,
                         "gc_adacomp_compress: out and its idx, val, seg_off, seg_scale must be non-null");
    if (!(scale_factor >= 1.0f) || std::isinf(scale_factor))
        return set_error(GC_EINVAL, "gc_adacomp_compress: scale_factor must be finite and >= 1");
    if (out->cap < plan->n_total)
        return set_error(GC_ECAPACITY, "gc_adacomp_compress: out->cap must be >= n_total");
    size_t need = adacomp_workspace_bytes(plan);
    if (!ws || ws_bytes < need)
        return set_error(GC_ECAPACITY,
                         "gc_adacomp_compress: workspace smaller than gc_plan_workspace_bytes");
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return set_error(GC_EINVAL, "gc_adacomp_compress: workspace must be 256-byte aligned");
    PlanDev P;
    gc_status st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    AdaWs w = ada_layout(plan, ws, nullptr);
    zero_words(w.zeroed, w.zero_words, stream);
    ada_pass_kernel<<<plan->nachunk, kBlock, 0, stream>>>(P, dW, R, scale_factor, w);
    ada_scale_kernel<<<plan->nseg, kBlock, 0, stream>>>(P, w, out->seg_off, out->seg_scale);
    ada_emit_kernel<<<plan->nachunk, kBlock, 0, stream>>>(P, R, w, out->seg_off, out->seg_scale,
                                                          out->idx, out->val);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_adacomp_compress launch");
    return GC_OK;
}
