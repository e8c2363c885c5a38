// AdaComp step on gfx950: residual accumulation, bin-local max, adaptive
// selection, sign x layer-scale quantization, new residual.
// "AdaComp: Adaptive Residual Gradient Compression for Data-Parallel
// Distributed Training" (Chen et al.), "Proposed method" and Abstract.
//
// Launch sequence (the layer scale needs every bin of the layer, so the
// residual is finished in a second pass instead of being patched in place;
// both passes stream whole 16-byte-aligned lines):
//   max     one workgroup per chunk of whole bins: G = R + dW, bin maxima by
//           in-lane runs and LDS max, count of selected entries (selection
//           needs only the bin's max); reads R and dW, writes nothing dense
//   binsum  one workgroup per aligned group of 4096 bins: its node of the
//           layer's pairwise fp64 tree over the bin maxima
//   scale   one workgroup per segment: the rest of the tree -> layer scale;
//           prefix sums of the chunk counts
//   offsets one workgroup: segment totals -> the message's seg_off
//   apply   one workgroup per chunk, last chunk first (its inputs were read
//           last and may still sit in the Infinity Cache): G again, selection
//           against the stored bin maxima, R <- G - copysign(scale, G) or G,
//           message (idx, +-scale) in index order at its final slot
#include <cmath>

#include "gc_internal.hpp"

namespace gc {

namespace {

struct AdaWs {
    uint32_t *seg_total;
    float *gmax;
    double *bpartial;
    uint32_t *ccount, *cpre;
};

AdaWs ada_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    AdaWs w{};
    w.seg_total = c.take<uint32_t>(p->nseg);
    w.gmax = c.take<float>(p->total_bins);
    w.bpartial = c.take<double>(p->nbgroup);
    w.ccount = c.take<uint32_t>(p->nachunk);
    w.cpre = c.take<uint32_t>(p->nachunk);
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

// G = R + dW for the chunk in the 4-wide layout, with each element's bin.
__device__ __forceinline__ void chunk_G(const AChunk &a, const float *R, const float *dW, float invL,
                                        float (&g)[kRows][4], uint32_t (&bin)[kRows][4]) {
    const BufRsrc rr = chunk_buf(R + a.lo, a.cnt), rd = chunk_buf(dW + a.lo, a.cnt);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        float r[4], d[4];
        load4(rr, row_elem(j), r);
        load4(rd, row_elem(j), d);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            g[j][q] = r[q] + d[q];
            bin[j][q] = div_small(row_elem(j) + q, a.seg.bin_len, invL);
        }
    }
}

__global__ __launch_bounds__(kBlock) void ada_max_kernel(PlanDev P, const float *__restrict__ dW,
                                                         const float *__restrict__ R, float sf,
                                                         AdaWs w) {
    const uint32_t c = blockIdx.x;
    const AChunk a = achunk_info(P, c);
    const uint32_t L = a.seg.bin_len;
    const float invL = 1.0f / static_cast<float>(L);
    const uint32_t nb = (a.cnt + L - 1) / L;
    __shared__ uint32_t gm[kChunk];
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gm[b] = 0u;
    float g[kRows][4];
    uint32_t bin[kRows][4];
    chunk_G(a, R, dW, invL, g, bin);
    __syncthreads();
    // bin maxima of |G| (as bit patterns, which order like the values)
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        const uint32_t e0 = row_elem(j);
        uint32_t mag[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) mag[q] = e0 + q < a.cnt ? (dev_f2u(g[j][q]) & 0x7FFFFFFFu) : 0u;
        const uint32_t b_first = __shfl(bin[j][0], 0, kWave);
        const uint32_t b_last = __shfl(bin[j][3], kWave - 1, kWave);
        const uint32_t row0 = e0 - 4u * lane_id();
        if (b_first == b_last) {
            // the wave's 256 elements of this row share one bin
            uint32_t m = max(max(mag[0], mag[1]), max(mag[2], mag[3]));
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(m, d, kWave)));
            if (lane_id() == 0 && row0 < a.cnt) atomicMax(&gm[b_first], m);
        } else {
            // runs of equal bins inside the lane, one LDS max per run
            uint32_t cur = bin[j][0], mv = mag[0];
            bool live = e0 < a.cnt;
#pragma unroll
            for (int q = 1; q < 4; ++q) {
                if (bin[j][q] == cur) {
                    mv = max(mv, mag[q]);
                } else {
                    if (live) atomicMax(&gm[cur], mv);
                    cur = bin[j][q];
                    mv = mag[q];
                    live = e0 + q < a.cnt;
                }
            }
            if (live) atomicMax(&gm[cur], mv);
        }
    }
    __syncthreads();
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        const uint32_t e0 = row_elem(j);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool in = e0 + q < a.cnt;
            const float gmx = dev_u2f(gm[in ? bin[j][q] : 0u]);
            const float t = sf * fabsf(g[j][q]);
            mine += (in && gmx > 0.0f && t >= gmx) ? 1u : 0u;
        }
    }
    uint32_t total;
    (void)block_exclusive_scan(mine, &total);
    float *gout = w.gmax + a.seg.bin0 + a.pos * (a.seg.achunk_len / L);
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gout[b] = dev_u2f(gm[b]);
    if (threadIdx.x == 0) w.ccount[c] = total;
}

// Level 1 of the layer scale's pairwise sum: one workgroup per aligned group
// of 4096 bins of a segment (a node of the segment's tree); thread t holds
// the 16-leaf subtree of bins [16 t, 16 t + 16) of the group.
__global__ __launch_bounds__(kBlock) void ada_binsum_kernel(PlanDev P, AdaWs w) {
    const uint32_t grp = blockIdx.x;
    const uint32_t s = P.bgroup_seg[grp];
    const SegDev seg = P.seg[s];
    const uint32_t b0 = (grp - seg.bgroup0) * kBinGroup + threadIdx.x * (kBinGroup / kBlock);
    const float *gm = w.gmax + seg.bin0;
    double a[kBinGroup / kBlock];
#pragma unroll
    for (uint32_t i = 0; i < kBinGroup / kBlock; ++i)
        a[i] = b0 + i < seg.nbins ? static_cast<double>(gm[b0 + i]) : 0.0;
#pragma unroll
    for (uint32_t h = 1; h < kBinGroup / kBlock; h <<= 1)
#pragma unroll
        for (uint32_t i = 0; i < kBinGroup / kBlock; i += 2 * h) a[i] = a[i] + a[i + h];
    const double sum = block_tree_sum(a[0]);
    if (threadIdx.x == 0) w.bpartial[grp] = sum;
}

__global__ __launch_bounds__(kBlock) void ada_scale_kernel(PlanDev P, AdaWs w,
                                                           float *__restrict__ seg_scale) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    const double *part = w.bpartial + seg.bgroup0;
    double S = block_pairwise_sum(seg.nbgroup, [&](uint64_t i) { return part[i]; });
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
}

__global__ __launch_bounds__(kBlock) void ada_offsets_kernel(int nseg, AdaWs w,
                                                             uint32_t *__restrict__ seg_off) {
    uint32_t run = 0;
    for (int r = 0; r < nseg; r += kBlock) {
        bool in = r + int(threadIdx.x) < nseg;
        uint32_t v = in ? w.seg_total[r + threadIdx.x] : 0u;
        uint32_t tot;
        uint32_t pre = block_exclusive_scan(v, &tot);
        if (in) seg_off[r + threadIdx.x] = run + pre;
        run += tot;
    }
    if (threadIdx.x == 0) seg_off[nseg] = run;
}

__global__ __launch_bounds__(kBlock) void ada_apply_kernel(PlanDev P, const float *__restrict__ dW,
                                                           float *__restrict__ R, float sf, AdaWs w,
                                                           const uint32_t *__restrict__ seg_off,
                                                           const float *__restrict__ seg_scale,
                                                           uint32_t *__restrict__ out_idx,
                                                           float *__restrict__ out_val) {
    const uint32_t c = P.nachunk - 1 - blockIdx.x;
    const AChunk a = achunk_info(P, c);
    const uint32_t L = a.seg.bin_len;
    const float invL = 1.0f / static_cast<float>(L);
    const uint32_t nb = (a.cnt + L - 1) / L;
    __shared__ float gm[kChunk];
    const float *gin = w.gmax + a.seg.bin0 + a.pos * (a.seg.achunk_len / L);
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gm[b] = gin[b];
    float g[kRows][4];
    uint32_t bin[kRows][4];
    chunk_G(a, R, dW, invL, g, bin);
    const float scale = seg_scale[a.s];
    const uint32_t base = seg_off[a.s] + w.cpre[c];
    const uint32_t count = w.ccount[c];  // slots reserved for this chunk by ada_max
    __syncthreads();
    bool flag[kRows][4];
    uint32_t pos[kRows][4];
    const BufRsrc rr = chunk_buf(R + a.lo, a.cnt);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        const uint32_t e0 = row_elem(j);
        float r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool in = e0 + q < a.cnt;
            const float gmx = gm[in ? bin[j][q] : 0u];
            const float t = sf * fabsf(g[j][q]);
            flag[j][q] = in && gmx > 0.0f && t >= gmx;
            const float qv = copysignf(scale, g[j][q]);
            r[q] = flag[j][q] ? g[j][q] - qv : g[j][q];
        }
        store4(rr, e0, r);
    }
    (void)block_compact4(flag, pos);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (flag[j][q] && pos[j][q] < count) {
                out_idx[base + pos[j][q]] = static_cast<uint32_t>(a.lo + row_elem(j) + q);
                out_val[base + pos[j][q]] = copysignf(scale, g[j][q]);
            }
        }
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
    GC_LAUNCH("ada_max", stream, ada_max_kernel<<<plan->nachunk, kBlock, 0, stream>>>(P, dW, R, scale_factor, w));
    GC_LAUNCH("ada_binsum", stream, ada_binsum_kernel<<<plan->nbgroup, kBlock, 0, stream>>>(P, w));
    GC_LAUNCH("ada_scale", stream, ada_scale_kernel<<<plan->nseg, kBlock, 0, stream>>>(P, w, out->seg_scale));
    GC_LAUNCH("ada_offsets", stream, ada_offsets_kernel<<<1, kBlock, 0, stream>>>(plan->nseg, w, out->seg_off));
    GC_LAUNCH("ada_apply", stream, ada_apply_kernel<<<plan->nachunk, kBlock, 0, stream>>>(
        P, dW, R, scale_factor, w, out->seg_off, out->seg_scale, out->idx, out->val));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_adacomp_compress launch");
    return GC_OK;
}
