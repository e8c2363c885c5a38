// DGC step on gfx950: local clipping, momentum correction, exact top-k by
// radix select on |V| bit patterns, ordered compaction, momentum factor
// masking.  "Deep Gradient Compression" (Lin et al.), §3.1–§3.3, App. C, D.
//
// Launch sequence (one workgroup per 4096-element chunk of a segment):
//   zero          histograms and tickets
//   norm          (clip only) pairwise fp64 sum of G^2 per chunk; the last
//                 chunk of a segment finishes the tree and the clip factor
//   update        U <- fl(fl(m U) + fl(c G)); V <- fl(V + U); LDS histogram of
//                 key >> 20; the last chunk of a segment finds digit 1
//   stage         re-read V, keep entries whose digit 1 is at or above the
//                 k-th largest's (ordered, at the chunk's own offset); histogram
//                 digit 2 of the boundary bucket; last chunk finds digit 2
//   refine        digit-3 histogram over staged boundary entries; last chunk
//                 fixes the threshold key T and the tie count
//   count         per chunk: keys > T and keys == T; last chunk scans the
//                 segment's chunks into output slots and ties to take
//   emit          write (idx, V) in index order, then zero U and V there
#include <cmath>

#include "gc_internal.hpp"

namespace gc {

namespace {

struct SegState {
    float clip;
    uint32_t d1, above1, d2, above2, T, gt, need_eq;
};

enum { kTicketNorm, kTicketUpdate, kTicketStage, kTicketRefine, kTicketCount, kTickets };

struct DgcWs {
    uint32_t *zeroed;   // start of the region cleared every call
    size_t zero_words;
    uint32_t *hist1, *hist2, *hist3, *ticket;
    SegState *st;
    double *partial;
    uint32_t *ccount, *cgt, *ceq, *cout, *ctake;
    uint32_t *sidx;
    float *sval;
};

DgcWs dgc_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    DgcWs w{};
    size_t per_seg = size_t(kHist1) + kHist2 + kHist3 + kTickets;
    w.zero_words = per_seg * p->nseg;
    w.zeroed = c.take<uint32_t>(w.zero_words);
    w.hist1 = w.zeroed;
    w.hist2 = w.hist1 + size_t(kHist1) * p->nseg;
    w.hist3 = w.hist2 + size_t(kHist2) * p->nseg;
    w.ticket = w.hist3 + size_t(kHist3) * p->nseg;
    w.st = c.take<SegState>(p->nseg);
    w.partial = c.take<double>(p->ndchunk);
    w.ccount = c.take<uint32_t>(p->ndchunk);
    w.cgt = c.take<uint32_t>(p->ndchunk);
    w.ceq = c.take<uint32_t>(p->ndchunk);
    w.cout = c.take<uint32_t>(p->ndchunk);
    w.ctake = c.take<uint32_t>(p->ndchunk);
    w.sidx = c.take<uint32_t>(p->n_total);
    w.sval = c.take<float>(p->n_total);
    if (bytes) *bytes = c.used + 256;
    return w;
}

struct ChunkInfo {
    uint32_t s;
    SegDev seg;
    uint64_t lo;   // first flat element of the chunk
    uint32_t cnt;  // elements in the chunk
};

__device__ __forceinline__ ChunkInfo chunk_info(const PlanDev &P, uint32_t c) {
    ChunkInfo ci;
    ci.s = P.dchunk_seg[c];
    ci.seg = P.seg[ci.s];
    uint32_t pos = c - ci.seg.dchunk0;
    ci.lo = ci.seg.off + (uint64_t(pos) << kChunkLog2);
    uint32_t rem = ci.seg.len - (pos << kChunkLog2);
    ci.cnt = rem < uint32_t(kChunk) ? rem : uint32_t(kChunk);
    return ci;
}

__device__ __forceinline__ uint32_t mag_key(float v) { return dev_f2u(v) & 0x7FFFFFFFu; }

// ------------------------------------------------------------------ norm
__global__ __launch_bounds__(kBlock) void dgc_norm_kernel(PlanDev P, const float *__restrict__ G,
                                                          DgcWs w, float thr) {
    const uint32_t c = blockIdx.x;
    const ChunkInfo ci = chunk_info(P, c);
    __shared__ float tile[kChunk];
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t e = j * kBlock + threadIdx.x;
        tile[e] = e < ci.cnt ? G[ci.lo + e] : 0.0f;
    }
    __syncthreads();
    // leaves [16t, 16t+16) of the chunk: a perfect 16-leaf subtree per thread
    double a[kEPT];
#pragma unroll
    for (int i = 0; i < kEPT; ++i) {
        double x = static_cast<double>(tile[threadIdx.x * kEPT + i]);
        a[i] = x * x;
    }
#pragma unroll
    for (int w2 = 1; w2 < kEPT; w2 <<= 1)
#pragma unroll
        for (int i = 0; i < kEPT; i += 2 * w2) a[i] = a[i] + a[i + w2];
    double chunk_sum = block_tree_sum(a[0]);
    if (threadIdx.x == 0) w.partial[c] = chunk_sum;
    if (block_arrive_last(&w.ticket[ci.s * kTickets + kTicketNorm], ci.seg.dnchunk)) {
        const double *part = w.partial + ci.seg.dchunk0;
        double S = block_pairwise_sum(ci.seg.dnchunk,
                                      [&](uint64_t g) { return load_coherent(part + g); });
        if (threadIdx.x == 0) {
            double norm = sqrt(S);
            float cl = 1.0f;
            if (norm > static_cast<double>(thr)) cl = static_cast<float>(static_cast<double>(thr) / norm);
            w.st[ci.s].clip = cl;
        }
    }
}

// ---------------------------------------------------------------- update
__global__ __launch_bounds__(kBlock) void dgc_update_kernel(PlanDev P, const float *__restrict__ G,
                                                            float *__restrict__ U,
                                                            float *__restrict__ V, float m,
                                                            int use_clip, DgcWs w) {
    const uint32_t c = blockIdx.x;
    const ChunkInfo ci = chunk_info(P, c);
    __shared__ uint32_t hist[kHist1];
    for (int i = threadIdx.x; i < kHist1; i += kBlock) hist[i] = 0u;
    const float clip = use_clip ? w.st[ci.s].clip : 1.0f;
    float g[kEPT], u[kEPT], v[kEPT];
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t e = j * kBlock + threadIdx.x;
        if (e < ci.cnt) {
            g[j] = G[ci.lo + e];
            u[j] = U[ci.lo + e];
            v[j] = V[ci.lo + e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t e = j * kBlock + threadIdx.x;
        if (e < ci.cnt) {
            float gc = clip * g[j];
            float un = m * u[j];
            un = un + gc;
            float vn = v[j] + un;
            U[ci.lo + e] = un;
            V[ci.lo + e] = vn;
            atomicAdd(&hist[mag_key(vn) >> (kDigit2Bits + kDigit3Bits)], 1u);
        }
    }
    __syncthreads();
    uint32_t *h1 = w.hist1 + size_t(ci.s) * kHist1;
    for (int i = threadIdx.x; i < kHist1; i += kBlock) {
        uint32_t n = hist[i];
        if (n) atomicAdd(&h1[i], n);
    }
    if (block_arrive_last(&w.ticket[ci.s * kTickets + kTicketUpdate], ci.seg.dnchunk)) {
        uint32_t above;
        uint32_t d1 = block_find_bucket<kHist1>(
            ci.seg.k, [&](int b) { return load_coherent(h1 + b); }, &above);
        if (threadIdx.x == 0) {
            w.st[ci.s].d1 = d1;
            w.st[ci.s].above1 = above;
        }
    }
}

// ----------------------------------------------------------------- stage
__global__ __launch_bounds__(kBlock) void dgc_stage_kernel(PlanDev P, const float *__restrict__ V,
                                                           DgcWs w) {
    const uint32_t c = blockIdx.x;
    const ChunkInfo ci = chunk_info(P, c);
    const uint32_t d1 = w.st[ci.s].d1;
    uint32_t *h2 = w.hist2 + size_t(ci.s) * kHist2;
    float v[kEPT];
    bool flag[kEPT];
    uint32_t pos[kEPT];
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t e = j * kBlock + threadIdx.x;
        v[j] = e < ci.cnt ? V[ci.lo + e] : 0.0f;
        uint32_t key = mag_key(v[j]);
        uint32_t dig1 = key >> (kDigit2Bits + kDigit3Bits);
        flag[j] = e < ci.cnt && dig1 >= d1;
        if (e < ci.cnt && dig1 == d1) atomicAdd(&h2[(key >> kDigit3Bits) & (kHist2 - 1)], 1u);
    }
    uint32_t total = block_compact<kEPT>(flag, pos);
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        if (flag[j]) {
            uint32_t e = j * kBlock + threadIdx.x;
            w.sidx[ci.lo + pos[j]] = static_cast<uint32_t>(ci.lo + e);
            w.sval[ci.lo + pos[j]] = v[j];
        }
    }
    if (threadIdx.x == 0) w.ccount[c] = total;
    if (block_arrive_last(&w.ticket[ci.s * kTickets + kTicketStage], ci.seg.dnchunk)) {
        const uint32_t need = ci.seg.k - w.st[ci.s].above1;
        uint32_t above;
        uint32_t d2 = block_find_bucket<kHist2>(
            need, [&](int b) { return load_coherent(h2 + b); }, &above);
        if (threadIdx.x == 0) {
            w.st[ci.s].d2 = d2;
            w.st[ci.s].above2 = w.st[ci.s].above1 + above;
        }
    }
}

// ---------------------------------------------------------------- refine
__global__ __launch_bounds__(kBlock) void dgc_refine_kernel(PlanDev P, DgcWs w) {
    const uint32_t c = blockIdx.x;
    const ChunkInfo ci = chunk_info(P, c);
    const uint32_t n = w.ccount[c];
    const uint32_t prefix = (w.st[ci.s].d1 << kDigit2Bits) | w.st[ci.s].d2;
    uint32_t *h3 = w.hist3 + size_t(ci.s) * kHist3;
    for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
        uint32_t key = mag_key(w.sval[ci.lo + i]);
        if ((key >> kDigit3Bits) == prefix) atomicAdd(&h3[key & (kHist3 - 1)], 1u);
    }
    if (block_arrive_last(&w.ticket[ci.s * kTickets + kTicketRefine], ci.seg.dnchunk)) {
        const uint32_t need = ci.seg.k - w.st[ci.s].above2;
        uint32_t above;
        uint32_t d3 = block_find_bucket<kHist3>(
            need, [&](int b) { return load_coherent(h3 + b); }, &above);
        if (threadIdx.x == 0) {
            uint32_t gt = w.st[ci.s].above2 + above;
            w.st[ci.s].T = (prefix << kDigit3Bits) | d3;
            w.st[ci.s].gt = gt;
            w.st[ci.s].need_eq = ci.seg.k - gt;
        }
    }
}

// ----------------------------------------------------------------- count
__global__ __launch_bounds__(kBlock) void dgc_count_kernel(PlanDev P, DgcWs w,
                                                           uint32_t *__restrict__ seg_off) {
    const uint32_t c = blockIdx.x;
    const ChunkInfo ci = chunk_info(P, c);
    const uint32_t n = w.ccount[c];
    const uint32_t T = w.st[ci.s].T;
    uint32_t ngt = 0, neq = 0;
    for (uint32_t i = threadIdx.x; i < n; i += kBlock) {
        uint32_t key = mag_key(w.sval[ci.lo + i]);
        ngt += key > T;
        neq += key == T;
    }
    uint32_t tgt, teq;
    (void)block_exclusive_scan(ngt, &tgt);
    (void)block_exclusive_scan(neq, &teq);
    if (threadIdx.x == 0) {
        w.cgt[c] = tgt;
        w.ceq[c] = teq;
    }
    if (block_arrive_last(&w.ticket[ci.s * kTickets + kTicketCount], ci.seg.dnchunk)) {
        // scan the segment's chunks in order: ties go to the lowest indices
        const uint32_t need_eq = w.st[ci.s].need_eq;
        uint32_t eq_before = 0, sel_before = 0;
        for (uint32_t r = 0; r < ci.seg.dnchunk; r += kBlock) {
            uint32_t cc = ci.seg.dchunk0 + r + threadIdx.x;
            bool in = r + threadIdx.x < ci.seg.dnchunk;
            uint32_t eq = in ? load_coherent(w.ceq + cc) : 0u;
            uint32_t gt = in ? load_coherent(w.cgt + cc) : 0u;
            uint32_t eq_tot;
            uint32_t eq_pre = eq_before + block_exclusive_scan(eq, &eq_tot);
            uint32_t take = 0;
            if (need_eq > eq_pre) take = min(need_eq - eq_pre, eq);
            uint32_t sel = gt + take;
            uint32_t sel_tot;
            uint32_t sel_pre = sel_before + block_exclusive_scan(sel, &sel_tot);
            if (in) {
                w.ctake[cc] = take;
                w.cout[cc] = ci.seg.kbase + sel_pre;
            }
            eq_before += eq_tot;
            sel_before += sel_tot;
        }
        if (threadIdx.x == 0) {
            seg_off[ci.s] = ci.seg.kbase;
            if (ci.s == uint32_t(P.nseg - 1)) seg_off[P.nseg] = ci.seg.kbase + ci.seg.k;
        }
    }
}

// ------------------------------------------------------------------ emit
__global__ __launch_bounds__(kBlock) void dgc_emit_kernel(PlanDev P, float *__restrict__ U,
                                                          float *__restrict__ V, DgcWs w,
                                                          uint32_t *__restrict__ out_idx,
                                                          float *__restrict__ out_val) {
    const uint32_t c = blockIdx.x;
    const ChunkInfo ci = chunk_info(P, c);
    const uint32_t n = w.ccount[c];
    if (n == 0) return;
    const uint32_t T = w.st[ci.s].T;
    const uint32_t take = w.ctake[c];
    const uint32_t base = w.cout[c];
    bool eqf[kEPT], self[kEPT];
    uint32_t eqpos[kEPT], pos[kEPT];
    uint32_t id[kEPT];
    float val[kEPT];
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        uint32_t i = j * kBlock + threadIdx.x;
        bool in = i < n;
        id[j] = in ? w.sidx[ci.lo + i] : 0u;
        val[j] = in ? w.sval[ci.lo + i] : 0.0f;
        uint32_t key = mag_key(val[j]);
        eqf[j] = in && key == T;
        self[j] = in && key > T;
    }
    (void)block_compact<kEPT>(eqf, eqpos);
#pragma unroll
    for (int j = 0; j < kEPT; ++j) self[j] = self[j] || (eqf[j] && eqpos[j] < take);
    (void)block_compact<kEPT>(self, pos);
    // a segment owns message slots [kbase, kbase + k): never write past them
    const uint32_t limit = ci.seg.kbase + ci.seg.k;
#pragma unroll
    for (int j = 0; j < kEPT; ++j) {
        if (self[j] && base + pos[j] < limit) {
            out_idx[base + pos[j]] = id[j];
            out_val[base + pos[j]] = val[j];
            V[id[j]] = 0.0f;
            U[id[j]] = 0.0f;
        }
    }
}

}  // namespace

size_t dgc_workspace_bytes(const gc_plan *plan) {
    size_t b = 0;
    (void)dgc_layout(plan, nullptr, &b);
    return b;
}

}  // namespace gc

using namespace gc;

extern "C" gc_status gc_dgc_step(const gc_plan *plan, const float *G, float *U, float *V,
                                 float momentum, float thr_G, int num_nodes, gc_sparse *out,
                                 void *ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_dgc_step: plan is null");
    if (!G || !U || !V) return set_error(GC_EINVAL, "gc_dgc_step: G, U and V must be non-null");
    if (!out || !out->idx || !out->val || !out->seg_off)
        return set_error(GC_EINVAL, "gc_dgc_step: out, out->idx, out->val, out->seg_off must be non-null");
    if (!(momentum >= 0.0f && momentum < 1.0f))
        return set_error(GC_EINVAL, "gc_dgc_step: momentum must be in [0, 1)");
    if (std::isnan(thr_G) || std::isinf(thr_G))
        return set_error(GC_EINVAL, "gc_dgc_step: thr_G must be finite");
    if (num_nodes < 1) return set_error(GC_EINVAL, "gc_dgc_step: num_nodes must be >= 1");
    if (out->cap < plan->total_k)
        return set_error(GC_ECAPACITY, "gc_dgc_step: out->cap below the plan's total k");
    size_t need = dgc_workspace_bytes(plan);
    if (!ws || ws_bytes < need)
        return set_error(GC_ECAPACITY, "gc_dgc_step: workspace smaller than gc_plan_workspace_bytes");
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return set_error(GC_EINVAL, "gc_dgc_step: workspace must be 256-byte aligned");
    PlanDev P;
    gc_status st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    DgcWs w = dgc_layout(plan, ws, nullptr);
    const unsigned grid = plan->ndchunk;
    const bool clip = thr_G > 0.0f;
    const float thr = clip ? static_cast<float>(static_cast<double>(thr_G) /
                                                std::sqrt(static_cast<double>(num_nodes)))
                           : 0.0f;
    zero_words(w.zeroed, w.zero_words, stream);
    if (clip) dgc_norm_kernel<<<grid, kBlock, 0, stream>>>(P, G, w, thr);
    dgc_update_kernel<<<grid, kBlock, 0, stream>>>(P, G, U, V, momentum, clip ? 1 : 0, w);
    dgc_stage_kernel<<<grid, kBlock, 0, stream>>>(P, V, w);
    dgc_refine_kernel<<<grid, kBlock, 0, stream>>>(P, w);
    dgc_count_kernel<<<grid, kBlock, 0, stream>>>(P, w, out->seg_off);
    dgc_emit_kernel<<<grid, kBlock, 0, stream>>>(P, U, V, w, out->idx, out->val);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_dgc_step launch");
    return GC_OK;
}
