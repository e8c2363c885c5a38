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
    uint16_t *sign;  // [nachunk][kBlock] deferred mode: sign bits of this step's G
};

// Deferred-residual state of one learner (caller-owned, zero before the
// first step).  Thread t of chunk c holds 16 elements, (row j, q) at bit
// 4 j + q of word c * kBlock + t.
struct AdaState {
    uint16_t *sel;  // [nachunk][kBlock] entries sent in the last step
    float *scale;   // [nseg] layer scales of the last step
};

AdaState ada_state_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    AdaState st{};
    st.sel = c.take<uint16_t>(size_t(p->nachunk) * kBlock);
    st.scale = c.take<float>(p->nseg);
    if (bytes) *bytes = c.used;
    return st;
}

AdaWs ada_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    AdaWs w{};
    w.seg_total = c.take<uint32_t>(p->nseg);
    w.gmax = c.take<float>(p->total_bins);
    w.bpartial = c.take<double>(p->nbgroup);
    w.ccount = c.take<uint32_t>(p->nachunk);
    w.cpre = c.take<uint32_t>(p->nachunk);
    w.sign = c.take<uint16_t>(size_t(p->nachunk) * kBlock);
    if (bytes) *bytes = c.used + 256;
    return w;
}

// A chunk from its 16-byte record, so the chunk's data loads can go out
// after one round trip; the bin length comes from the segment record, which
// is fetched alongside.
struct AChunk {
    uint32_t s;
    uint64_t lo;         // first flat element
    uint32_t cnt;        // elements
    uint32_t bin_first;  // first bin of the chunk in the plan-wide bin array
    uint32_t L;          // bin length
};

__device__ __forceinline__ AChunk achunk_info(const PlanDev &P, uint32_t c) {
    const ChunkRec rec = P.achunk_rec[c];
    AChunk a;
    a.lo = rec.x;
    a.cnt = rec.y;
    a.s = rec.z;
    a.bin_first = rec.w;
    a.L = P.seg[a.s].bin_len;
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

// The two readings of the adaptive threshold (the page's "Proposed method"
// gives a scale factor s, empirically 2, without fixing what it multiplies):
//   kRuleResidual (default): sent when g_max(bin) > 0 and fl(s |G|) >= g_max;
//   kRuleGradient: the factor weighs the new gradient, H = fl(G + fl((s - 1)
//     dW)) (for s = 2, fl(G + dW)); sent when g_max(bin) > 0 and |H| >= g_max,
//     and every entry with |G| = g_max is sent too.
constexpr int kRuleResidual = GC_ADACOMP_RULE_RESIDUAL;
constexpr int kRuleGradient = GC_ADACOMP_RULE_GRADIENT;

// G = R + dW for the chunk in the 4-wide layout, with each element's bin;
// under kRuleGradient also H = G + (s - 1) dW (s1 = s - 1).
template <int kRule>
__device__ __forceinline__ void chunk_G(const AChunk &a, const float *R, const float *dW, float invL, float s1,
                                        float (&g)[kRows][4], float (&h)[kRows][4], uint32_t (&bin)[kRows][4]) {
    const BufRsrc rr = chunk_buf(R + a.lo, a.cnt), rd = chunk_buf(dW + a.lo, a.cnt);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        float r[4], d[4];
        load4(rr, row_elem(j), r);
        load4(rd, row_elem(j), d);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            g[j][q] = r[q] + d[q];
            if (kRule == kRuleGradient) h[j][q] = g[j][q] + s1 * d[q];
            bin[j][q] = div_small(row_elem(j) + q, a.L, invL);
        }
    }
}

// Bin maxima of |G| over the chunk into the LDS array gm (zeroed by the
// caller, then a barrier), as bit patterns, which order like the values.  A
// NaN (pattern above +Inf's) counts as 0: it never raises a bin's max.
__device__ __forceinline__ uint32_t mag_bits(float v) {
    const uint32_t m = dev_f2u(v) & 0x7FFFFFFFu;
    return m > 0x7F800000u ? 0u : m;
}

__device__ __forceinline__ void chunk_bin_max(const AChunk &a, const float (&g)[kRows][4],
                                              const uint32_t (&bin)[kRows][4], uint32_t *gm) {
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        const uint32_t e0 = row_elem(j);
        uint32_t mag[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) mag[q] = e0 + q < a.cnt ? mag_bits(g[j][q]) : 0u;
        const uint32_t b_first = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin[j][0]), 0));
        const uint32_t b_last = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(bin[j][3]), kWave - 1));
        const uint32_t row0 = e0 - 4u * lane_id();
        if (b_first == b_last) {
            // the wave's 256 elements of this row share one bin
            const uint32_t m = wave_max_all(max(max(mag[0], mag[1]), max(mag[2], mag[3])));
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
}

// Whether an entry (G, H) is sent against its bin's max gmx, by the rule.
template <int kRule>
__device__ __forceinline__ bool send_rule(float gq, float hq, float gmx, float sf) {
    if (kRule == kRuleGradient) return gmx > 0.0f && (fabsf(hq) >= gmx || fabsf(gq) >= gmx);
    const float t = sf * fabsf(gq);
    return gmx > 0.0f && t >= gmx;
}

// Selection against the bin maxima (LDS bit patterns) of element e.
template <int kRule>
__device__ __forceinline__ bool selected(const AChunk &a, uint32_t e, float gq, float hq, uint32_t b, float sf,
                                         const uint32_t *gm) {
    const bool in = e < a.cnt;
    const float gmx = dev_u2f(gm[in ? b : 0u]);
    return in && send_rule<kRule>(gq, hq, gmx, sf);
}

template <int kRule>
__global__ __launch_bounds__(kBlock) void ada_max_kernel(PlanDev P, const float *__restrict__ dW,
                                                         const float *__restrict__ R, float sf,
                                                         AdaWs w) {
    const uint32_t c = blockIdx.x;
    const AChunk a = achunk_info(P, c);
    const uint32_t L = a.L;
    const float invL = 1.0f / static_cast<float>(L);
    const uint32_t nb = (a.cnt + L - 1) / L;
    __shared__ uint32_t gm[kChunk];
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gm[b] = 0u;
    float g[kRows][4], h[kRows][4];
    uint32_t bin[kRows][4];
    chunk_G<kRule>(a, R, dW, invL, sf - 1.0f, g, h, bin);
    __syncthreads();
    chunk_bin_max(a, g, bin, gm);
    __syncthreads();
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
            mine += selected<kRule>(a, row_elem(j) + q, g[j][q], h[j][q], bin[j][q], sf, gm) ? 1u : 0u;
    uint32_t total;
    (void)block_exclusive_scan(mine, &total);
    float *gout = w.gmax + a.bin_first;
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
                                                           float *__restrict__ seg_scale,
                                                           float *__restrict__ state_scale) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    const double *part = w.bpartial + seg.bgroup0;
    double S = block_pairwise_sum(seg.nbgroup, [&](uint64_t i) { return part[i]; });
    if (threadIdx.x == 0) {
        const float scale = static_cast<float>(S / static_cast<double>(seg.nbins));
        seg_scale[s] = scale;
        if (state_scale) state_scale[s] = scale;
    }
    // chunk prefixes: thread t owns a contiguous run of up to kScanRun
    // chunks (loads in flight together); one block scan per round
    constexpr uint32_t kScanRun = 32;
    const uint32_t *cc = w.ccount + seg.achunk0;
    uint32_t before = 0;
    for (uint32_t r0 = 0; r0 < seg.anchunk; r0 += kBlock * kScanRun) {
        const uint32_t nr = min(seg.anchunk - r0, kBlock * kScanRun);
        const uint32_t per = (nr + kBlock - 1) / kBlock;
        const uint32_t t0 = r0 + threadIdx.x * per;
        const uint32_t t1 = min(t0 + per, r0 + nr);
        uint32_t v[kScanRun];
#pragma unroll
        for (uint32_t u = 0; u < kScanRun; ++u) v[u] = cc[min(t0 + u, r0 + nr - 1)];
        uint32_t sum = 0;
#pragma unroll
        for (uint32_t u = 0; u < kScanRun; ++u)
            if (t0 + u < t1) sum += v[u];
        uint32_t tot;
        uint32_t run = before + block_exclusive_scan(sum, &tot);
#pragma unroll
        for (uint32_t u = 0; u < kScanRun; ++u) {
            if (t0 + u >= t1) break;
            w.cpre[seg.achunk0 + t0 + u] = run;
            run += v[u];
        }
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

template <int kRule>
__global__ __launch_bounds__(kBlock) void ada_apply_kernel(PlanDev P, const float *__restrict__ dW,
                                                           float *__restrict__ R, float sf, AdaWs w,
                                                           const uint32_t *__restrict__ seg_off,
                                                           const float *__restrict__ seg_scale,
                                                           uint32_t *__restrict__ out_idx,
                                                           float *__restrict__ out_val) {
    const uint32_t c = P.nachunk - 1 - blockIdx.x;
    const AChunk a = achunk_info(P, c);
    const uint32_t L = a.L;
    const float invL = 1.0f / static_cast<float>(L);
    const uint32_t nb = (a.cnt + L - 1) / L;
    __shared__ float gm[kChunk];
    const float *gin = w.gmax + a.bin_first;
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gm[b] = gin[b];
    float g[kRows][4], h[kRows][4];
    uint32_t bin[kRows][4];
    chunk_G<kRule>(a, R, dW, invL, sf - 1.0f, g, h, bin);
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
            flag[j][q] = in && send_rule<kRule>(g[j][q], h[j][q], gmx, sf);
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

// ---------------------------------------------------------- deferred mode
// The residual of an entry sent in step t is fl(G - copysign(scale_t, G)).
// In deferred mode R keeps G after the call and the state keeps which
// entries were sent and scale_t; the next call (or gc_adacomp_residual)
// applies exactly that expression to R before anything else reads it.  One
// dense pass then reads R and dW once and writes R once:
//   fold   one workgroup per chunk: R' = pending correction of R, G = R' + dW,
//          R <- G; bin maxima; selection bits (state) and sign bits
//          (workspace); count of selected entries
//   (binsum, scale, offsets as in the exact mode; scale also records scale_t)
//   emit   one workgroup per chunk: message (idx, copysign(scale, G)) from the
//          bits, in index order at its final slot

// R' for the element at bit `bit` of the thread's word.
__device__ __forceinline__ float pending(float r, uint32_t held, int bit, float pscale) {
    return ((held >> bit) & 1u) ? r - copysignf(pscale, r) : r;
}

template <int kRule>
__global__ __launch_bounds__(kBlock) void ada_fold_kernel(PlanDev P, const float *__restrict__ dW,
                                                          float *__restrict__ R, float sf, AdaWs w,
                                                          AdaState S) {
    const uint32_t c = blockIdx.x;
    const AChunk a = achunk_info(P, c);
    const uint32_t L = a.L;
    const float invL = 1.0f / static_cast<float>(L);
    const uint32_t nb = (a.cnt + L - 1) / L;
    __shared__ uint32_t gm[kChunk];
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gm[b] = 0u;
    const BufRsrc rr = chunk_buf(R + a.lo, a.cnt), rd = chunk_buf(dW + a.lo, a.cnt);
    const size_t word = size_t(c) * kBlock + threadIdx.x;
    const uint32_t held = S.sel[word];
    const float pscale = S.scale[a.s];
    const float s1 = sf - 1.0f;
    float g[kRows][4], h[kRows][4];
    uint32_t bin[kRows][4];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        float r[4], d[4];
        load4(rr, row_elem(j), r);
        load4(rd, row_elem(j), d);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            g[j][q] = pending(r[q], held, 4 * j + q, pscale) + d[q];
            if (kRule == kRuleGradient) h[j][q] = g[j][q] + s1 * d[q];
            bin[j][q] = div_small(row_elem(j) + q, L, invL);
        }
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) store4(rr, row_elem(j), g[j]);
    __syncthreads();
    chunk_bin_max(a, g, bin, gm);
    __syncthreads();
    uint32_t bits = 0, signs = 0, mine = 0;
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool f = selected<kRule>(a, row_elem(j) + q, g[j][q], h[j][q], bin[j][q], sf, gm);
            bits |= uint32_t(f) << (4 * j + q);
            signs |= (dev_f2u(g[j][q]) >> 31) << (4 * j + q);
            mine += f ? 1u : 0u;
        }
    S.sel[word] = static_cast<uint16_t>(bits);
    w.sign[word] = static_cast<uint16_t>(signs);
    uint32_t total;
    (void)block_exclusive_scan(mine, &total);
    float *gout = w.gmax + a.bin_first;
    for (uint32_t b = threadIdx.x; b < nb; b += kBlock) gout[b] = dev_u2f(gm[b]);
    if (threadIdx.x == 0) w.ccount[c] = total;
}

// Thread t takes the 16 consecutive elements [16 t, 16 t + 16) of the chunk.
// In the fold's layout element 1024 j + 4 t' + q is bit 4 j + q of word t',
// so they are the 4-bit groups at 4 j (j = t / 64) of the four words
// 4 (t mod 64) .. + 3: one 8-byte load each for the selection and sign bits.
// One block scan orders the chunk's entries; they are staged in LDS as
// (element | sign << 15) and written out with coalesced stores.
__device__ __forceinline__ uint32_t gather16(uint64_t words, uint32_t j) {
    uint32_t v = 0;
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) v |= static_cast<uint32_t>((words >> (16 * k + 4 * j)) & 0xFu) << (4 * k);
    return v;
}

__global__ __launch_bounds__(kBlock) void ada_emit_kernel(PlanDev P, AdaWs w, AdaState S,
                                                          const uint32_t *__restrict__ seg_off,
                                                          const float *__restrict__ seg_scale,
                                                          uint32_t *__restrict__ out_idx,
                                                          float *__restrict__ out_val) {
    const uint32_t c = blockIdx.x;
    const ChunkRec rec = P.achunk_rec[c];
    const uint32_t s = rec.z;
    const size_t w4 = size_t(c) * kBlock + 4 * (threadIdx.x & (kWave - 1));
    const uint64_t selw = *reinterpret_cast<const uint64_t *>(S.sel + w4);
    const uint64_t sgnw = *reinterpret_cast<const uint64_t *>(w.sign + w4);
    const uint32_t j = threadIdx.x / kWave;
    const uint32_t bits = gather16(selw, j), signs = gather16(sgnw, j);
    const float scale = seg_scale[s];
    const uint32_t base = seg_off[s] + w.cpre[c];
    const uint32_t count = w.ccount[c];
    __shared__ uint16_t ent[kChunk];
    uint32_t total;
    uint32_t slot = block_exclusive_scan(static_cast<uint32_t>(__popc(bits)), &total);
#pragma unroll
    for (uint32_t i = 0; i < 16; ++i)
        if ((bits >> i) & 1u) ent[slot++] = static_cast<uint16_t>((16 * threadIdx.x + i) | (((signs >> i) & 1u) << 15));
    __syncthreads();
    const uint32_t n = min(total, count);  // equal unless the inputs were tampered with
    for (uint32_t k = threadIdx.x; k < n; k += kBlock) {
        const uint32_t v = ent[k];
        // non-temporal stores: measured faster over the whole step, although pack
        // and decode read the message next
        __builtin_nontemporal_store(static_cast<uint32_t>(rec.x + (v & 0x7FFFu)), out_idx + base + k);
        __builtin_nontemporal_store(copysignf(scale, (v >> 15) ? -1.0f : 1.0f), out_val + base + k);
    }
}

// R_out <- the exact residual held by (R, state), segment elements only.
__global__ __launch_bounds__(kBlock) void ada_residual_kernel(PlanDev P, const float *__restrict__ R,
                                                              AdaState S, float *__restrict__ R_out) {
    const uint32_t c = blockIdx.x;
    const AChunk a = achunk_info(P, c);
    const BufRsrc rr = chunk_buf(R + a.lo, a.cnt), ro = chunk_buf(R_out + a.lo, a.cnt);
    const uint32_t held = S.sel[size_t(c) * kBlock + threadIdx.x];
    const float pscale = S.scale[a.s];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        float r[4];
        load4(rr, row_elem(j), r);
#pragma unroll
        for (int q = 0; q < 4; ++q) r[q] = pending(r[q], held, 4 * j + q, pscale);
        store4(ro, row_elem(j), r);
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

extern "C" uint64_t gc_adacomp_message_cap(const gc_plan *plan) { return plan ? plan->seg_elems : 0; }

extern "C" size_t gc_adacomp_state_bytes(const gc_plan *plan) {
    if (!plan) return 0;
    size_t b = 0;
    (void)ada_state_layout(plan, nullptr, &b);
    return b;
}

template <int kRule>
static void adacomp_launch(const gc_plan *plan, const PlanDev &P, AdaWs w, const float *dW, float *R, void *state,
                    float sf, gc_sparse *out, hipStream_t stream) {
    if (state) {
        const AdaState S = ada_state_layout(plan, state, nullptr);
        GC_LAUNCH("ada_fold", stream, ada_fold_kernel<kRule><<<plan->nachunk, kBlock, 0, stream>>>(P, dW, R, sf, w, S));
        GC_LAUNCH("ada_binsum", stream, ada_binsum_kernel<<<plan->nbgroup, kBlock, 0, stream>>>(P, w));
        GC_LAUNCH("ada_scale", stream, ada_scale_kernel<<<plan->nseg, kBlock, 0, stream>>>(P, w, out->seg_scale, S.scale));
        GC_LAUNCH("ada_offsets", stream, ada_offsets_kernel<<<1, kBlock, 0, stream>>>(plan->nseg, w, out->seg_off));
        GC_LAUNCH("ada_emit", stream, ada_emit_kernel<<<plan->nachunk, kBlock, 0, stream>>>(
            P, w, S, out->seg_off, out->seg_scale, out->idx, out->val));
    } else {
        GC_LAUNCH("ada_max", stream, ada_max_kernel<kRule><<<plan->nachunk, kBlock, 0, stream>>>(P, dW, R, sf, w));
        GC_LAUNCH("ada_binsum", stream, ada_binsum_kernel<<<plan->nbgroup, kBlock, 0, stream>>>(P, w));
        GC_LAUNCH("ada_scale", stream, ada_scale_kernel<<<plan->nseg, kBlock, 0, stream>>>(P, w, out->seg_scale, nullptr));
        GC_LAUNCH("ada_offsets", stream, ada_offsets_kernel<<<1, kBlock, 0, stream>>>(plan->nseg, w, out->seg_off));
        GC_LAUNCH("ada_apply", stream, ada_apply_kernel<kRule><<<plan->nachunk, kBlock, 0, stream>>>(
            P, dW, R, sf, w, out->seg_off, out->seg_scale, out->idx, out->val));
    }
}

static gc_status adacomp_compress(const char *fn, const gc_plan *plan, const float *dW, float *R, void *state,
                           size_t state_bytes, float scale_factor, int rule, gc_sparse *out, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
    const std::string f(fn);
    if (!plan) return set_error(GC_EINVAL, f + ": plan is null");
    if (!dW || !R) return set_error(GC_EINVAL, f + ": dW and R must be non-null");
    if (!out || !out->idx || !out->val || !out->seg_off || !out->seg_scale)
        return set_error(GC_EINVAL, f + ": out and its idx, val, seg_off, seg_scale must be non-null");
    if (!(scale_factor >= 1.0f) || std::isinf(scale_factor))
        return set_error(GC_EINVAL, f + ": scale_factor must be finite and >= 1");
    if (rule != GC_ADACOMP_RULE_RESIDUAL && rule != GC_ADACOMP_RULE_GRADIENT)
        return set_error(GC_EINVAL, f + ": rule must be GC_ADACOMP_RULE_RESIDUAL or GC_ADACOMP_RULE_GRADIENT");
    if (out->cap < plan->seg_elems)
        return set_error(GC_ECAPACITY, f + ": out->cap below gc_adacomp_message_cap");
    size_t need = adacomp_workspace_bytes(plan);
    if (!ws || ws_bytes < need) return set_error(GC_ECAPACITY, f + ": workspace smaller than gc_plan_workspace_bytes");
    if (reinterpret_cast<uintptr_t>(ws) % 256) return set_error(GC_EINVAL, f + ": workspace must be 256-byte aligned");
    if (state && state_bytes < gc_adacomp_state_bytes(plan))
        return set_error(GC_ECAPACITY, f + ": state smaller than gc_adacomp_state_bytes");
    if (state && reinterpret_cast<uintptr_t>(state) % 256)
        return set_error(GC_EINVAL, f + ": state must be 256-byte aligned");
    PlanDev P;
    gc_status st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    AdaWs w = ada_layout(plan, ws, nullptr);
    if (rule == GC_ADACOMP_RULE_GRADIENT)
        adacomp_launch<kRuleGradient>(plan, P, w, dW, R, state, scale_factor, out, stream);
    else
        adacomp_launch<kRuleResidual>(plan, P, w, dW, R, state, scale_factor, out, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, (f + " launch").c_str());
    return GC_OK;
}

extern "C" gc_status gc_adacomp_compress(const gc_plan *plan, const float *dW, float *R, void *state,
                                         size_t state_bytes, float scale_factor, gc_sparse *out,
                                         void *ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    return adacomp_compress("gc_adacomp_compress", plan, dW, R, state, state_bytes, scale_factor,
                            GC_ADACOMP_RULE_RESIDUAL, out, ws, ws_bytes, stream);
}

extern "C" gc_status gc_adacomp_compress_ex(const gc_plan *plan, const float *dW, float *R, void *state,
                                            size_t state_bytes, const gc_adacomp_options *opt,
                                            gc_sparse *out, void *ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    if (!opt) return set_error(GC_EINVAL, "gc_adacomp_compress_ex: opt is null");
    if (opt->reserved[0] || opt->reserved[1])
        return set_error(GC_EINVAL, "gc_adacomp_compress_ex: reserved fields must be 0");
    return adacomp_compress("gc_adacomp_compress_ex", plan, dW, R, state, state_bytes, opt->scale_factor,
                            opt->rule, out, ws, ws_bytes, stream);
}

extern "C" gc_status gc_adacomp_residual(const gc_plan *plan, const float *R, const void *state,
                                         size_t state_bytes, float *R_out, hipStream_t stream) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_adacomp_residual: plan is null");
    if (!R || !R_out) return set_error(GC_EINVAL, "gc_adacomp_residual: R and R_out must be non-null");
    const uint64_t bytes = plan->n_total * sizeof(float);
    const uintptr_t r0 = reinterpret_cast<uintptr_t>(R), o0 = reinterpret_cast<uintptr_t>(R_out);
    if (bytes && r0 < o0 + bytes && o0 < r0 + bytes)
        return set_error(GC_EINVAL, "gc_adacomp_residual: R_out must not overlap R");
    if (state && state_bytes < gc_adacomp_state_bytes(plan))
        return set_error(GC_ECAPACITY, "gc_adacomp_residual: state smaller than gc_adacomp_state_bytes");
    if (state && reinterpret_cast<uintptr_t>(state) % 256)
        return set_error(GC_EINVAL, "gc_adacomp_residual: state must be 256-byte aligned");
    PlanDev P;
    gc_status st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    // elements outside every segment carry over unchanged
    hipError_t e = hipMemcpyAsync(R_out, R, bytes, hipMemcpyDeviceToDevice, stream);
    if (e != hipSuccess) return hip_error(e, "gc_adacomp_residual copy");
    if (state) {
        const AdaState S = ada_state_layout(plan, const_cast<void *>(state), nullptr);
        GC_LAUNCH("ada_residual", stream, ada_residual_kernel<<<plan->nachunk, kBlock, 0, stream>>>(P, R, S, R_out));
    }
    e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_adacomp_residual launch");
    return GC_OK;
}
