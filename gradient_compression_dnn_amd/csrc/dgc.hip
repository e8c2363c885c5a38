// Top-k selection on gfx950 for DGC and Slim-DP.
//   DGC ("Deep Gradient Compression", Lin et al., §3.1-§3.3, §5, §6, App. B,
//   C, D): local clipping, momentum correction (vanilla or Nesterov), top-k by
//   radix select on |V| bit patterns (exact, or from a sampled threshold with
//   a hierarchical exact fallback), ordered compaction, momentum factor
//   masking.
//   Slim-DP ("Slim-DP", §3): the core (top-k by significance) and the
//   explorer (top-k of random keys outside the core) through the same
//   kernels, with the key source chosen by a template mode.
//
// Two launch sequences.  Selection at the pages' densities (every tensor of
// more than one chunk keeps at most 1/512 of its entries) takes the exact
// path described further down: norm, prepare, update, collect, select,
// emit (the sampled threshold replaces prepare by its sample and quantile
// and adds sbase).  Denser selections (warm-up, Slim-DP's core and
// explorer, the sampled threshold on such plans) take the candidate kernels
// below.  Chunk kernels run
// one workgroup (or one wave) per 4096-element chunk of a segment; segment
// kernels one workgroup per segment.  Chunk kernels hand results to segment
// kernels through global memory at kernel boundaries only (no cross-
// workgroup fences, which on gfx950 write back the XCD's L2).  The
// candidate sequence:
//   norm    (chunk, clip only) pairwise fp64 sum of G^2 over the chunk
//   prep    (segment) clear the segment's histograms; finish the pairwise
//           tree over the chunk sums and set the clip factor
//   sample  (chunk) the ranked value of 32 contiguous elements in up to 512
//           chunks per segment, computed as the update will compute it
//   bound   (segment) from the sample, a key Lkey that the k-th largest key
//           almost surely reaches (the page estimates its threshold from a
//           sample, §5)
//   update  (chunk) U <- fl(fl(m U) + fl(c G)); V <- fl(V + U) (or the mode's
//           value); LDS histogram of digit 1, flushed with global atomics;
//           entries with key at or above Lkey staged in index order at the
//           chunk's own offset
//   select1 (segment) digit 1 of the k-th largest key, d1; if fewer than k
//           entries were staged, the k-th largest key is below Lkey, the
//           staging missed candidates and the segment is re-staged
//   stage   (chunk) histogram digit 2 of the staged entries in the boundary
//           bucket; for a re-staged segment, re-read V and stage digit 1 >= d1
//           (Slim-DP's core uses stagew, 32 chunks per workgroup, for the
//           histogram)
//   select2 (segment) digit 2
//   refine  (chunk) histogram digit 3 of staged entries in the boundary bucket
//   select3 (segment) threshold key T, count above it, ties to send
//   count   (chunk) staged keys > T and == T
//   scan    (segment) message slot and tie quota of every chunk
//   emit    (chunk) write (idx, value) in index order; DGC zeroes U and V
//           there, Slim-DP's core writes its bitmap words
// Staged entries below d1 are never counted or sent (their keys are below T),
// so the looser staging changes no result.
//
// Sampled selection replaces sample + bound by
//   ssample (chunk) V' at the sample positions (one 32-entry block per window
//           of 32 P entries), keys stored at the segment's staging offset
//   squant  (segment) the estimate: the r-th largest sample key,
//           r = ceil(S k / n), by a three-digit LDS radix select (or, for
//           segments with more than 32,768 samples, qhist/qfind pairs with 32
//           workgroups per segment)
// and the update stages exactly the keys at or above the estimate.  The
// segment then sends all of them when they fit the budget min(n, over k),
// and otherwise the exact top-k among them: on the exact path's kernels
// (collect and select as for exact selection, select settling each
// segment's count), or with the candidate kernels (select1 marks "all"
// segments, which skip stage, refine and the later selects).  sbase (one
// workgroup) lays the segments' variable-size outputs end to end.
#include <algorithm>
#include <cmath>
#include <string>

#include "gc_internal.hpp"

namespace gc {

namespace {

struct SegState {
    float clip;
    uint32_t d1, above1, d2, above2, T, gt, need_eq;
    uint32_t Lkey;  // staging bound on the key, from the sample
    uint32_t redo;  // fewer than k staged: re-stage the segment from V
    uint32_t all;   // sampled selection: every staged entry is sent
    uint32_t sent;  // entries the segment sends
    uint32_t base;  // first message slot of the segment
    uint32_t qrank, qprefix;  // sampled selection: quantile search state
    uint32_t fshift;          // exact path: fine bins above Lkey are 2^fshift keys wide
    uint32_t hkey;            // sampled selection on the exact path: the largest sample key
};

// What the selection kernels rank (the key is the magnitude bits of a value):
//   kVanilla, kNesterov  DGC: V after the momentum-corrected update (U, V
//                        updated in place; sent entries masked)
//   kSignif              Slim-DP core: S = |w| + c |g| (read only)
//   kExplore             Slim-DP explorer: a Philox key outside the core, 0
//                        inside it (read only; the message carries delta)
enum Mode { kVanilla = 0, kNesterov = 1, kSignif = 2, kExplore = 3 };

struct Src {
    const float *G;  // DGC: gradient; kSignif: g; kExplore: delta
    float *U;        // DGC: momentum; kSignif: w (read only)
    float *V;        // DGC: accumulator
    float m;         // DGC: momentum; kSignif: c
    uint32_t k0, k1, slo, shi;  // kExplore: Philox key (seed) and step
    uint32_t *mask;  // kSignif: core bitmap out; kExplore: core bitmap in
};

// Momentum correction (§3.2; App. B and D).  Vanilla: U <- m U + G',
// V <- V + U.  Nesterov: U <- m U + G', V <- V + (m U + G') with the updated U,
// the Nesterov step direction accumulated in place of being applied.  One
// rounding per operation, in this order.
template <int kMode>
__device__ __forceinline__ void momentum_update(float m, float gc, float &u, float &v) {
    float un = m * u;
    un = un + gc;
    u = un;
    if (kMode == kNesterov) {
        float d = m * un;
        d = d + gc;
        v = v + d;
    } else {
        v = v + un;
    }
}

// Sample of a segment: in every stride-th chunk (at most kSampleChunks
// chunks), kSamples contiguous elements starting at a per-chunk offset
// (spread over the chunk so that strided tensor layouts are not always
// sampled at the same columns).
constexpr uint32_t kSamples = 32;
constexpr uint32_t kSampleChunks = 512;
__device__ __forceinline__ uint32_t sample_offset(uint32_t c, uint32_t cnt) {
    return cnt == uint32_t(kChunk) ? 128u * ((c * 13u) & 31u) : 0u;
}
__device__ __forceinline__ uint32_t sample_stride(uint32_t dnchunk) {
    return (dnchunk + kSampleChunks - 1) / kSampleChunks;
}

// Digit-1 and digit-2 histograms are kept in kHistRep replicas per segment,
// picked by workgroup (update) or chunk (stage): concurrent global atomics on
// one address serialize, and a large segment is covered by hundreds of
// workgroups.  The select kernels add the replicas.
constexpr uint32_t kHistRep = 16;
static_assert(kHist1 == kHist2, "the sample bound reuses one LDS histogram for digits 1 and 2");

// Exact path (DGC, exact selection, and sampled selection on its kernels):
// the staged keys are binned in kFineBins bins above the staging bound Lkey,
// Lkey alone in the first and 2^fshift keys in each of the others (the last
// bin takes every key above the range).
constexpr uint32_t kFineBins = kHist1;
// Its fine histogram of the staged keys (the update adds each key) is kept
// in the segment's digit-1 area; the keys in T's fine bin are gathered into
// an LDS list of at most kXListCap keys.
constexpr uint32_t kXListCap = 8192;

struct DgcWs {
    uint32_t *hist1, *hist2, *hist3;
    SegState *st;
    double *partial;
    uint32_t *ccount, *cgt, *ceq, *cout, *ctake;
    uint32_t *sidx;
    float *sval;
    uint32_t *skey;  // [ndchunk][kSamples] key of the sampled V'
    uint32_t *qhist; // [nseg][kHist1] sample-quantile histogram (sampled selection)
    // exact path
    uint4 *crec;     // [ndchunk] emit record: first slot, end slot, T, staged count | quota << 16
    uint32_t *cpack; // [ndchunk] per-chunk counts (two u16) for segments past the LDS tables
    // the call's top-k count per segment: ceil(n_s * knum / kden) in [1, n_s],
    // or the plan's k when kden is 0
    uint32_t knum, kden;
};

// k_s of a segment for this call (warm-up densities are set per call).
__host__ __device__ __forceinline__ uint32_t seg_topk(uint32_t len, uint32_t plan_k, uint32_t knum, uint32_t kden) {
    if (kden == 0) return plan_k;
    const uint64_t k = (uint64_t(len) * knum + kden - 1) / kden;
    return k < 1 ? 1u : (k > len ? len : static_cast<uint32_t>(k));
}
__device__ __forceinline__ uint32_t seg_k(const SegDev &seg, const DgcWs &w) {
    return seg_topk(seg.len, seg.k, w.knum, w.kden);
}
// The exact path's fine histogram of segment s.
__device__ __forceinline__ uint32_t *xtables(const DgcWs &w, uint32_t s) {
    return w.hist1 + size_t(s) * kHistRep * kHist1;
}
// Fine bins of the staged keys (all >= Lkey): bin 0 holds Lkey itself, bin
// b >= 1 the 2^fs keys from Lkey + 1 + (b - 1) 2^fs, and the last bin every
// key above the range.  Lkey has a bin of its own because keys crowd there
// (a tensor of zeros has Lkey = 0): T in bin 0 is then known without
// listing the bin's keys, however wide the other bins are.
__device__ __forceinline__ uint32_t fine_bin(uint32_t key, uint32_t Lkey, uint32_t fs) {
    return key == Lkey ? 0u : min(((key - Lkey - 1u) >> fs) + 1u, kFineBins - 1);
}
// The smallest key of fine bin b (b below the last).
__device__ __forceinline__ uint32_t fine_lo(uint32_t b, uint32_t Lkey, uint32_t fs) {
    return b == 0 ? Lkey : Lkey + 1u + ((b - 1u) << fs);
}
// Width 2^fs of the fine bins: the narrowest that brings Hkey into a bin
// below the last.
__device__ __forceinline__ uint32_t fine_shift(uint32_t Lkey, uint32_t Hkey) {
    uint32_t fs = 0;
    if (Hkey > Lkey)
        while (((Hkey - Lkey - 1u) >> fs) > kFineBins - 3) ++fs;
    return fs;
}

DgcWs dgc_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    DgcWs w{};
    w.hist1 = c.take<uint32_t>(size_t(kHist1) * kHistRep * p->nseg);
    w.hist2 = c.take<uint32_t>(size_t(kHist2) * kHistRep * p->nseg);
    w.hist3 = c.take<uint32_t>(size_t(kHist3) * p->nseg);
    w.st = c.take<SegState>(p->nseg);
    w.partial = c.take<double>(p->ndchunk);
    w.ccount = c.take<uint32_t>(p->ndchunk);
    w.cgt = c.take<uint32_t>(p->ndchunk);
    w.ceq = c.take<uint32_t>(p->ndchunk);
    w.cout = c.take<uint32_t>(p->ndchunk);
    w.ctake = c.take<uint32_t>(p->ndchunk);
    // staging: at a chunk's first element (the candidate kernels), or in the
    // chunk's own 4096-entry slot (the exact path), whichever is larger
    const size_t nstage = std::max<size_t>(p->n_total, size_t(p->ndchunk) << kChunkLog2);
    w.sidx = c.take<uint32_t>(nstage);
    w.sval = c.take<float>(nstage);
    w.skey = c.take<uint32_t>(size_t(p->ndchunk) * kSamples);
    w.qhist = c.take<uint32_t>(size_t(p->nseg) * kHist1);
    w.crec = c.take<uint4>(p->ndchunk);
    w.cpack = c.take<uint32_t>(p->ndchunk);
    if (bytes) *bytes = c.used + 256;
    return w;
}

struct ChunkInfo {
    uint32_t s;
    SegDev seg;
    uint64_t lo;   // first flat element of the chunk
    uint32_t cnt;  // elements in the chunk
};

__device__ __forceinline__ uint32_t mag_key(float v) { return dev_f2u(v) & 0x7FFFFFFFu; }

// Global histogram increments aggregated over a wave.  add() is called by
// the whole wave (full exec mask) with a wave-uniform histogram: the lanes
// that add to one bin become one count, and counts to the same bin of the
// same histogram accumulate over calls until another bin comes or flush()
// (lane 0 issues the atomic).  Keys that crowd into one bin (a tensor of
// zeros, a constant tensor) then cost one atomic per run of calls instead of
// one per key: one global address takes about one atomic per 10 ns, so a
// 20M-element tensor of zeros took 235 ms with an atomic per key.
// An LDS histogram increment by the whole wave (full exec mask): when every
// adding lane has the same bin (a sample of zeros), one atomic adds them all,
// which LDS would otherwise take one lane at a time; else each lane adds its
// own.  (Used by prepare, where it took a tensor of zeros from 38 to 18 us;
// in the sampled threshold's quantile its extra tests cost more than they
// saved.)
__device__ __forceinline__ void lds_hist_add(uint32_t *h, bool f, uint32_t b) {
    const uint64_t m = __ballot(f);
    if (m == 0) return;
    const int first = __builtin_ctzll(m);
    const uint32_t b0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), first));
    if (__ballot(f && b != b0) == 0) {
        if (lane_id() == first) atomicAdd(&h[b0], static_cast<uint32_t>(__popcll(m)));
    } else if (f) {
        atomicAdd(&h[b], 1u);
    }
}

struct WaveHist {
    uint32_t *h = nullptr;
    uint32_t bin = 0, cnt = 0;
    __device__ __forceinline__ void flush() {
        if (cnt != 0 && lane_id() == 0) atomicAdd(h + bin, cnt);
        cnt = 0;
    }
    __device__ __forceinline__ void add(uint32_t *hist, bool f, uint32_t b) {
        uint64_t todo = __ballot(f);
        while (todo) {
            const int leader = __builtin_ctzll(todo);
            const uint32_t lb = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), leader));
            const uint64_t same = __ballot(f && b == lb) & todo;
            if (hist != h || lb != bin) {
                flush();
                h = hist;
                bin = lb;
            }
            cnt += static_cast<uint32_t>(__popcll(same));
            todo &= ~same;
        }
    }
};

// Slim-DP significance (Slim-DP §3.2, a weighted sum of the magnitudes of
// the parameter and of its gradient): fl(|w| + fl(c |g|)).
__device__ __forceinline__ float significance(float w, float g, float c) {
    const float cg = c * fabsf(g);
    return fabsf(w) + cg;
}

// Slim-DP explorer values of the 4 entries [j0, j0 + 4) of segment s (j0 a
// multiple of 4): the key r >> 1 | 1 of Philox4x32-10 word j % 4 (counter
// (j / 4, s, step), key = seed) as float bits, 0 for core entries.  `words`
// bounds the bitmap read (lanes past the segment end read its last word).
__device__ __forceinline__ void explore_values(const Src &a, const SegDev &seg, uint32_t s, uint32_t j0,
                                               float (&v)[4]) {
    const uint4 r = philox4x32_10(make_uint4(j0 >> 2, s, a.slo, a.shi), a.k0, a.k1);
    const uint32_t words = (seg.len + 31) / 32;
    const uint32_t mw = a.mask[seg.mbase + min(j0 >> 5, words - 1)] >> (j0 & 31);
    const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = dev_u2f(((mw >> q) & 1u) ? 0u : ((rw[q] >> 1) | 1u));
}

// Chunk geometry with the segment record cached while the chunks stay in one
// segment.
struct ChunkWalker {
    uint32_t s = 0;
    SegDev seg{};
    __device__ ChunkInfo at(const PlanDev &P, uint32_t c) {
        if (c < seg.dchunk0 || c >= seg.dchunk0 + seg.dnchunk) {
            s = P.dchunk_seg[c];
            seg = P.seg[s];
        }
        ChunkInfo ci;
        ci.s = s;
        ci.seg = seg;
        const uint32_t pos = c - seg.dchunk0;
        ci.lo = seg.off + (uint64_t(pos) << kChunkLog2);
        const uint32_t rem = seg.len - (pos << kChunkLog2);
        ci.cnt = rem < uint32_t(kChunk) ? rem : uint32_t(kChunk);
        return ci;
    }
};

// Dense kernels: workgroup b walks chunks [first, last), a contiguous range
// (one chunk when the grid has a workgroup per chunk), so consecutive chunks
// mostly share a segment.
__device__ __forceinline__ void chunk_range(uint32_t nchunk, uint32_t *first, uint32_t *last) {
    const uint32_t per = (nchunk + gridDim.x - 1) / gridDim.x;
    *first = blockIdx.x * per;
    *last = min(*first + per, nchunk);
}

// ------------------------------------------------------------------ norm
// One workgroup per chunk.  Lane l of wave w holds elements
// [1024 j + 256 w + 4 l, +4) of row j: its (x0^2 + x1^2) + (x2^2 + x3^2) is a
// level-2 node of the pairwise tree.  The lane nodes go to LDS in index
// order; thread t then owns the 4 consecutive level-2 nodes [4 t, 4 t + 4)
// (a 16-element subtree), and the 256 thread sums are combined by
// block_tree_sum into the chunk's level-12 node.  (A persistent grid striding
// over the chunks, each workgroup loading its next chunk during the tree,
// measured 1-2 us slower on the DeepSpeech sizes: the resident workgroups
// already keep enough loads in flight.)
__global__ __launch_bounds__(kBlock) void dgc_norm_kernel(PlanDev P, const float *__restrict__ G,
                                                          DgcWs w) {
    const uint32_t c = blockIdx.x;
    __shared__ double node[kChunk / 4];  // level-2 nodes of the chunk, in order
    float x[kRows][4];
    const ChunkRec rec = P.dchunk_rec[c];
    const BufRsrc rg = chunk_buf(G + rec.x, rec.y);
#pragma unroll
    for (int j = 0; j < kRows; ++j) load4(rg, row_elem(j), x[j]);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        double a[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const double d = static_cast<double>(x[j][q]);
            a[q] = d * d;
        }
        node[j * kBlock + threadIdx.x] = (a[0] + a[1]) + (a[2] + a[3]);
    }
    __syncthreads();
    // four consecutive level-2 nodes: the 16-element level-4 node of thread t
    const double t0 = node[4 * threadIdx.x] + node[4 * threadIdx.x + 1];
    const double t1 = node[4 * threadIdx.x + 2] + node[4 * threadIdx.x + 3];
    const double chunk_sum = block_tree_sum(t0 + t1);
    if (threadIdx.x == 0) w.partial[c] = chunk_sum;
}

// ------------------------------------------------------------------ prep
// fine (sampled selection on the exact path): only the fine histogram is
// cleared, and the segment state the exact path's prepare sets is set here.
__global__ __launch_bounds__(kBlock) void dgc_prep_kernel(PlanDev P, DgcWs w, int use_clip,
                                                          float thr, int zero_q, int fine) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    if (zero_q)
        for (int i = threadIdx.x; i < kHist1; i += kBlock) w.qhist[size_t(s) * kHist1 + i] = 0u;
    if (fine) {
        uint4 *x4 = reinterpret_cast<uint4 *>(xtables(w, s));
        for (int i = threadIdx.x; i < int(kFineBins / 4); i += kBlock) x4[i] = make_uint4(0u, 0u, 0u, 0u);
    } else {
        uint4 *h4 = reinterpret_cast<uint4 *>(w.hist1 + size_t(s) * kHistRep * kHist1);
        for (int i = threadIdx.x; i < int(kHistRep * kHist1 / 4); i += kBlock) h4[i] = make_uint4(0u, 0u, 0u, 0u);
        h4 = reinterpret_cast<uint4 *>(w.hist2 + size_t(s) * kHistRep * kHist2);
        for (int i = threadIdx.x; i < int(kHistRep * kHist2 / 4); i += kBlock) h4[i] = make_uint4(0u, 0u, 0u, 0u);
        uint32_t *h = w.hist3 + size_t(s) * kHist3;
        for (int i = threadIdx.x; i < kHist3; i += kBlock) h[i] = 0u;
    }
    float cl = 1.0f;
    if (use_clip) {
        const double *part = w.partial + seg.dchunk0;
        double S = block_pairwise_sum(seg.dnchunk, [&](uint64_t g) { return part[g]; });
        double norm = sqrt(S);
        if (norm > static_cast<double>(thr)) cl = static_cast<float>(static_cast<double>(thr) / norm);
    }
    if (threadIdx.x == 0) {
        w.st[s].clip = cl;
        w.st[s].hkey = 0u;  // the sample's largest key, by atomicMax over the qhist workgroups
        if (fine) {
            w.st[s].sent = seg.k;
            w.st[s].base = seg.kbase;
            w.st[s].redo = 0u;
            w.st[s].all = 0u;
        }
    }
}

// ---------------------------------------------------------------- sample
// Half a wave per chunk: in a sampled chunk, lane l < min(32, cnt) computes
// V' of element sample_offset + l with the update's own arithmetic and
// records its key (plain stores: no atomics).
template <int kMode>
__global__ __launch_bounds__(kBlock) void dgc_sample_kernel(PlanDev P, Src a, DgcWs w) {
    const uint32_t c = (blockIdx.x * kWaves + wave_id()) * 2u + (uint32_t(lane_id()) >> 5);
    const uint32_t l = lane_id() & 31;
    if (c >= P.ndchunk) return;
    const ChunkRec rec = P.dchunk_rec[c];
    const uint32_t cnt = rec.y;
    const SegDev seg = P.seg[rec.z];
    if ((c - seg.dchunk0) % sample_stride(seg.dnchunk) != 0 || l >= min(kSamples, cnt)) return;
    const uint32_t jc = sample_offset(c, cnt) + l;  // inside the chunk
    const uint64_t e = uint64_t(rec.x) + jc;
    float vn;
    if (kMode == kSignif) {
        vn = significance(a.U[e], a.G[e], a.m);
    } else if (kMode == kExplore) {
        const uint32_t j = (rec.w << kChunkLog2) + jc;
        float v4[4];
        explore_values(a, seg, rec.z, j & ~3u, v4);
        vn = v4[j & 3];
    } else {
        const float clip = w.st[rec.z].clip;
        const float gc = clip * a.G[e];
        float un = a.U[e];
        vn = a.V[e];
        momentum_update<kMode>(a.m, gc, un, vn);
    }
    w.skey[size_t(c) * kSamples + l] = mag_key(vn);
}

// --------------------------------------------------------------- ssample
// Sampled selection's sample: window w of a segment covers entries
// [32 P w, 32 P (w + 1)); its block is the 32 entries from
// 32 P w + sample_block_offset(w, P), those past the segment end excluded.
// Only the last window can be cut, so the keys of sample j = 32 w + l form
// the contiguous range [0, S) at the segment's staging offset (j never
// exceeds the sampled position, so it stays inside the segment).  One wave
// per chunk, half a wave per window whose block starts in the chunk.
__device__ __forceinline__ uint32_t sample_block_offset(uint32_t w, uint32_t period) {
    return 32u * ((w * 2654435769u) % period);  // Fibonacci hash of the window, mod 2^32
}

template <int kMode>
__global__ __launch_bounds__(kBlock) void dgc_ssample_kernel(PlanDev P, Src a, uint32_t period, DgcWs w) {
    const uint32_t c = blockIdx.x * kWaves + wave_id();
    if (c >= P.ndchunk) return;
    const ChunkRec rec = P.dchunk_rec[c];
    const uint32_t cnt = rec.y, s = rec.z;
    const SegDev seg = P.seg[s];
    const uint64_t win = 32ull * period;
    const uint64_t pos0 = uint64_t(rec.w) << kChunkLog2, pos1 = pos0 + cnt;
    const uint64_t w0 = pos0 / win, w1 = (pos1 - 1) / win;
    const float clip = w.st[s].clip;
    const uint32_t l = lane_id() & 31;
    for (uint64_t wb = w0; wb <= w1; wb += 2) {
        const uint64_t wi = wb + (uint32_t(lane_id()) >> 5);
        if (wi > w1) continue;
        const uint64_t start = wi * win + sample_block_offset(static_cast<uint32_t>(wi), period);
        const uint64_t p = start + l;
        if (start < pos0 || start >= pos1 || p >= seg.len) continue;
        const uint64_t e = seg.off + p;
        const float gc = clip * a.G[e];
        float un = a.U[e], vn = a.V[e];
        momentum_update<kMode>(a.m, gc, un, vn);
        w.sidx[seg.off + wi * 32 + l] = mag_key(vn);
    }
}

// ---------------------------------------------------------------- squant
// The estimate of the k-th largest key: the r-th largest of the S sample
// keys, r = ceil(S k / n) (u64 arithmetic), by radix select over the 11, 11
// and 9-bit digits with an LDS histogram per digit (keys re-read from
// global memory each level; they are L2-resident after the first).
// Sampled entries S of a segment of `len` entries: every window but the last
// holds a whole block.
__host__ __device__ __forceinline__ uint32_t sample_count(uint32_t len, uint32_t period) {
    const uint64_t win = 32ull * period;
    const uint64_t nwin = (len + win - 1) / win;
    const uint64_t wl = nwin - 1;
    const uint64_t last_start = wl * win + 32u * ((static_cast<uint32_t>(wl) * 2654435769u) % period);
    const uint64_t last_ns = last_start < len ? (len - last_start < 32 ? len - last_start : 32) : 0;
    return static_cast<uint32_t>(wl * 32 + last_ns);
}

// The top of the fine bins for sampled selection: the largest sample key, or
// when the estimate is that key itself (a sample of a few dozen keys gives
// r = 1) the largest finite key, since nothing is known above.  When the
// staged keys pass the budget, T then lies in a bin of at most 2^20 keys
// (an eighth of a binade) instead of above the bins.
__device__ __forceinline__ uint32_t sample_top(uint32_t est, uint32_t hkey) {
    return hkey > est ? hkey : 0x7F800000u;
}

// r = ceil(S k / n), the estimate's rank among the samples.
__device__ __forceinline__ uint32_t sample_rank(uint32_t S, const SegDev &seg) {
    return static_cast<uint32_t>((uint64_t(S) * seg.k + seg.len - 1) / seg.len);
}

__global__ __launch_bounds__(kBlock) void dgc_squant_kernel(PlanDev P, uint32_t period, DgcWs w) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    const uint32_t S = sample_count(seg.len, period);
    uint32_t rank = sample_rank(S, seg);
    const uint32_t *keys = w.sidx + seg.off;
    __shared__ uint32_t h[kHist1];
    __shared__ uint32_t wmax[kWaves];
    uint32_t prefix = 0, kmax = 0;
    for (int level = 0; level < 3; ++level) {
        const int nb = level == 2 ? kHist3 : kHist1;
        const int shift = level == 0 ? kDigit2Bits + kDigit3Bits : level == 1 ? kDigit3Bits : 0;
        const int pshift = level == 1 ? kDigit2Bits + kDigit3Bits : kDigit3Bits;  // prefix bits below
        for (int i = threadIdx.x; i < nb; i += kBlock) h[i] = 0u;
        __syncthreads();
        constexpr uint32_t kB = 8;
        for (uint32_t j0 = 0; j0 < S; j0 += kB * kBlock) {
            uint32_t key[kB];
#pragma unroll
            for (uint32_t u = 0; u < kB; ++u) key[u] = keys[min(j0 + u * kBlock + threadIdx.x, S - 1)];
#pragma unroll
            for (uint32_t u = 0; u < kB; ++u) {
                if (j0 + u * kBlock + threadIdx.x >= S) continue;
                if (level == 0) kmax = max(kmax, key[u]);
                if (level > 0 && (key[u] >> pshift) != prefix) continue;
                atomicAdd(&h[(key[u] >> shift) & uint32_t(nb - 1)], 1u);
            }
        }
        __syncthreads();
        uint32_t above, d;
        if (level == 2) d = block_find_bucket<kHist3>(rank, [&](int b) { return h[b]; }, &above);
        else d = block_find_bucket<kHist1>(rank, [&](int b) { return h[b]; }, &above);
        rank -= above;
        prefix = level == 0 ? d : level == 1 ? ((prefix << kDigit2Bits) | d) : ((prefix << kDigit3Bits) | d);
        __syncthreads();
    }
    kmax = wave_max_all(kmax);
    if (lane_id() == 0) wmax[wave_id()] = kmax;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t hk = 0;
        for (int i = 0; i < kWaves; ++i) hk = max(hk, wmax[i]);
        w.st[s].Lkey = prefix;
        w.st[s].hkey = hk;
        w.st[s].fshift = fine_shift(prefix, sample_top(prefix, hk));
    }
}

// The same radix select spread over kQBlocks workgroups per segment, for
// samples too many for one workgroup: per digit, a histogram kernel (each
// workgroup an LDS histogram of its share of the keys that match the prefix,
// flushed into the segment's qhist) and a find kernel (one workgroup per
// segment: the digit, the rank left, qhist cleared for the next digit).
constexpr uint32_t kQBlocks = 32;
constexpr uint32_t kQuantOneBlock = 32768;  // most samples one workgroup handles alone

template <int kLevel>
__global__ __launch_bounds__(kBlock) void dgc_qhist_kernel(PlanDev P, uint32_t period, DgcWs w) {
    const uint32_t s = blockIdx.x / kQBlocks, b = blockIdx.x % kQBlocks;
    const SegDev seg = P.seg[s];
    const uint32_t S = sample_count(seg.len, period);
    const uint32_t per = (S + kQBlocks - 1) / kQBlocks;
    const uint32_t j0 = b * per, j1 = min(S, j0 + per);
    if (j0 >= j1) return;
    constexpr int nb = kLevel == 2 ? kHist3 : kHist1;
    constexpr int shift = kLevel == 0 ? kDigit2Bits + kDigit3Bits : kLevel == 1 ? kDigit3Bits : 0;
    constexpr int pshift = kLevel == 1 ? kDigit2Bits + kDigit3Bits : kDigit3Bits;
    const uint32_t prefix = kLevel > 0 ? w.st[s].qprefix : 0u;
    __shared__ uint32_t h[nb];
    for (int i = threadIdx.x; i < nb; i += kBlock) h[i] = 0u;
    __syncthreads();
    const uint32_t *keys = w.sidx + seg.off;
    constexpr uint32_t kB = 8;
    uint32_t kmax = 0;
    for (uint32_t i0 = j0; i0 < j1; i0 += kB * kBlock) {
        uint32_t key[kB];
#pragma unroll
        for (uint32_t u = 0; u < kB; ++u) key[u] = keys[min(i0 + u * kBlock + threadIdx.x, j1 - 1)];
#pragma unroll
        for (uint32_t u = 0; u < kB; ++u) {
            if (i0 + u * kBlock + threadIdx.x >= j1) continue;
            if (kLevel == 0) kmax = max(kmax, key[u]);
            if (kLevel > 0 && (key[u] >> pshift) != prefix) continue;
            atomicAdd(&h[(key[u] >> shift) & uint32_t(nb - 1)], 1u);
        }
    }
    if (kLevel == 0) {
        // the largest sample key (hkey is cleared by prep)
        __shared__ uint32_t wmax[kWaves];
        kmax = wave_max_all(kmax);
        if (lane_id() == 0) wmax[wave_id()] = kmax;
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t hk = 0;
            for (int i = 0; i < kWaves; ++i) hk = max(hk, wmax[i]);
            atomicMax(&w.st[s].hkey, hk);
        }
    }
    __syncthreads();
    uint32_t *g = w.qhist + size_t(s) * kHist1;
    for (int i = threadIdx.x; i < nb; i += kBlock)
        if (h[i]) atomicAdd(&g[i], h[i]);
}

template <int kLevel>
__global__ __launch_bounds__(kBlock) void dgc_qfind_kernel(PlanDev P, uint32_t period, DgcWs w) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    uint32_t *g = w.qhist + size_t(s) * kHist1;
    const uint32_t rank = kLevel == 0 ? sample_rank(sample_count(seg.len, period), seg) : w.st[s].qrank;
    const uint32_t prefix = kLevel > 0 ? w.st[s].qprefix : 0u;
    uint32_t above, d;
    if (kLevel == 2) d = block_find_bucket<kHist3>(rank, [&](int b) { return g[b]; }, &above);
    else d = block_find_bucket<kHist1>(rank, [&](int b) { return g[b]; }, &above);
    for (int i = threadIdx.x; i < kHist1; i += kBlock) g[i] = 0u;  // clean for the next digit or call
    if (threadIdx.x == 0) {
        const uint32_t np = kLevel == 0 ? d : kLevel == 1 ? ((prefix << kDigit2Bits) | d) : ((prefix << kDigit3Bits) | d);
        w.st[s].qrank = rank - above;
        w.st[s].qprefix = np;
        if (kLevel == 2) {
            w.st[s].Lkey = np;
            w.st[s].fshift = fine_shift(np, sample_top(np, w.st[s].hkey));
        }
    }
}

// ----------------------------------------------------------------- bound
// Of S samples, about E = S k / n fall in the segment's top k (a binomial
// count).  Lkey is the (E + 4 sqrt(E) + 16)-th largest sample key, rounded
// down to its 22-bit prefix (digits 1 and 2), or 0 (stage everything) when
// the sample is too small for that.  A sampled chunk's 32 keys are 128
// contiguous bytes: thread i loads 16-byte pieces i, i + 256, ... (piece
// 8 j + p of sampled chunk j), at most 16 per thread, all in flight
// together, and keeps them for the two LDS histogram passes.
__global__ __launch_bounds__(kBlock) void dgc_bound_kernel(PlanDev P, DgcWs w) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    __shared__ uint32_t h[kHist1];
    const uint32_t stride = sample_stride(seg.dnchunk);
    const uint32_t nsc = (seg.dnchunk + stride - 1) / stride;  // sampled chunks
    const uint32_t last = (nsc - 1) * stride;                   // last sampled chunk
    const uint32_t last_cnt = min(seg.len - last * uint32_t(kChunk), uint32_t(kChunk));
    const uint32_t last_ns = min(kSamples, last_cnt);
    const uint32_t total = (nsc - 1) * kSamples + last_ns;
    const double E = double(total) * double(seg_k(seg, w)) / double(seg.len);
    const double target = E + 4.0 * sqrt(E) + 16.0;
    if (!(target < double(total))) {  // uniform: too few samples, stage everything
        if (threadIdx.x == 0) w.st[s].Lkey = 0u;
        return;
    }
    constexpr uint32_t kPer = kSampleChunks * (kSamples / 4) / kBlock;
    const uint32_t npiece = nsc * (kSamples / 4);
    uint4 piece[kPer];
#pragma unroll
    for (uint32_t u = 0; u < kPer; ++u) {
        const uint32_t i = min(u * kBlock + threadIdx.x, npiece - 1);
        const uint32_t c = seg.dchunk0 + (i / (kSamples / 4)) * stride;
        piece[u] = *reinterpret_cast<const uint4 *>(w.skey + size_t(c) * kSamples + (i % (kSamples / 4)) * 4);
    }
    // key q of piece u, or none (past the samples)
    auto key_of = [&](uint32_t u, uint32_t q, uint32_t *key) {
        const uint32_t i = u * kBlock + threadIdx.x;
        const uint32_t lim = i / (kSamples / 4) == nsc - 1 ? last_ns : kSamples;
        const uint32_t l = (i % (kSamples / 4)) * 4 + q;
        *key = q == 0 ? piece[u].x : q == 1 ? piece[u].y : q == 2 ? piece[u].z : piece[u].w;
        return i < npiece && l < lim;
    };
    uint32_t rank = static_cast<uint32_t>(target), prefix = 0;
    for (int level = 0; level < 2; ++level) {
        for (int i = threadIdx.x; i < kHist1; i += kBlock) h[i] = 0u;
        __syncthreads();
#pragma unroll
        for (uint32_t u = 0; u < kPer; ++u)
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) {
                uint32_t key;
                if (!key_of(u, q, &key)) continue;
                const uint32_t d1 = key >> (kDigit2Bits + kDigit3Bits);
                if (level == 0) atomicAdd(&h[d1], 1u);
                else if (d1 == prefix) atomicAdd(&h[(key >> kDigit3Bits) & (kHist2 - 1)], 1u);
            }
        __syncthreads();
        uint32_t above;
        const uint32_t d = block_find_bucket<kHist1>(rank, [&](int b) { return h[b]; }, &above);
        rank -= above;
        prefix = level == 0 ? d : ((prefix << kDigit2Bits) | d);
        __syncthreads();
    }
    if (threadIdx.x == 0) w.st[s].Lkey = prefix << kDigit3Bits;
}

// ---------------------------------------------------------------- update
// The digit-1 histogram lives in LDS across the workgroup's chunks and is
// flushed to the segment's global histogram only when the segment changes.
// Staging: in row j, wave w holds elements [1024 j + 256 w, +256) of the
// chunk (lane-major, 4 per lane), so an entry's rank in the chunk is the
// staged count of the (row, wave) pieces before its own, plus the ballot
// ranks of lower lanes, plus its own earlier flags.  The piece counts go
// through a double-buffered LDS table with one barrier per chunk.
//
// The DGC modes read G, U and V and write U and V; kSignif reads g and w and
// writes nothing dense; kExplore reads only the core bitmap.
//
// kFine (the exact path): no digit-1 histogram; the staged entries go to the
// chunk's own 4096-entry slot (c * 4096, 16-byte aligned) instead of its
// first element, and each staged key is added to the segment's fine
// histogram by a global atomic (a few dozen per chunk at the pages' 0.1%
// density).  (An LDS histogram flushed per segment raised the kernel to 130
// VGPRs, three waves per SIMD, and cost it 5% of its bandwidth.)
template <int kMode, bool kFine = false>
__global__ __launch_bounds__(kBlock) void dgc_update_kernel(PlanDev P, Src a, DgcWs w) {
    constexpr bool kDgc = kMode == kVanilla || kMode == kNesterov;
    uint32_t c0, c1;
    chunk_range(P.ndchunk, &c0, &c1);
    __shared__ uint32_t hist[kHist1];
    __shared__ uint32_t piece[2][kRows * kWaves];
    for (int i = threadIdx.x; i < kHist1; i += kBlock) hist[i] = 0u;
    if (c0 >= c1) return;
    float g[kRows][4], u[kRows][4], v[kRows][4];
    ChunkWalker walk;
    ChunkInfo ci = walk.at(P, c0);
    BufRsrc rg, ru, rv;
    auto fetch = [&](const ChunkInfo &k) {
        if (kMode == kExplore) return;
        rg = chunk_buf(a.G + k.lo, k.cnt);
        ru = chunk_buf(a.U + k.lo, k.cnt);
        if (kDgc) rv = chunk_buf(a.V + k.lo, k.cnt);
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            load4(rg, row_elem(j), g[j]);
            load4(ru, row_elem(j), u[j]);
            if (kDgc) load4(rv, row_elem(j), v[j]);
        }
    };
    fetch(ci);
    __syncthreads();
    const int lane = lane_id(), wave = wave_id();
    WaveHist fine;  // the exact path's fine histogram
    for (uint32_t c = c0; c < c1; ++c) {
        const float clip = kDgc ? w.st[ci.s].clip : 1.0f;
        const uint32_t Lkey = w.st[ci.s].Lkey;
        const uint32_t fs = kFine ? w.st[ci.s].fshift : 0u;
        const uint32_t pos = static_cast<uint32_t>(ci.lo - ci.seg.off);  // chunk start in the segment
        uint32_t flags[kRows], before[kRows];
#pragma unroll
        for (int j = 0; j < kRows; ++j) {
            const uint32_t e0 = row_elem(j);
            flags[j] = 0;
            before[j] = 0;
            uint32_t piece_total = 0;
            if (kMode == kExplore) explore_values(a, ci.seg, ci.s, pos + e0, v[j]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (kDgc) {
                    const float gc = clip * g[j][q];
                    momentum_update<kMode>(a.m, gc, u[j][q], v[j][q]);
                } else if (kMode == kSignif) {
                    v[j][q] = significance(u[j][q], g[j][q], a.m);
                }
                const float vn = v[j][q];
                const bool in = e0 + q < ci.cnt;
                const uint32_t key = mag_key(vn);
                const bool f = in && key >= Lkey;
                if (!kFine && in) atomicAdd(&hist[key >> (kDigit2Bits + kDigit3Bits)], 1u);
                flags[j] |= uint32_t(f) << q;
                const uint64_t bm = __ballot(f);
                before[j] += lane_rank(bm);
                piece_total += static_cast<uint32_t>(__popcll(bm));
            }
            if (lane == 0) piece[(c - c0) & 1][j * kWaves + wave] = piece_total;
            if (kDgc) {
                store4(ru, e0, u[j]);
                store4(rv, e0, v[j]);
            }
        }
        __syncthreads();
        {
            const uint32_t *pc = piece[(c - c0) & 1];
            uint32_t run = 0, base[kRows];
#pragma unroll
            for (int j = 0; j < kRows; ++j)
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) {
                    if (ww == wave) base[j] = run;
                    run += pc[j * kWaves + ww];
                }
            if (threadIdx.x == 0) w.ccount[c] = run;
            // the staging area: the chunk's first element, or its own slot
            // (64-bit: a plan may hold more than 2^20 chunks)
            const size_t slot0 = kFine ? (size_t(c) << kChunkLog2) : size_t(ci.lo);
            uint32_t *const sidx = w.sidx + slot0;
            float *const sval = w.sval + slot0;
            uint32_t *const xt = xtables(w, ci.s);
#pragma unroll
            for (int j = 0; j < kRows; ++j) {
                if (flags[j]) {
                    uint32_t slot = base[j] + before[j];
                    const uint32_t e0 = static_cast<uint32_t>(ci.lo) + row_elem(j);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if ((flags[j] >> q) & 1u) {
                            sidx[slot] = e0 + q;
                            sval[slot] = v[j][q];
                            ++slot;
                        }
                    }
                }
                if (kFine) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        fine.add(xt, (flags[j] >> q) & 1u, fine_bin(mag_key(v[j][q]), Lkey, fs));
                }
            }
        }
        const uint32_t s_done = ci.s;
        const bool more = c + 1 < c1;
        if (more) {
            ci = walk.at(P, c + 1);
            fetch(ci);
        }
        if (!kFine && (!more || ci.s != s_done)) {
            __syncthreads();
            uint32_t *h1 = w.hist1 + (size_t(s_done) * kHistRep + blockIdx.x % kHistRep) * kHist1;
            for (int i = threadIdx.x; i < kHist1; i += kBlock) {
                const uint32_t n = hist[i];
                if (n) {
                    atomicAdd(&h1[i], n);
                    hist[i] = 0u;
                }
            }
            __syncthreads();
        }
    }
    if (kFine) {
        // the waves' last counts, combined in the workgroup (in a tensor of
        // zeros every wave ends on the same bin)
        __shared__ uint32_t *fh[kWaves];
        __shared__ uint32_t fbin[kWaves], fcnt[kWaves];
        if (lane == 0) {
            fh[wave] = fine.h;
            fbin[wave] = fine.bin;
            fcnt[wave] = fine.cnt;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 0; i < kWaves; ++i) {
                if (fcnt[i] == 0) continue;
                uint32_t n = fcnt[i];
                for (int j = i + 1; j < kWaves; ++j)
                    if (fcnt[j] != 0 && fh[j] == fh[i] && fbin[j] == fbin[i]) {
                        n += fcnt[j];
                        fcnt[j] = 0;
                    }
                atomicAdd(fh[i] + fbin[i], n);
            }
        }
    }
}

// --------------------------------------------------------------- selects
template <int NB>
__device__ __forceinline__ uint32_t replica_sum(const uint32_t *h, int b) {
    uint32_t t = 0;
#pragma unroll
    for (uint32_t r = 0; r < kHistRep; ++r) t += h[r * NB + b];
    return t;
}

// Level 1..3 of the radix select for one segment.  Level 1 also settles the
// segment's output: in sampled selection (budget > 0) a segment whose staged
// entries (every key at or above the estimate) fit the budget sends them all.
template <int kLevel>
__global__ __launch_bounds__(kBlock) void dgc_select_kernel(PlanDev P, DgcWs w, uint32_t over) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    SegState st = w.st[s];
    uint32_t above;
    if (kLevel == 1) {
        const uint32_t *h = w.hist1 + size_t(s) * kHistRep * kHist1;
        const uint32_t ks = seg_k(seg, w);
        uint32_t d = block_find_bucket<kHist1>(ks, [&](int b) { return replica_sum<kHist1>(h, b); }, &above);
        // entries the update staged in the segment (all keys >= Lkey)
        uint32_t staged = 0;
        for (uint32_t i0 = 0; i0 < seg.dnchunk; i0 += 8 * kBlock) {
            uint32_t n[8];
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u)
                n[u] = w.ccount[seg.dchunk0 + min(i0 + u * kBlock + threadIdx.x, seg.dnchunk - 1)];
#pragma unroll
            for (uint32_t u = 0; u < 8; ++u)
                if (i0 + u * kBlock + threadIdx.x < seg.dnchunk) staged += n[u];
        }
        uint32_t staged_total;
        (void)block_exclusive_scan(staged, &staged_total);
        if (threadIdx.x == 0) {
            w.st[s].d1 = d;
            w.st[s].above1 = above;
            w.st[s].redo = 0u;
            w.st[s].all = 0u;
            w.st[s].sent = ks;
            w.st[s].base = seg.kbase;
            if (over == 0) {
                w.st[s].redo = staged_total < ks ? 1u : 0u;
            } else {
                const uint64_t budget = umin64(seg.len, uint64_t(over) * seg.k);
                if (staged_total <= budget) {
                    w.st[s].all = 1u;
                    w.st[s].sent = staged_total;
                    w.st[s].T = st.Lkey;  // every staged key is >= the estimate
                    w.st[s].gt = 0u;
                    w.st[s].need_eq = 0xFFFFFFFFu;
                }
            }
        }
    } else if (kLevel == 2) {
        if (st.all) return;
        const uint32_t *h = w.hist2 + size_t(s) * kHistRep * kHist2;
        uint32_t d = block_find_bucket<kHist2>(seg_k(seg, w) - st.above1, [&](int b) { return replica_sum<kHist2>(h, b); },
                                               &above);
        if (threadIdx.x == 0) {
            w.st[s].d2 = d;
            w.st[s].above2 = st.above1 + above;
        }
    } else {
        if (st.all) return;
        const uint32_t *h = w.hist3 + size_t(s) * kHist3;
        const uint32_t ks = seg_k(seg, w);
        uint32_t d = block_find_bucket<kHist3>(ks - st.above2, [&](int b) { return h[b]; }, &above);
        if (threadIdx.x == 0) {
            uint32_t gt = st.above2 + above;
            w.st[s].T = (((st.d1 << kDigit2Bits) | st.d2) << kDigit3Bits) | d;
            w.st[s].gt = gt;
            w.st[s].need_eq = ks - gt;
        }
    }
}

// ----------------------------------------------------------------- sbase
// Sampled selection: segments send variable counts, laid end to end in
// segment order.  With seg_off (sampled selection on the exact path, where
// the counts are settled by select) the message's offsets are written too.
__global__ __launch_bounds__(kBlock) void dgc_sbase_kernel(PlanDev P, DgcWs w, uint32_t *__restrict__ seg_off) {
    uint32_t run = 0;
    for (int s0 = 0; s0 < P.nseg; s0 += kBlock) {
        const int s = s0 + int(threadIdx.x);
        const uint32_t v = s < P.nseg ? w.st[s].sent : 0u;
        uint32_t tot;
        const uint32_t pre = block_exclusive_scan(v, &tot);
        if (s < P.nseg) {
            w.st[s].base = run + pre;
            if (seg_off) seg_off[s] = run + pre;
        }
        run += tot;
    }
    if (seg_off && threadIdx.x == 0) seg_off[P.nseg] = run;
}

// ------------------------------------------- candidate kernels (waves)
// stage, refine, count and emit give each wave CPW consecutive chunks.  A
// chunk holds a few staged entries, so what these kernels cost is the chain
// of dependent loads: chunk record, segment state, staged entries.  The wave
// issues the loads of all its chunks at once (lane j holds chunk j's record
// and state, and every lane its entry of each chunk's first 64), then takes
// the chunks in turn.  Plans of at least kWideChunks chunks use kCpwWide
// (on the 122M-element layout emit went from 21 to 17 us and refine from 9
// to 7.5 us; stage, bound by its histogram atomics, stayed the same).
// Smaller plans keep one chunk per wave, since fewer waves leave the chip
// idle while each walks its chunks (the 1M-element tensor ran 9% slower at
// 4 chunks per wave).
constexpr uint32_t kCpwWide = 4;
constexpr uint32_t kWideChunks = 16384;

__device__ __forceinline__ uint32_t lane_val(uint32_t v, uint32_t j) { return __builtin_amdgcn_readlane(v, j); }

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) { return wave_total(x); }

template <uint32_t CPW>
__device__ __forceinline__ uint32_t wave_chunk0() { return (blockIdx.x * kWaves + wave_id()) * CPW; }

// Lane j < CPW: record and staged count of chunk c0 + j (lanes past the
// last chunk, and lanes >= CPW, hold a copy of a valid chunk's).
struct WaveChunks {
    ChunkRec rec;
    uint32_t n;
};

template <uint32_t CPW>
__device__ __forceinline__ WaveChunks wave_chunks(const PlanDev &P, const DgcWs &w, uint32_t c0) {
    const uint32_t c = min(c0 + uint32_t(lane_id()) % CPW, P.ndchunk - 1);
    WaveChunks wc;
    wc.rec = P.dchunk_rec[c];
    wc.n = min(w.ccount[c], wc.rec.y);
    return wc;
}

// Staged entry `lane` (clamped) of chunk j of the wave, or 0 when it has none.
__device__ __forceinline__ uint32_t first_key(const DgcWs &w, const WaveChunks &wc, uint32_t j) {
    const uint32_t n = lane_val(wc.n, j);
    return n ? mag_key(w.sval[lane_val(wc.rec.x, j) + min(uint32_t(lane_id()), n - 1)]) : 0u;
}

// Calls f(i, key) for the staged entries i < n of the chunk at lo (each lane
// its own entries; entries past n are skipped): the first 64 from k0, the
// rest four batches of loads at a time.
template <typename F>
__device__ __forceinline__ void for_staged_keys(const DgcWs &w, uint32_t lo, uint32_t n, uint32_t k0, F &&f) {
    const uint32_t lane = lane_id();
    if (lane < n) f(lane, k0);
    for (uint32_t i0 = kWave; i0 < n; i0 += 4 * kWave) {
        uint32_t key[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) key[q] = mag_key(w.sval[lo + min(i0 + q * kWave + lane, n - 1)]);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (i0 + q * kWave + lane < n) f(i0 + q * kWave + lane, key[q]);
    }
}

// The same walk with the whole wave in every call: f(valid, key), valid
// false for the lanes past n (for WaveHist, whose ballots need every lane).
template <typename F>
__device__ __forceinline__ void for_staged_keys_wave(const DgcWs &w, uint32_t lo, uint32_t n, uint32_t k0, F &&f) {
    const uint32_t lane = lane_id();
    f(lane < n, k0);
    for (uint32_t i0 = kWave; i0 < n; i0 += 4 * kWave) {
        uint32_t key[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) key[q] = mag_key(w.sval[lo + min(i0 + q * kWave + lane, n - 1)]);
#pragma unroll
        for (int q = 0; q < 4; ++q) f(i0 + q * kWave + lane < n, key[q]);
    }
}

// ----------------------------------------------------------------- stage
// Normally the update staged every candidate: the wave histograms digit 2 of
// the staged entries whose digit 1 is d1.  In a re-staged segment it re-reads
// the chunk's values instead (stage_chunk_again).
constexpr int kWaveRows = kChunk / (4 * kWave);
// A chunk of the candidate path that sends at least this many entries masks
// U and V by rewriting the chunk (64 KB of traffic) instead of two scattered
// 4-byte writes per entry (each a partial line, some 128 B of traffic).
constexpr uint32_t kDenseMask = 512;

// One wave re-stages chunk c: lane l holds elements [256 r + 4 l, +4) for
// rows r = 0..15, so 16 KB of V is in flight per wave and the ordered
// compaction needs only ballots (rank = running count + lanes below + within
// lane); no LDS, no workgroup barrier.
template <int kMode>
__device__ __forceinline__ void stage_chunk_again(const PlanDev &P, const Src &a, const DgcWs &w, uint32_t c,
                                                  const ChunkRec &rec, uint32_t d1, uint32_t *h2) {
    const uint32_t lo = rec.x, cnt = rec.y, s = rec.z;
    const int lane = lane_id();
    // the ranked values again: V (DGC, already updated), or recomputed
    float v[kWaveRows][4];
    if (kMode == kVanilla || kMode == kNesterov) {
        const BufRsrc rv = chunk_buf(a.V + lo, cnt);
#pragma unroll
        for (int r = 0; r < kWaveRows; ++r) load4(rv, r * (4 * kWave) + 4u * lane, v[r]);
    } else if (kMode == kSignif) {
        const BufRsrc rg = chunk_buf(a.G + lo, cnt), rw = chunk_buf(a.U + lo, cnt);
        float gg[kWaveRows][4];
#pragma unroll
        for (int r = 0; r < kWaveRows; ++r) {
            load4(rg, r * (4 * kWave) + 4u * lane, gg[r]);
            load4(rw, r * (4 * kWave) + 4u * lane, v[r]);
        }
#pragma unroll
        for (int r = 0; r < kWaveRows; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) v[r][q] = significance(v[r][q], gg[r][q], a.m);
    } else {
        const SegDev seg = P.seg[s];
#pragma unroll
        for (int r = 0; r < kWaveRows; ++r)
            explore_values(a, seg, s, (rec.w << kChunkLog2) + r * (4 * kWave) + 4u * lane, v[r]);
    }
    uint32_t run = 0;  // wave-uniform count of entries staged so far
    WaveHist wh;
#pragma unroll
    for (int r = 0; r < kWaveRows; ++r) {
        const uint32_t e0 = r * (4 * kWave) + 4u * lane;
        bool flag[4];
        uint32_t before = 0, row_total = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const bool in = e0 + q < cnt;
            const uint32_t key = mag_key(v[r][q]);
            const uint32_t dig1 = key >> (kDigit2Bits + kDigit3Bits);
            flag[q] = in && dig1 >= d1;
            wh.add(h2, in && dig1 == d1, (key >> kDigit3Bits) & (kHist2 - 1));
            const uint64_t m = __ballot(flag[q]);
            before += lane_rank(m);
            row_total += static_cast<uint32_t>(__popcll(m));
        }
        if (row_total) {
            uint32_t slot = lo + run + before;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (flag[q]) {
                    w.sidx[slot] = lo + e0 + q;
                    w.sval[slot] = v[r][q];
                    ++slot;
                }
            }
        }
        run += row_total;
    }
    wh.flush();
    if (lane == 0) w.ccount[c] = run;
}

template <int kMode, uint32_t CPW>
__global__ __launch_bounds__(kBlock) void dgc_stage_kernel(PlanDev P, Src a, DgcWs w, int redo_only) {
    const uint32_t c0 = wave_chunk0<CPW>();
    if (c0 >= P.ndchunk) return;
    const WaveChunks wc = wave_chunks<CPW>(P, w, c0);
    const SegState &sl = w.st[wc.rec.z];
    const uint32_t all_l = sl.all, redo_l = sl.redo, d1_l = sl.d1;
    uint32_t k0[CPW];
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) k0[j] = redo_only ? 0u : first_key(w, wc, j);
    auto hist2_of = [&](uint32_t c, uint32_t s) { return w.hist2 + (size_t(s) * kHistRep + c % kHistRep) * kHist2; };
    if (!redo_only) {
        WaveHist wh;
#pragma unroll
        for (uint32_t j = 0; j < CPW; ++j) {
            const uint32_t c = c0 + j;
            if (c >= P.ndchunk) break;
            if (lane_val(all_l, j) || lane_val(redo_l, j)) continue;
            const uint32_t d1 = lane_val(d1_l, j);
            uint32_t *h2 = hist2_of(c, lane_val(wc.rec.z, j));
            for_staged_keys_wave(w, lane_val(wc.rec.x, j), lane_val(wc.n, j), k0[j], [&](bool valid, uint32_t key) {
                wh.add(h2, valid && (key >> (kDigit2Bits + kDigit3Bits)) == d1, (key >> kDigit3Bits) & (kHist2 - 1));
            });
        }
        wh.flush();
    }
    // re-staged segments (the fallback): one chunk at a time
#pragma unroll 1
    for (uint32_t j = 0; j < CPW; ++j) {
        const uint32_t c = c0 + j;
        if (c >= P.ndchunk) break;
        if (lane_val(all_l, j) || !lane_val(redo_l, j)) continue;
        const ChunkRec rec = make_uint4(lane_val(wc.rec.x, j), lane_val(wc.rec.y, j), lane_val(wc.rec.z, j),
                                        lane_val(wc.rec.w, j));
        stage_chunk_again<kMode>(P, a, w, c, rec, lane_val(d1_l, j), hist2_of(c, rec.z));
    }
}

// Digit-2 histogram of the boundary bucket for dense selections (Slim-DP's
// core at 10% density puts millions of staged entries in the boundary
// digit-1 bucket, where one global atomic per entry dominated): a workgroup
// takes kStageSpan consecutive chunks, counts in LDS and flushes once per
// segment it touched.  Re-staged segments are left to dgc_stage_kernel.
// The chunks' records, counts and segment states are loaded together before
// the walk, so that each chunk costs one round of key loads (Slim-DP's core
// on the DeepSpeech layout: 62 -> 34 us at 16 chunks per workgroup, 40 us
// at 32).
constexpr uint32_t kStageSpan = 16;

__global__ __launch_bounds__(kBlock) void dgc_stagew_kernel(PlanDev P, DgcWs w) {
    static_assert(kStageSpan <= kBlock, "one thread per chunk loads its record");
    const uint32_t c0 = blockIdx.x * kStageSpan, c1 = min(P.ndchunk, c0 + kStageSpan);
    __shared__ uint32_t h[kHist2];
    // every chunk's record, staged count and segment state, loaded together
    __shared__ uint32_t cx[kStageSpan], cz[kStageSpan], cn[kStageSpan], cd[kStageSpan];
    for (int i = threadIdx.x; i < kHist2; i += kBlock) h[i] = 0u;
    if (threadIdx.x < c1 - c0) {
        const ChunkRec rec = P.dchunk_rec[c0 + threadIdx.x];
        const uint32_t n = min(w.ccount[c0 + threadIdx.x], rec.y);
        const SegState &st = w.st[rec.z];
        cx[threadIdx.x] = rec.x;
        cz[threadIdx.x] = rec.z;
        cn[threadIdx.x] = st.all || st.redo ? 0u : n;  // skipped segments count nothing
        cd[threadIdx.x] = st.d1;
    }
    __syncthreads();
    uint32_t cur = cz[0];
    auto flush = [&](uint32_t seg) {
        __syncthreads();
        uint32_t *h2 = w.hist2 + (size_t(seg) * kHistRep + blockIdx.x % kHistRep) * kHist2;
        for (int i = threadIdx.x; i < kHist2; i += kBlock) {
            const uint32_t v = h[i];
            if (v) {
                atomicAdd(&h2[i], v);
                h[i] = 0u;
            }
        }
        __syncthreads();
    };
    for (uint32_t c = c0; c < c1; ++c) {
        const uint32_t z = cz[c - c0];
        if (z != cur) {
            flush(cur);
            cur = z;
        }
        const uint32_t n = cn[c - c0], d1 = cd[c - c0], lo = cx[c - c0];
        for (uint32_t i0 = 0; i0 < n; i0 += 4 * kBlock) {
            uint32_t key[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) key[q] = mag_key(w.sval[lo + min(i0 + q * kBlock + threadIdx.x, n - 1)]);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (i0 + q * kBlock + threadIdx.x < n && (key[q] >> (kDigit2Bits + kDigit3Bits)) == d1)
                    atomicAdd(&h[(key[q] >> kDigit3Bits) & (kHist2 - 1)], 1u);
        }
    }
    flush(cur);
}

// ------------------------------------------------------- refine, count
template <uint32_t CPW>
__global__ __launch_bounds__(kBlock) void dgc_refine_kernel(PlanDev P, DgcWs w) {
    const uint32_t c0 = wave_chunk0<CPW>();
    if (c0 >= P.ndchunk) return;
    const WaveChunks wc = wave_chunks<CPW>(P, w, c0);
    const SegState &sl = w.st[wc.rec.z];
    const uint32_t all_l = sl.all, prefix_l = (sl.d1 << kDigit2Bits) | sl.d2;
    uint32_t k0[CPW];
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) k0[j] = first_key(w, wc, j);
    WaveHist wh;
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) {
        if (c0 + j >= P.ndchunk) break;
        const uint32_t n = lane_val(wc.n, j);
        if (n == 0 || lane_val(all_l, j)) continue;
        const uint32_t prefix = lane_val(prefix_l, j);
        uint32_t *h3 = w.hist3 + size_t(lane_val(wc.rec.z, j)) * kHist3;
        for_staged_keys_wave(w, lane_val(wc.rec.x, j), n, k0[j], [&](bool valid, uint32_t key) {
            wh.add(h3, valid && (key >> kDigit3Bits) == prefix, key & (kHist3 - 1));
        });
    }
    wh.flush();
}

template <uint32_t CPW>
__global__ __launch_bounds__(kBlock) void dgc_count_kernel(PlanDev P, DgcWs w) {
    const uint32_t c0 = wave_chunk0<CPW>();
    if (c0 >= P.ndchunk) return;
    const WaveChunks wc = wave_chunks<CPW>(P, w, c0);
    const uint32_t T_l = w.st[wc.rec.z].T;
    uint32_t k0[CPW];
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) k0[j] = first_key(w, wc, j);
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) {
        const uint32_t c = c0 + j;
        if (c >= P.ndchunk) break;
        const uint32_t T = lane_val(T_l, j);
        uint32_t gt = 0, eq = 0;  // this lane's entries
        for_staged_keys(w, lane_val(wc.rec.x, j), lane_val(wc.n, j), k0[j], [&](uint32_t, uint32_t key) {
            gt += key > T ? 1u : 0u;
            eq += key == T ? 1u : 0u;
        });
        const uint32_t ngt = wave_sum(gt), neq = wave_sum(eq);
        if (lane_id() == 0) {
            w.cgt[c] = ngt;
            w.ceq[c] = neq;
        }
    }
}

// ------------------------------------------------------------------ scan
// Ties at the threshold go to the lowest indices: scan the segment's chunks
// in order for the tie quota and the message slot of each chunk.  Thread t
// owns a contiguous run of chunks (loads batched), so one round of two block
// scans covers up to kBlock * kScanRun chunks.  The ties taken in a run are a
// greedy prefix fill of the quota, so a run's total is known from its tie
// prefix alone: min(max(need - before, 0), run ties).
constexpr uint32_t kScanRun = 32;

__global__ __launch_bounds__(kBlock) void dgc_scan_kernel(PlanDev P, DgcWs w,
                                                          uint32_t *__restrict__ seg_off) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    const uint32_t need_eq = w.st[s].need_eq;
    const uint32_t base = w.st[s].base;
    const uint32_t *ceq = w.ceq + seg.dchunk0, *cgt = w.cgt + seg.dchunk0;
    uint32_t eq_before = 0, sel_before = 0;
    for (uint32_t r0 = 0; r0 < seg.dnchunk; r0 += kBlock * kScanRun) {
        const uint32_t nr = min(seg.dnchunk - r0, kBlock * kScanRun);
        const uint32_t per = (nr + kBlock - 1) / kBlock;
        const uint32_t t0 = r0 + threadIdx.x * per;
        const uint32_t t1 = min(t0 + per, r0 + nr);
        uint32_t e[kScanRun], g[kScanRun];  // the run, all loads in flight together
#pragma unroll
        for (uint32_t u = 0; u < kScanRun; ++u) {
            const uint32_t i = min(t0 + u, r0 + nr - 1);
            e[u] = ceq[i];
            g[u] = cgt[i];
        }
        uint32_t eq_sum = 0, gt_sum = 0;
#pragma unroll
        for (uint32_t u = 0; u < kScanRun; ++u)
            if (t0 + u < t1) {
                eq_sum += e[u];
                gt_sum += g[u];
            }
        uint32_t eq_tot;
        const uint32_t eq_pre = eq_before + block_exclusive_scan(eq_sum, &eq_tot);
        const uint32_t take_run = need_eq > eq_pre ? min(need_eq - eq_pre, eq_sum) : 0u;
        uint32_t sel_tot;
        const uint32_t sel_pre = sel_before + block_exclusive_scan(gt_sum + take_run, &sel_tot);
        uint32_t eq_run = eq_pre, sel_run = sel_pre;
#pragma unroll
        for (uint32_t u = 0; u < kScanRun; ++u) {
            if (t0 + u >= t1) break;
            const uint32_t take = need_eq > eq_run ? min(need_eq - eq_run, e[u]) : 0u;
            w.ctake[seg.dchunk0 + t0 + u] = take;
            w.cout[seg.dchunk0 + t0 + u] = base + sel_run;
            eq_run += e[u];
            sel_run += g[u] + take;
        }
        eq_before += eq_tot;
        sel_before += sel_tot;
    }
    if (threadIdx.x == 0) {
        seg_off[s] = base;
        if (s == uint32_t(P.nseg - 1)) seg_off[P.nseg] = base + w.st[s].sent;
    }
}

// ------------------------------------------------------------------ emit
// Each of the wave's chunks in turn: staged entries in index order, 64 at a
// time; ties at T are taken in index order up to the chunk's quota; ranks
// from ballots.  DGC masks U and V at the sent entries.  kSignif also writes
// the chunk's words of the core bitmap (every word, zeros included: the
// chunk's 4096 entries start on a word boundary of the segment's run),
// assembled in LDS.  kExplore sends delta at the chosen entries.
template <int kMode, uint32_t CPW>
__global__ __launch_bounds__(kBlock) void dgc_emit_kernel(PlanDev P, Src a, DgcWs w,
                                                          uint32_t *__restrict__ out_idx,
                                                          float *__restrict__ out_val) {
    constexpr bool kDgc = kMode == kVanilla || kMode == kNesterov;
    const uint32_t c0 = wave_chunk0<CPW>();
    if (c0 >= P.ndchunk) return;
    const int lane = lane_id();
    const WaveChunks wc = wave_chunks<CPW>(P, w, c0);
    const uint32_t cl = min(c0 + uint32_t(lane) % CPW, P.ndchunk - 1);
    const SegState &sl = w.st[wc.rec.z];
    const uint32_t T_l = sl.T, take_l = w.ctake[cl], base_l = w.cout[cl];
    const uint32_t gt_l = kDgc ? w.cgt[cl] : 0u;
    // a segment owns message slots [base, base + sent): never write past them
    const uint32_t limit_l = sl.base + sl.sent;
    uint32_t id0[CPW];
    float v0[CPW];
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) {
        const uint32_t n = lane_val(wc.n, j);
        const uint32_t ic = lane_val(wc.rec.x, j) + (n ? min(uint32_t(lane), n - 1) : 0u);
        id0[j] = n ? w.sidx[ic] : 0u;
        v0[j] = n ? w.sval[ic] : 0.0f;
    }
    // a bitmap of the chunk's sent entries: Slim-DP's core writes it out; DGC
    // uses it to mask a chunk that sends many entries (below)
    __shared__ uint32_t cmask[kWaves][kMode == kSignif || kDgc ? kChunk / 32 : 1];
    uint32_t *cm = cmask[wave_id()];
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) {
        if (c0 + j >= P.ndchunk) break;
        const uint32_t n = lane_val(wc.n, j), lo = lane_val(wc.rec.x, j);
        // DGC masking of a chunk that sends at least kDenseMask entries (the
        // warm-up's first densities): the bitmap, then the chunk's U and V
        // rewritten whole, instead of two scattered 4-byte writes per entry
        const bool dense = kDgc && lane_val(gt_l, j) + lane_val(take_l, j) >= kDenseMask;
        if (kMode == kSignif || dense) {
            cm[lane] = 0u;
            cm[lane + kWave] = 0u;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
        } else if (n == 0) {
            continue;
        }
        const uint32_t T = lane_val(T_l, j), take = lane_val(take_l, j), base = lane_val(base_l, j);
        const uint32_t limit = lane_val(limit_l, j);
        uint32_t eq_run = 0, sel_run = 0;
        auto one = [&](uint32_t i, uint32_t id, float val) {
            const uint32_t key = mag_key(val);
            const bool in = i < n;
            const bool eq = in && key == T;
            const uint64_t eqm = __ballot(eq);
            const bool sel = (in && key > T) || (eq && eq_run + lane_rank(eqm) < take);
            const uint64_t selm = __ballot(sel);
            const uint32_t p = base + sel_run + lane_rank(selm);
            if (sel && p < limit) {
                out_idx[p] = id;
                out_val[p] = kMode == kExplore ? a.G[id] : val;
                if (kDgc && !dense) {
                    a.V[id] = 0.0f;
                    a.U[id] = 0.0f;
                }
                if (kMode == kSignif || dense) atomicOr(&cm[(id - lo) >> 5], 1u << ((id - lo) & 31u));
            }
            eq_run += static_cast<uint32_t>(__popcll(eqm));
            sel_run += static_cast<uint32_t>(__popcll(selm));
        };
        if (n) one(lane, id0[j], v0[j]);
        for (uint32_t i0 = kWave; i0 < n; i0 += 4 * kWave) {
            uint32_t id[4];
            float val[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t ic = lo + min(i0 + q * kWave + lane, n - 1);
                id[q] = w.sidx[ic];
                val[q] = w.sval[ic];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (i0 + q * kWave < n) one(i0 + q * kWave + lane, id[q], val[q]);
        }
        if (kMode == kSignif) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            const uint32_t wbase = P.seg[lane_val(wc.rec.z, j)].mbase + (lane_val(wc.rec.w, j) << (kChunkLog2 - 5));
            const uint32_t nw = (lane_val(wc.rec.y, j) + 31) / 32;
            for (uint32_t l = lane; l < nw; l += kWave) a.mask[wbase + l] = cm[l];
        }
        if (dense) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            // lane l holds elements [256 r + 4 l, +4) of rows r; four rows of U
            // and V in flight at a time
            const uint32_t cnt = lane_val(wc.rec.y, j);
            const BufRsrc ru = chunk_buf(a.U + lo, cnt), rv = chunk_buf(a.V + lo, cnt);
#pragma unroll
            for (int r0 = 0; r0 < kWaveRows; r0 += 4) {
                float u[4][4], v[4][4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t e0 = (r0 + r) * (4 * kWave) + 4u * lane;
                    load4(ru, e0, u[r]);
                    load4(rv, e0, v[r]);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const uint32_t e0 = (r0 + r) * (4 * kWave) + 4u * lane;
                    const uint32_t bits = cm[e0 >> 5] >> (e0 & 31u);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if ((bits >> q) & 1u) {
                            u[r][q] = 0.0f;
                            v[r][q] = 0.0f;
                        }
                    }
                    store4(ru, e0, u[r]);
                    store4(rv, e0, v[r]);
                }
            }
        }
    }
}

// ================================================================ exact path
// Exact DGC selection (vanilla and Nesterov) in five launches after the clip
// norm, for plans where every tensor of more than one chunk keeps at most
// 1/512 of its entries:
//   prepare (segment) the clip factor; V' at a sample of up to 16,384
//           entries; the staging bound Lkey and the width 2^fshift of the
//           fine bins above it (the bins reach the largest sampled key)
//   update  (chunk)   dgc_update_kernel<kMode, true>: U, V, the staging of
//           every key >= Lkey in the chunk's own slot, and the segment's
//           histogram of the staged keys by fine bin
//   collect (chunk)   T's bin off the histogram; each chunk's keys above and
//           in the bin, and the bin's keys to the segment's list
//   select  (segment) T from the list (three LDS radix passes); then each
//           chunk's message slots and tie quota, in index order
//   emit    (chunk)   the chunk's entries in index order, U and V masked
// Rare cases stay exact on slower branches of select: T's bin holding more
// keys than the list, or T above the fine bins (three radix passes over the
// staged keys), and fewer than k staged entries (the sample bound was too
// high: three radix passes over V, then the segment is staged again); those
// and segments past one round of the ordered scan with bins wider than one
// key count the chunks' keys at T again.
constexpr int kSelBlock = 1024;
constexpr uint32_t kSampleMax = 16384;  // sampled entries per tensor at most
constexpr uint32_t kPrepPer = kSampleMax / kSelBlock;
constexpr uint32_t kQuadRun = 10;       // chunks per quad of lanes in a round of a per-chunk pass
constexpr uint32_t kWalkChunks = kSelBlock / 4 * kQuadRun;  // chunks per round of a per-chunk pass
constexpr uint32_t kSelScanRun = 5;                         // chunks per thread in a round of the ordered scan
constexpr uint32_t kSelChunks = kSelBlock * kSelScanRun;   // chunks per round of the ordered scan, and
                                                            // of per-chunk values kept in LDS
constexpr uint32_t kThreadN = 128;      // staged entries one thread counts; more: a wave
constexpr uint32_t kFastDensity = 512;  // exact path when k_s * 512 <= n_s (or one chunk)
constexpr uint32_t kGatherBig = kXListCap / kSamples;  // chunks with more than kSamples keys in T's bin, at most
static_assert(2 * kGatherBig <= kWalkChunks, "select's gather keeps those chunks in the walk's LDS list");

// Sample of a tensor for the exact path: one chunk, all of it; up to 512
// chunks, a block of sc = min(4096, (16384 / chunks) rounded down to 32)
// contiguous entries per chunk; more chunks, 32 entries of every stride-th
// chunk.  Full chunks start their block at min(128 ((13 c) mod 32),
// 4096 - sc) (c the plan-wide chunk number), a partial last chunk at 0.
struct SampleShape {
    uint32_t stride, nsc, sc, total, last_cnt;
};
__device__ __forceinline__ SampleShape sample_shape(const SegDev &seg) {
    SampleShape z;
    if (seg.dnchunk == 1) {
        z.stride = 1;
        z.nsc = 1;
        z.sc = seg.len;
    } else if (seg.dnchunk <= kSampleChunks) {
        z.stride = 1;
        z.nsc = seg.dnchunk;
        z.sc = min(uint32_t(kChunk), (kSampleMax / seg.dnchunk) & ~(kSamples - 1));
    } else {
        z.stride = sample_stride(seg.dnchunk);
        z.nsc = (seg.dnchunk + z.stride - 1) / z.stride;
        z.sc = kSamples;
    }
    z.last_cnt = min(seg.len - (z.nsc - 1) * z.stride * uint32_t(kChunk), uint32_t(kChunk));
    z.total = (z.nsc - 1) * z.sc + min(z.sc, z.last_cnt);
    return z;
}

template <int kMode>
__global__ __launch_bounds__(kSelBlock) void dgc_prepare_kernel(PlanDev P, Src a, DgcWs w, int use_clip,
                                                                 float thr) {
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    const uint32_t k = seg_k(seg, w);
    // the update adds every staged key to the fine histogram
    uint32_t *xt = xtables(w, s);
    for (int i = threadIdx.x; i < int(kFineBins); i += kSelBlock) xt[i] = 0u;
    // the sample's G, U, V first (in flight during the clip factor's tree);
    // sample q = sc j + l is entry l of sampled chunk j, thread t takes
    // q = t, t + 1024, ...
    const SampleShape z = sample_shape(seg);
    float gs[kPrepPer], us[kPrepPer], vs[kPrepPer];
    uint32_t valid = 0;
#pragma unroll
    for (uint32_t u = 0; u < kPrepPer; ++u) {
        const uint32_t q = u * kSelBlock + threadIdx.x;
        gs[u] = us[u] = vs[u] = 0.0f;
        if (q < z.total) {
            const uint32_t j = q / z.sc, l = q - j * z.sc;
            const uint32_t cnt = j + 1 < z.nsc ? uint32_t(kChunk) : z.last_cnt;
            const uint32_t off = cnt == uint32_t(kChunk)
                                     ? min(sample_offset(seg.dchunk0 + j * z.stride, cnt), uint32_t(kChunk) - z.sc)
                                     : 0u;
            const uint64_t e = seg.off + (uint64_t(j * z.stride) << kChunkLog2) + off + l;
            gs[u] = a.G[e];
            us[u] = a.U[e];
            vs[u] = a.V[e];
            valid |= 1u << u;
        }
    }
    float cl = 1.0f;
    if (use_clip) {
        const double *part = w.partial + seg.dchunk0;
        const double S = block_pairwise_sum<kSelBlock>(seg.dnchunk, [&](uint64_t g) { return part[g]; });
        const double norm = sqrt(S);
        if (norm > static_cast<double>(thr)) cl = static_cast<float>(static_cast<double>(thr) / norm);
    }
    uint32_t key[kPrepPer], kmax = 0;
#pragma unroll
    for (uint32_t u = 0; u < kPrepPer; ++u) {
        const float gc = cl * gs[u];
        float un = us[u], vn = vs[u];
        momentum_update<kMode>(a.m, gc, un, vn);
        key[u] = mag_key(vn);
        if ((valid >> u) & 1u) kmax = max(kmax, key[u]);
    }
    __shared__ uint32_t h[kHist1];
    __shared__ uint32_t wmax[kSelBlock / kWave];
    kmax = wave_max_all(kmax);
    if (lane_id() == 0) wmax[wave_id()] = kmax;
    __syncthreads();
    uint32_t Hkey = 0;
    for (int i = 0; i < kSelBlock / kWave; ++i) Hkey = max(Hkey, wmax[i]);
    // Lkey: the (E + 4 sqrt(E) + 16)-th largest sample key rounded down to its
    // 22-bit prefix, with E = total k / n the expected sampled top-k entries
    // (0, stage everything, when the sample is too small for that)
    const double E = double(z.total) * double(k) / double(seg.len);
    const double target = E + 4.0 * sqrt(E) + 16.0;
    uint32_t Lkey = 0;
    if (target < double(z.total)) {
        uint32_t rank = static_cast<uint32_t>(target), prefix = 0;
        for (int level = 0; level < 2; ++level) {
            for (int i = threadIdx.x; i < kHist1; i += kSelBlock) h[i] = 0u;
            __syncthreads();
#pragma unroll
            for (uint32_t u = 0; u < kPrepPer; ++u) {
                const uint32_t d1 = key[u] >> (kDigit2Bits + kDigit3Bits);
                lds_hist_add(h, ((valid >> u) & 1u) && (level == 0 || d1 == prefix),
                             level == 0 ? d1 : (key[u] >> kDigit3Bits) & (kHist2 - 1));
            }
            __syncthreads();
            uint32_t above;
            const uint32_t d = block_find_bucket<kHist1, kSelBlock>(rank, [&](int b) { return h[b]; }, &above);
            rank -= above;
            prefix = level == 0 ? d : ((prefix << kDigit2Bits) | d);
            __syncthreads();
        }
        Lkey = prefix << kDigit3Bits;
    }
    if (threadIdx.x == 0) {
        SegState &st = w.st[s];
        st.clip = cl;
        st.Lkey = Lkey;
        st.fshift = fine_shift(Lkey, Hkey);
        st.sent = k;
        st.base = seg.kbase;
        st.redo = 0u;
        st.all = 0u;
    }
}

// Per-chunk values over the staged keys of a segment's chunks [r0, r1):
// settle(i, n, &v) may give chunk i's value without its keys; otherwise
// v = sum of count(key) over its staged keys (two u16 counts in a u32, so
// count may also record keys elsewhere); then store(i, v).  Four lanes (a
// quad) share a chunk, so one wave load covers 16 chunks' first 16 keys in 16
// lines (a chunk's staged keys start its 16 KB slot): quad Q takes the chunks
// [r0 + Q per, +per), per <= kQuadRun, loads all their counts, then 16 keys
// of every one of them per round of loads (a chunk holds some 13 at the 0.1%
// density of the pages).  A chunk of more than kThreadN staged entries goes
// to a list whose chunks are counted one per wave, 1024 keys per round.
template <class Settle, class Count, class Store>
__device__ __forceinline__ void sel_walk_round(const SegDev &seg, const DgcWs &w, uint32_t r0, uint32_t r1,
                                               Settle settle, Count count, Store store, uint32_t *big,
                                               uint32_t *nbig) {
    if (threadIdx.x == 0) *nbig = 0u;
    __syncthreads();
    const uint32_t quad = threadIdx.x >> 2, ql = threadIdx.x & 3u;
    const uint32_t per = (r1 - r0 + kSelBlock / 4 - 1) / (kSelBlock / 4);  // <= kQuadRun
    const uint32_t t0 = r0 + quad * per;
    uint32_t n[kQuadRun], v[kQuadRun];
    uint32_t need = 0;  // bit b: chunk t0 + b is counted by the quad
#pragma unroll
    for (uint32_t b = 0; b < kQuadRun; ++b) {
        const uint32_t i = t0 + b;
        const bool act = b < per && i < r1;
        n[b] = act ? min(w.ccount[seg.dchunk0 + i], min(uint32_t(kChunk), seg.len - (i << kChunkLog2))) : 0u;
    }
#pragma unroll
    for (uint32_t b = 0; b < kQuadRun; ++b) {
        const uint32_t i = t0 + b;
        v[b] = 0u;
        if (b < per && i < r1 && !settle(i, n[b], &v[b])) {
            if (n[b] > kThreadN) {
                if (ql == 0) big[atomicAdd(nbig, 1u)] = i;
            } else {
                need |= 1u << b;
            }
        }
    }
    auto add4 = [&](uint32_t &acc, const uint4 &q, uint32_t e, uint32_t nn) {
        if (e < nn) acc += count(q.x & 0x7FFFFFFFu);
        if (e + 1 < nn) acc += count(q.y & 0x7FFFFFFFu);
        if (e + 2 < nn) acc += count(q.z & 0x7FFFFFFFu);
        if (e + 3 < nn) acc += count(q.w & 0x7FFFFFFFu);
    };
    uint32_t nmax = 0;
#pragma unroll
    for (uint32_t b = 0; b < kQuadRun; ++b) nmax = max(nmax, ((need >> b) & 1u) ? n[b] : 0u);
    for (uint32_t q0 = 0; q0 < nmax; q0 += 16) {
        uint4 x[kQuadRun];
#pragma unroll
        for (uint32_t b = 0; b < kQuadRun; ++b) {
            const bool ld = ((need >> b) & 1u) && q0 < n[b];
            const uint4 *src = reinterpret_cast<const uint4 *>(
                w.sval + (size_t(seg.dchunk0 + (ld ? t0 + b : 0u)) << kChunkLog2));
            x[b] = ld ? src[(q0 >> 2) + ql] : make_uint4(0u, 0u, 0u, 0u);  // inside the chunk's 4096-entry slot
        }
#pragma unroll
        for (uint32_t b = 0; b < kQuadRun; ++b)
            if ((need >> b) & 1u) add4(v[b], x[b], q0 + 4 * ql, n[b]);
    }
    // the quad's four partial counts of each chunk
#pragma unroll
    for (uint32_t b = 0; b < kQuadRun; ++b) {
        if ((need >> b) & 1u) {
            v[b] += __shfl_xor(v[b], 1);
            v[b] += __shfl_xor(v[b], 2);
        }
    }
    // (the shuffles above run in every lane of a quad alike: need, n and per
    // are the quad's)
#pragma unroll
    for (uint32_t b = 0; b < kQuadRun; ++b)
        if (ql == 0 && b < per && t0 + b < r1) store(t0 + b, v[b]);
    __syncthreads();
    const uint32_t nb = *nbig;
    const int lane = lane_id();
    for (uint32_t bi = wave_id(); bi < nb; bi += kSelBlock / kWave) {
        const uint32_t i = big[bi];
        const uint32_t nn = min(w.ccount[seg.dchunk0 + i], min(uint32_t(kChunk), seg.len - (i << kChunkLog2)));
        const uint4 *src = reinterpret_cast<const uint4 *>(w.sval + (size_t(seg.dchunk0 + i) << kChunkLog2));
        uint32_t acc = 0;
        for (uint32_t q0 = 0; q0 < nn; q0 += 4 * 4 * kWave) {
            uint4 y[4];
#pragma unroll
            for (uint32_t u = 0; u < 4; ++u) y[u] = src[min((q0 >> 2) + u * kWave + lane, uint32_t(kChunk / 4 - 1))];
#pragma unroll
            for (uint32_t u = 0; u < 4; ++u) add4(acc, y[u], q0 + 4 * (u * kWave + lane), nn);
        }
        acc = wave_total(acc);
        if (lane == 0) store(i, acc);
    }
    __syncthreads();
}

template <class Settle, class Count, class Store>
__device__ __forceinline__ void sel_walk(const SegDev &seg, const DgcWs &w, uint32_t r0, uint32_t r1,
                                         Settle settle, Count count, Store store, uint32_t *big, uint32_t *nbig) {
    for (uint32_t q0 = r0; q0 < r1; q0 += kWalkChunks)
        sel_walk_round(seg, w, q0, min(r1, q0 + kWalkChunks), settle, count, store, big, nbig);
}

// The rank-th largest key (1 <= rank <= keys visited) among the keys that
// each(f) visits (f(key) for every key, from whichever threads), by three
// LDS histogram passes over the 11, 11 and 9-bit digits.  *gt receives the
// number of keys above it.
template <class Each>
__device__ __forceinline__ uint32_t sel_radix(uint32_t rank, Each each, uint32_t *h, uint32_t *gt) {
    uint32_t prefix = 0, above_all = 0;
    for (int level = 0; level < 3; ++level) {
        const int nb = level == 2 ? kHist3 : kHist1;
        const int shift = level == 0 ? kDigit2Bits + kDigit3Bits : level == 1 ? kDigit3Bits : 0;
        const int pshift = level == 1 ? kDigit2Bits + kDigit3Bits : kDigit3Bits;
        for (int i = threadIdx.x; i < nb; i += kSelBlock) h[i] = 0u;
        __syncthreads();
        each([&](uint32_t key) {
            if (level == 0 || (key >> pshift) == prefix) atomicAdd(&h[(key >> shift) & uint32_t(nb - 1)], 1u);
        });
        __syncthreads();
        uint32_t above, d;
        if (level == 2) d = block_find_bucket<kHist3, kSelBlock>(rank, [&](int b) { return h[b]; }, &above);
        else d = block_find_bucket<kHist1, kSelBlock>(rank, [&](int b) { return h[b]; }, &above);
        rank -= above;
        above_all += above;
        prefix = level == 0 ? d : level == 1 ? ((prefix << kDigit2Bits) | d) : ((prefix << kDigit3Bits) | d);
        __syncthreads();
    }
    *gt = above_all;
    return prefix;
}

// One workgroup per collect block (up to kXBlockChunks chunks of one
// segment, a quarter per wave): T's fine bin b* is found once from the
// segment's histogram (256 threads, 8 bins each: fewer than k staged keys in
// the bins above b*, at least k in b* and above); then each chunk's staged
// keys above b* (low u16) and in it (high u16) go to cpack, and (bins wider
// than one key) its first kSamples keys in the bin, in staging order, to its
// row of skey (select gathers the rows; a chunk with more in the bin is read
// again there).  Segments whose selection takes a slower branch of select
// (fewer than k staged keys, b* the last bin, or more keys in b* than the
// list holds) are skipped, and so are those where every staged key equals T
// (bins of one key, all of them in b*).  Each wave reads the first 64 staged keys of its
// chunks with their counts, before b* is known (a chunk's 4096-entry slot is
// always there to read; keys past the staged count are ignored).  (Appending
// the bin's keys to one list per segment through a shared counter, or
// finding the bin per wave from the whole histogram, took 20 us on the
// DeepSpeech sizes.)
constexpr uint32_t kXCollectCpw = kXBlockChunks / kWaves;
struct FineBin {
    uint32_t bstar, above, in;
    bool ok;
};
__global__ __launch_bounds__(kBlock) void dgc_xcollect_kernel(PlanDev P, DgcWs w) {
    const uint2 blk = P.xblock[blockIdx.x];
    const uint32_t s = blk.x;
    const SegDev seg = P.seg[s];
    const uint32_t cend = seg.dchunk0 + seg.dnchunk;  // the segment's chunks end here
    const uint32_t lane = lane_id();
    const uint32_t c0 = blk.y + wave_id() * kXCollectCpw;
    const uint32_t cl = min(c0 + lane % kXCollectCpw, cend - 1);
    const uint32_t my_n = min(w.ccount[cl], P.dchunk_rec[cl].y);
    uint32_t key0[kXCollectCpw];
#pragma unroll
    for (uint32_t j = 0; j < kXCollectCpw; ++j)
        key0[j] = mag_key(w.sval[(size_t(min(c0 + j, cend - 1)) << kChunkLog2) + lane]);
    const uint32_t k = seg_k(seg, w);
    const uint32_t Lkey = w.st[s].Lkey, fs = w.st[s].fshift;
    // thread t holds bins [2040 - 8 t, 2048 - 8 t): thread 0 the highest
    __shared__ FineBin sh_fb;
    const uint32_t b0 = kFineBins - 8u * (threadIdx.x + 1u);
    const uint4 *h4 = reinterpret_cast<const uint4 *>(xtables(w, s) + b0);
    const uint4 qa = h4[0], qb = h4[1];
    const uint32_t hv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    uint32_t tsum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) tsum += hv[i];
    if (threadIdx.x == 0) sh_fb = FineBin{0u, 0u, 0u, false};
    uint32_t total;
    const uint32_t pre = block_exclusive_scan<uint32_t, kBlock>(tsum, &total);
    if (total >= k && pre < k && pre + tsum >= k) {
        uint32_t acc = pre;
        bool found = false;
#pragma unroll
        for (int i = 7; i >= 0; --i) {
            if (!found && acc + hv[i] >= k) {
                found = true;
                const uint32_t bs = b0 + i;
                sh_fb = FineBin{bs, acc, hv[i], bs != kFineBins - 1 && (fs == 0 || bs == 0 || hv[i] <= kXListCap)};
            }
            acc += hv[i];
        }
    }
    __syncthreads();
    const FineBin fb = sh_fb;
    // nothing to collect: T's bin unusable here, or (bins of one key) every
    // staged key in T's bin, where select takes each chunk's staged count
    const bool one_key = fs == 0 || fb.bstar == 0;  // T's bin holds one key
    if (!fb.ok || (one_key && fb.in == total)) return;
#pragma unroll
    for (uint32_t j = 0; j < kXCollectCpw; ++j) {
        const uint32_t c = c0 + j;
        if (c >= cend) break;
        const uint32_t n = lane_val(my_n, j);
        uint32_t gt = 0, in = 0;
        auto count = [&](uint32_t i, uint32_t key) {
            const uint32_t b = fine_bin(key, Lkey, fs);
            const bool valid = i < n;
            const bool inb = valid && b == fb.bstar;
            const uint64_t gtm = __ballot(valid && b > fb.bstar);
            const uint64_t inm = __ballot(inb);
            const uint32_t at = in + lane_rank(inm);
            if (!one_key && inb && at < kSamples) w.skey[size_t(c) * kSamples + at] = key;
            gt += static_cast<uint32_t>(__popcll(gtm));
            in += static_cast<uint32_t>(__popcll(inm));
        };
        count(lane, key0[j]);
        // a chunk of many staged keys (a tensor of near-zeros stages every
        // entry): the rest four batches of loads at a time
        const uint32_t *sv = reinterpret_cast<const uint32_t *>(w.sval) + (size_t(c) << kChunkLog2);
        for (uint32_t i0 = kWave; i0 < n; i0 += 4 * kWave) {
            uint32_t key[4];
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q) key[q] = sv[min(i0 + q * kWave + lane, uint32_t(kChunk) - 1)] & 0x7FFFFFFFu;
#pragma unroll
            for (uint32_t q = 0; q < 4; ++q)
                if (i0 + q * kWave < n) count(i0 + q * kWave + lane, key[q]);
        }
        if (lane == 0) w.cpack[c] = gt | (in << 16);
    }
}

// The rank-th largest (1 <= rank <= m) of the m <= kWaveSel keys list[0, m),
// all in [lo, lo + 2^fs), by one wave: the fs bits of key - lo from the
// highest, each set when at least rank keys match the prefix with it set
// (else rank drops by that count).  *gt_out: the keys above the result.
constexpr uint32_t kWaveSel = 512;
__device__ __forceinline__ uint32_t wave_select(const uint32_t *list, uint32_t m, uint32_t lo, uint32_t fs,
                                                uint32_t rank, uint32_t *gt_out) {
    constexpr uint32_t kPer = kWaveSel / kWave;
    const uint32_t lane = lane_id();
    uint32_t x[kPer];  // key - lo (< 2^31), or ~0u past the list
#pragma unroll
    for (uint32_t q = 0; q < kPer; ++q) {
        const uint32_t i = q * kWave + lane;
        x[q] = i < m ? list[i] - lo : ~0u;
    }
    uint32_t prefix = 0;
    for (int bit = int(fs) - 1; bit >= 0; --bit) {
        const uint32_t want = (prefix >> bit) | 1u;
        uint32_t cnt = 0;
#pragma unroll
        for (uint32_t q = 0; q < kPer; ++q) cnt += static_cast<uint32_t>(__popcll(__ballot((x[q] >> bit) == want)));
        if (cnt >= rank) prefix |= 1u << bit;
        else rank -= cnt;
    }
    uint32_t g = 0;
#pragma unroll
    for (uint32_t q = 0; q < kPer; ++q) g += static_cast<uint32_t>(__popcll(__ballot(x[q] != ~0u && x[q] > prefix)));
    *gt_out = g;
    return lo + prefix;
}

// One workgroup per segment.  kSampled (sampled selection): the staged keys
// are those at or above the sample's estimate; when they fit the budget
// min(n, over k) they are all sent (each chunk's slots from the staged counts
// alone), otherwise the exact top-k among them is taken as below.  Slots are
// then relative to the segment, whose base sbase lays out afterwards.
// The common case (at least k staged keys, T's
// fine bin below the last and holding at most kXListCap keys, the segment's
// chunks in one round of kSelChunks): thread t's chunks [t per, +per) have
// their staged counts and collect words loaded with two histogram bins; one
// scan gives T's bin and each thread's first place in the list of the bin's
// keys; T is taken from the list (one wave when it is short); the keys at and
// above T in the bin go back to their chunks (LDS atomics); the per-chunk
// words wait in LDS (cpk, cnn) meanwhile; one more scan of
// the counts above and at T gives every chunk's first slot and tie quota:
// the quota of thread t's chunks is what the ties of the chunks before them
// leave, and the ties taken before them are min(need_eq, ties before them).
template <int kMode, bool kSampled>
__global__ __launch_bounds__(kSelBlock) void dgc_xselect_kernel(PlanDev P, Src a, DgcWs w,
                                                                 uint32_t *__restrict__ seg_off, uint32_t over) {
    static_assert(kFineBins == 2 * kSelBlock, "two histogram bins per thread");
    const uint32_t s = blockIdx.x;
    const SegDev seg = P.seg[s];
    const uint32_t k = w.st[s].sent, Lkey = w.st[s].Lkey, fs = w.st[s].fshift;
    const uint32_t base = kSampled ? 0u : w.st[s].base;
    const uint32_t nch = seg.dnchunk, c0 = seg.dchunk0;
    __shared__ uint32_t h[kFineBins];
    __shared__ uint32_t list[kXListCap];
    __shared__ uint32_t lch[kXListCap];
    __shared__ uint32_t cpk[kSelChunks];
    __shared__ uint32_t cnn[kSelChunks];  // one-round segments: staged count of each chunk
    __shared__ uint32_t big[kWalkChunks];
    __shared__ uint32_t sh_nbig, sh_bstar, sh_above, sh_cnt, sh_T, sh_gtin;
    // per-chunk values: LDS when one round covers the segment, else the workspace
    const bool one_round = nch <= kSelChunks;
    auto pk_store = [&](uint32_t i, uint32_t v) {
        if (one_round) cpk[i] = v;
        else w.cpack[c0 + i] = v;
    };
    auto pk_load = [&](uint32_t i) { return one_round ? cpk[i] : w.cpack[c0 + i]; };
    auto chunk_len = [&](uint32_t i) { return min(uint32_t(kChunk), seg.len - (i << kChunkLog2)); };
    auto bin_of = [&](uint32_t key) { return fine_bin(key, Lkey, fs); };
    auto never = [](uint32_t, uint32_t, uint32_t *) { return false; };
    auto each_staged = [&](auto f) {
        sel_walk(
            seg, w, 0, nch, never,
            [&](uint32_t key) {
                f(key);
                return 0u;
            },
            [](uint32_t, uint32_t) {}, big, &sh_nbig);
    };
    // the keys in T's bin of thread t's chunks [t0, t0 + per) (collect words
    // pkr) to the LDS list from place `at`: a chunk's skey row, or a wave per
    // chunk with more than kSamples of them (fewer than kGatherBig chunks)
    auto gather = [&](const uint32_t (&pkr)[kSelScanRun], uint32_t t0, uint32_t at, uint32_t bstar) {
        if (threadIdx.x == 0) sh_nbig = 0u;
        __syncthreads();
#pragma unroll
        for (uint32_t b = 0; b < kSelScanRun; ++b) {
            const uint32_t e = pkr[b] >> 16, i = t0 + b;
            if (e > kSamples) {
                const uint32_t bi = atomicAdd(&sh_nbig, 1u);
                if (bi < kGatherBig) {
                    big[bi] = i;
                    big[kGatherBig + bi] = at;
                }
            } else {
                const uint32_t *row = w.skey + size_t(c0 + i) * kSamples;
                for (uint32_t q = 0; q < e; ++q)
                    if (at + q < kXListCap) {
                        list[at + q] = row[q];
                        lch[at + q] = i;
                    }
            }
            at += e;
        }
        __syncthreads();
        const uint32_t nb = min(sh_nbig, kGatherBig);
        const uint32_t lane = lane_id();
        for (uint32_t bi = wave_id(); bi < nb; bi += kSelBlock / kWave) {
            const uint32_t i = big[bi];
            uint32_t pos = big[kGatherBig + bi];
            const uint32_t n = min(w.ccount[c0 + i], chunk_len(i));
            for (uint32_t i0 = 0; i0 < n; i0 += kWave) {
                const uint32_t j = i0 + lane;
                const uint32_t key = j < n ? mag_key(w.sval[(size_t(c0 + i) << kChunkLog2) + j]) : 0u;
                const bool inb = j < n && bin_of(key) == bstar;
                const uint64_t mk = __ballot(inb);
                const uint32_t q = pos + lane_rank(mk);
                if (inb && q < kXListCap) {
                    list[q] = key;
                    lch[q] = i;
                }
                pos += static_cast<uint32_t>(__popcll(mk));
            }
        }
        __syncthreads();
    };

    // one round of loads: a one-round segment's staged counts and collect
    // words of thread t's chunks (to cnn and cpk), and bins 2047 - 2t and
    // 2046 - 2t
    const uint32_t per1 = one_round ? (nch + kSelBlock - 1) / kSelBlock : 0u;
    const uint32_t t1 = threadIdx.x * per1;
    uint32_t in_sum = 0;
    {
        uint32_t nn[kSelScanRun], pk[kSelScanRun];
#pragma unroll
        for (uint32_t b = 0; b < kSelScanRun; ++b) {
            const uint32_t i = t1 + b;
            const bool act = b < per1 && i < nch;
            nn[b] = act ? min(w.ccount[c0 + i], chunk_len(i)) : 0u;
            pk[b] = act ? w.cpack[c0 + i] : 0u;
        }
#pragma unroll
        for (uint32_t b = 0; b < kSelScanRun; ++b) {
            const uint32_t i = t1 + b;
            if (b < per1 && i < nch) {
                cnn[i] = nn[b];
                cpk[i] = pk[b];
            }
            in_sum += pk[b] >> 16;
        }
    }
    const uint2 hp = reinterpret_cast<const uint2 *>(xtables(w, s))[kFineBins / 2 - 1 - threadIdx.x];
    const uint32_t hsum = hp.x + hp.y;
    uint64_t tot64;
    const uint64_t pre64 =
        block_exclusive_scan<uint64_t, kSelBlock>(uint64_t(hsum) | (uint64_t(in_sum) << 32), &tot64);
    const uint32_t staged = static_cast<uint32_t>(tot64);  // every staged key is in the histogram once
    uint32_t T, gt;
    bool have_pk = false;  // pk_load(i): chunk i's keys above T's bin (low) and in it (high)
    bool pk_done = false;  // cpk: each chunk's keys above T (low) and at T (high), one round
    bool all_eq = false;   // every staged key equals T
    // sampled selection: every staged entry is sent
    const bool send_all = kSampled && uint64_t(staged) <= umin64(seg.len, uint64_t(over) * k);
    if (send_all) {
        // T = Lkey with every chunk's ties in its quota: the emit sends all
        // staged keys, each chunk's at the slots after the chunks before it
        uint32_t run = 0;
        for (uint32_t r0 = 0; r0 < nch; r0 += kSelChunks) {
            const uint32_t r1 = min(nch, r0 + kSelChunks);
            const uint32_t per = (r1 - r0 + kSelBlock - 1) / kSelBlock;
            const uint32_t t0 = r0 + threadIdx.x * per;
            uint32_t nr[kSelScanRun], sum = 0;
#pragma unroll
            for (uint32_t b = 0; b < kSelScanRun; ++b) {
                const uint32_t i = t0 + b;
                nr[b] = b < per && i < r1 ? min(w.ccount[c0 + i], chunk_len(i)) : 0u;
                sum += nr[b];
            }
            uint32_t tot;
            uint32_t at = run + block_exclusive_scan<uint32_t, kSelBlock>(sum, &tot);
#pragma unroll
            for (uint32_t b = 0; b < kSelScanRun; ++b) {
                const uint32_t i = t0 + b;
                if (b < per && i < r1) {
                    w.crec[c0 + i] = make_uint4(at, at + nr[b], Lkey, nr[b] | (nr[b] << 16));
                    at += nr[b];
                }
            }
            run += tot;
        }
        T = Lkey;
        gt = 0;
    } else if (staged < k) {
        // the sample bound was above the k-th key: select over V itself, then
        // stage every chunk's entries with key >= T again
        auto each_v = [&](auto f) {
            for (uint32_t i = 0; i < nch; ++i) {
                const uint32_t cnt = chunk_len(i);
                const BufRsrc rv = chunk_buf(a.V + seg.off + (uint64_t(i) << kChunkLog2), cnt);
                float v[4];
                load4(rv, 4u * threadIdx.x, v);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (4u * threadIdx.x + q < cnt) f(mag_key(v[q]));
            }
        };
        T = sel_radix(k, each_v, h, &gt);
        for (uint32_t i = 0; i < nch; ++i) {
            const uint32_t cnt = chunk_len(i);
            const uint64_t lo = seg.off + (uint64_t(i) << kChunkLog2);
            const BufRsrc rv = chunk_buf(a.V + lo, cnt);
            float v[4];
            load4(rv, 4u * threadIdx.x, v);
            bool f[4];
            uint32_t nf = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f[q] = 4u * threadIdx.x + q < cnt && mag_key(v[q]) >= T;
                nf += f[q] ? 1u : 0u;
            }
            uint32_t tot;
            uint32_t slot = block_exclusive_scan<uint32_t, kSelBlock>(nf, &tot);
            const size_t sbase = size_t(c0 + i) << kChunkLog2;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (f[q]) {
                    w.sidx[sbase + slot] = static_cast<uint32_t>(lo) + 4u * threadIdx.x + q;
                    w.sval[sbase + slot] = v[q];
                    ++slot;
                }
            if (threadIdx.x == 0) w.ccount[c0 + i] = tot;
        }
        __syncthreads();
    } else {
        // T's fine bin: thread t holds bins 2047 - 2t (first) and 2046 - 2t
        const uint32_t hpre = static_cast<uint32_t>(pre64);
        if (hpre < k && hpre + hsum >= k) {
            const bool hi = hpre + hp.y >= k;
            sh_bstar = kFineBins - 1 - 2 * threadIdx.x - (hi ? 0u : 1u);
            sh_above = hi ? hpre : hpre + hp.y;
            sh_cnt = hi ? hp.y : hp.x;
        }
        __syncthreads();
        const uint32_t bstar = sh_bstar, above = sh_above, cnt_b = sh_cnt;
        const bool one_key = fs == 0 || bstar == 0;  // T's fine bin holds one key
        if (bstar == kFineBins - 1 || (!one_key && cnt_b > kXListCap)) {
            // T above the fine bins, or its bin too full for the list
            T = sel_radix(k, each_staged, h, &gt);
        } else if (one_key && cnt_b == staged) {
            T = Lkey + bstar;  // a bin of one key (fs = 0, or Lkey's own), and every staged key in it
            gt = 0;
            all_eq = true;
            if (one_round) {
#pragma unroll
                for (uint32_t b = 0; b < kSelScanRun; ++b)
                    if (b < per1 && t1 + b < nch) cpk[t1 + b] = cnn[t1 + b] << 16;
                pk_done = true;
            }
        } else if (one_key) {
            // a bin of one key: the collect words count the keys above T and at T
            T = Lkey + bstar;
            gt = above;
            have_pk = true;
            pk_done = one_round;
        } else {
            // the collect kernel left each chunk's keys above T's bin (low
            // u16) and in it (high u16) in cpack, and up to kSamples of the
            // bin's keys in its skey row
            have_pk = true;
            uint32_t m;
            if (one_round) {
                m = min(static_cast<uint32_t>(tot64 >> 32), kXListCap);
                uint32_t pk[kSelScanRun];
#pragma unroll
                for (uint32_t b = 0; b < kSelScanRun; ++b) {
                    const bool act = b < per1 && t1 + b < nch;
                    pk[b] = act ? cpk[t1 + b] : 0u;
                    if (act) cpk[t1 + b] = pk[b] & 0xFFFFu;
                }
                gather(pk, t1, static_cast<uint32_t>(pre64 >> 32), bstar);
            } else {
                m = 0;
                for (uint32_t r0 = 0; r0 < nch; r0 += kSelChunks) {
                    const uint32_t r1 = min(nch, r0 + kSelChunks);
                    const uint32_t per = (r1 - r0 + kSelBlock - 1) / kSelBlock;
                    const uint32_t t0 = r0 + threadIdx.x * per;
                    uint32_t pkr[kSelScanRun], sum = 0;
#pragma unroll
                    for (uint32_t b = 0; b < kSelScanRun; ++b) {
                        const uint32_t i = t0 + b;
                        pkr[b] = b < per && i < r1 ? w.cpack[c0 + i] : 0u;
                        sum += pkr[b] >> 16;
                    }
                    uint32_t tot;
                    const uint32_t at = m + block_exclusive_scan<uint32_t, kSelBlock>(sum, &tot);
                    gather(pkr, t0, at, bstar);
                    m += tot;
                }
                m = min(m, kXListCap);
            }
            uint32_t gt_in;
            if (m <= kWaveSel) {
                if (wave_id() == 0) {
                    uint32_t g;
                    const uint32_t t = wave_select(list, m, fine_lo(bstar, Lkey, fs), fs, k - above, &g);  // bstar >= 1
                    if (lane_id() == 0) {
                        sh_T = t;
                        sh_gtin = g;
                    }
                }
                __syncthreads();
                T = sh_T;
                gt_in = sh_gtin;
            } else {
                T = sel_radix(k - above, [&](auto f) {
                    for (uint32_t i = threadIdx.x; i < m; i += kSelBlock) f(list[i]);
                }, h, &gt_in);
            }
            gt = above + gt_in;
            if (one_round) {
                // the bin's keys above and at T, back to their chunks
                for (uint32_t i = threadIdx.x; i < m; i += kSelBlock) {
                    const uint32_t key = list[i];
                    if (key > T) atomicAdd(&cpk[lch[i]], 1u);
                    else if (key == T) atomicAdd(&cpk[lch[i]], 1u << 16);
                }
                __syncthreads();
                pk_done = true;
            }
        }
    }
    const uint32_t need_eq = send_all ? 0xFFFFFFFFu : k - gt;
    if (send_all) {
        // the records are written
    } else if (pk_done) {
        // the ordered scan of a one-round segment from cpk and cnn
        uint32_t pk[kSelScanRun], eq_sum = 0, gt_sum = 0;
#pragma unroll
        for (uint32_t b = 0; b < kSelScanRun; ++b) {
            pk[b] = b < per1 && t1 + b < nch ? cpk[t1 + b] : 0u;
            eq_sum += pk[b] >> 16;
            gt_sum += pk[b] & 0xFFFFu;
        }
        uint64_t tot2;
        const uint64_t pre2 = block_exclusive_scan<uint64_t, kSelBlock>(uint64_t(gt_sum) | (uint64_t(eq_sum) << 32), &tot2);
        uint32_t eq_run = static_cast<uint32_t>(pre2 >> 32);
        uint32_t sel_run = static_cast<uint32_t>(pre2) + min(need_eq, eq_run);
        // each chunk's first slot to cpk and staged count | quota << 16 to
        // cnn; then the records in chunk order, a chunk's end slot being the
        // next one's first (k after the last: the chunks send gt + need_eq)
#pragma unroll
        for (uint32_t b = 0; b < kSelScanRun; ++b) {
            const uint32_t i = t1 + b;
            if (b < per1 && i < nch) {
                const uint32_t e = pk[b] >> 16, g = pk[b] & 0xFFFFu;
                const uint32_t take = need_eq > eq_run ? min(need_eq - eq_run, e) : 0u;
                cpk[i] = sel_run;
                cnn[i] |= take << 16;
                eq_run += e;
                sel_run += g + take;
            }
        }
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < nch; i += kSelBlock)
            w.crec[c0 + i] = make_uint4(base + cpk[i], base + (i + 1 < nch ? cpk[i + 1] : k), T, cnn[i]);
    } else {
        // each chunk's keys above and at T (low and high u16), then the
        // ordered scan in rounds
        auto settle2 = [&](uint32_t i, uint32_t n, uint32_t *v) {
            if (n == 0) {
                *v = 0u;
                return true;
            }
            if (all_eq) {
                *v = n << 16;
                return true;
            }
            if (have_pk) {
                const uint32_t p = pk_load(i);
                // nothing in T's bin (its keys above the bin are above T), or
                // a bin of one key (its keys equal T): bins of one key, or T
                // in Lkey's own bin (a test on values already held: a flag
                // kept for it made the kernel spill 37 registers)
                if ((p >> 16) == 0 || fs == 0 || T == Lkey) {
                    *v = p;
                    return true;
                }
            }
            return false;
        };
        auto count2 = [&](uint32_t key) { return (key > T ? 1u : 0u) | (key == T ? 1u << 16 : 0u); };
        uint32_t eq_before = 0, sel_before = 0;
        for (uint32_t r0 = 0; r0 < nch; r0 += kSelChunks) {
            const uint32_t r1 = min(nch, r0 + kSelChunks);
            sel_walk(seg, w, r0, r1, settle2, count2, [&](uint32_t i, uint32_t v) { pk_store(i, v); }, big, &sh_nbig);
            // the round's chunks in order: thread t takes [r0 + t per, +per)
            const uint32_t per = (r1 - r0 + kSelBlock - 1) / kSelBlock;
            const uint32_t t0 = r0 + threadIdx.x * per;
            uint32_t pkr[kSelScanRun], nr[kSelScanRun];
            uint32_t eq_sum = 0, gt_sum = 0;
#pragma unroll
            for (uint32_t b = 0; b < kSelScanRun; ++b) {
                const uint32_t i = t0 + b;
                const bool act = b < per && i < r1;
                pkr[b] = act ? pk_load(i) : 0u;
                nr[b] = act ? min(w.ccount[c0 + i], chunk_len(i)) : 0u;
                eq_sum += pkr[b] >> 16;
                gt_sum += pkr[b] & 0xFFFFu;
            }
            uint64_t tot2;
            const uint64_t pre2 =
                block_exclusive_scan<uint64_t, kSelBlock>(uint64_t(gt_sum) | (uint64_t(eq_sum) << 32), &tot2);
            uint32_t eq_run = eq_before + static_cast<uint32_t>(pre2 >> 32);
            uint32_t sel_run = sel_before + static_cast<uint32_t>(pre2) + min(need_eq, eq_run) - min(need_eq, eq_before);
#pragma unroll
            for (uint32_t b = 0; b < kSelScanRun; ++b) {
                const uint32_t i = t0 + b;
                if (b < per && i < r1) {
                    const uint32_t e = pkr[b] >> 16, g = pkr[b] & 0xFFFFu;
                    const uint32_t take = need_eq > eq_run ? min(need_eq - eq_run, e) : 0u;
                    w.crec[c0 + i] = make_uint4(base + sel_run, base + sel_run + g + take, T, nr[b] | (take << 16));
                    eq_run += e;
                    sel_run += g + take;
                }
            }
            const uint32_t eq_all = eq_before + static_cast<uint32_t>(tot2 >> 32);
            sel_before += static_cast<uint32_t>(tot2) + min(need_eq, eq_all) - min(need_eq, eq_before);
            eq_before = eq_all;
            __syncthreads();
        }
    }
    if (threadIdx.x == 0) {
        w.st[s].T = T;
        w.st[s].gt = gt;
        w.st[s].need_eq = need_eq;
        if (kSampled) {
            w.st[s].all = send_all ? 1u : 0u;
            w.st[s].sent = send_all ? staged : k;
        } else {
            seg_off[s] = base;
            if (s == uint32_t(P.nseg - 1)) seg_off[P.nseg] = base + k;
        }
    }
}

// Each of the wave's chunks in turn (records and first entries of all CPW
// chunks loaded together): staged entries in index order, 64 at a time;
// entries above T are sent, ties at T up to the chunk's quota in index order;
// slots from ballots, never past the chunk's last slot; U and V masked at the
// sent entries.  Record: first slot, end slot, T, staged count | quota << 16.
// kSampled: the slots are relative to the segment's base (set by sbase).
template <int kMode, uint32_t CPW, bool kSampled>
__global__ __launch_bounds__(kBlock) void dgc_xemit_kernel(PlanDev P, Src a, DgcWs w,
                                                           uint32_t *__restrict__ out_idx,
                                                           float *__restrict__ out_val) {
    const uint32_t c0 = wave_chunk0<CPW>();
    if (c0 >= P.ndchunk) return;
    const int lane = lane_id();
    const uint32_t cl = min(c0 + uint32_t(lane) % CPW, P.ndchunk - 1);
    uint4 rec = w.crec[cl];
    if (kSampled) {
        const uint32_t sb = w.st[P.dchunk_rec[cl].z].base;
        rec.x += sb;
        rec.y += sb;
    }
    uint32_t id0[CPW];
    float v0[CPW];
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) {
        const bool any = lane_val(rec.y, j) != lane_val(rec.x, j);
        const uint32_t n = any ? min(lane_val(rec.w, j) & 0xFFFFu, uint32_t(kChunk)) : 0u;
        const size_t ic = (size_t(c0 + j) << kChunkLog2) + (n ? min(uint32_t(lane), n - 1) : 0u);
        id0[j] = n ? w.sidx[ic] : 0u;
        v0[j] = n ? w.sval[ic] : 0.0f;
    }
#pragma unroll
    for (uint32_t j = 0; j < CPW; ++j) {
        if (c0 + j >= P.ndchunk) break;
        const uint32_t base = lane_val(rec.x, j), limit = lane_val(rec.y, j);
        if (limit == base) continue;  // nothing to send
        const uint32_t n = min(lane_val(rec.w, j) & 0xFFFFu, uint32_t(kChunk));
        const uint32_t take = lane_val(rec.w, j) >> 16, T = lane_val(rec.z, j);
        const size_t lo = size_t(c0 + j) << kChunkLog2;
        uint32_t eq_run = 0, sel_run = 0;
        auto one = [&](uint32_t i, uint32_t id, float val) {
            const uint32_t key = mag_key(val);
            const bool in = i < n;
            const bool eq = in && key == T;
            const uint64_t eqm = __ballot(eq);
            const bool sel = (in && key > T) || (eq && eq_run + lane_rank(eqm) < take);
            const uint64_t selm = __ballot(sel);
            const uint32_t p = base + sel_run + lane_rank(selm);
            if (sel && p < limit) {
                out_idx[p] = id;
                out_val[p] = val;
                a.V[id] = 0.0f;
                a.U[id] = 0.0f;
            }
            eq_run += static_cast<uint32_t>(__popcll(eqm));
            sel_run += static_cast<uint32_t>(__popcll(selm));
        };
        one(lane, id0[j], v0[j]);
        for (uint32_t i0 = kWave; i0 < n; i0 += 4 * kWave) {
            uint32_t id[4];
            float val[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const size_t ic = lo + min(i0 + q * kWave + lane, n - 1);
                id[q] = w.sidx[ic];
                val[q] = w.sval[ic];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (i0 + q * kWave < n) one(i0 + q * kWave + lane, id[q], val[q]);
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

namespace gc {
// Whether exact DGC selection takes the four-launch path for these
// densities: every tensor of more than one chunk keeps at most 1/512 of its
// entries (denser selections stage more entries than one workgroup per
// tensor counts quickly, and take the candidate kernels).
bool dgc_exact_fast(const gc_plan *plan, uint32_t knum, uint32_t kden) {
    for (const SegDev &d : plan->seg) {
        if (d.len <= uint32_t(kChunk)) continue;
        if (uint64_t(seg_topk(d.len, d.k, knum, kden)) * kFastDensity > d.len) return false;
    }
    return true;
}
}  // namespace gc

namespace {
// Entries a message of this plan and selection holds at most.
uint64_t dgc_capacity(const gc_plan *plan, int select, uint32_t over, uint32_t knum = 0, uint32_t kden = 0) {
    if (select != GC_SELECT_SAMPLED) {
        if (kden == 0) return plan->total_k;
        uint64_t cap = 0;
        for (const SegDev &d : plan->seg) cap += seg_topk(d.len, d.k, knum, kden);
        return cap;
    }
    uint64_t cap = 0;
    for (const SegDev &d : plan->seg) cap += std::min<uint64_t>(d.len, uint64_t(over) * d.k);
    return cap;
}

// Host checks shared by the selection calls: message, workspace, alignment.
gc_status check_select_io(const char *fn, const gc_plan *plan, const gc_sparse *out, uint64_t cap,
                          const void *ws, size_t ws_bytes) {
    const std::string f(fn);
    if (!out || !out->idx || !out->val || !out->seg_off)
        return set_error(GC_EINVAL, f + ": out, out->idx, out->val, out->seg_off must be non-null");
    if (out->cap < cap) return set_error(GC_ECAPACITY, f + ": out->cap below the message size");
    if (!ws || ws_bytes < dgc_workspace_bytes(plan))
        return set_error(GC_ECAPACITY, f + ": workspace smaller than gc_plan_workspace_bytes(GC_OP_DGC)");
    if (reinterpret_cast<uintptr_t>(ws) % 256) return set_error(GC_EINVAL, f + ": workspace must be 256-byte aligned");
    return GC_OK;
}

// The radix select levels and the candidate kernels after the update, at
// CPW chunks per wave.
template <int kMode, uint32_t CPW>
void launch_candidates(const gc_plan *plan, const PlanDev &P, const DgcWs &w, const Src &src, bool sampled,
                       uint32_t over, gc_sparse *out, hipStream_t stream) {
    const unsigned segs = static_cast<unsigned>(plan->nseg);
    const unsigned cand_grid = grid_1d(plan->ndchunk, kWaves * CPW);
    GC_LAUNCH("dgc_select", stream, dgc_select_kernel<1><<<segs, kBlock, 0, stream>>>(P, w, sampled ? over : 0u));
    // the boundary bucket's digit-2 histogram in LDS per span of chunks, then
    // the re-staged segments
    GC_LAUNCH("dgc_stage", stream, dgc_stagew_kernel<<<grid_1d(plan->ndchunk, kStageSpan), kBlock, 0, stream>>>(P, w));
    GC_LAUNCH("dgc_stage", stream, dgc_stage_kernel<kMode, CPW><<<cand_grid, kBlock, 0, stream>>>(P, src, w, 1));
    GC_LAUNCH("dgc_select", stream, dgc_select_kernel<2><<<segs, kBlock, 0, stream>>>(P, w, 0u));
    GC_LAUNCH("dgc_refine", stream, dgc_refine_kernel<CPW><<<cand_grid, kBlock, 0, stream>>>(P, w));
    GC_LAUNCH("dgc_select", stream, dgc_select_kernel<3><<<segs, kBlock, 0, stream>>>(P, w, 0u));
    if (sampled || w.kden) GC_LAUNCH("dgc_sbase", stream, dgc_sbase_kernel<<<1, kBlock, 0, stream>>>(P, w, nullptr));
    GC_LAUNCH("dgc_count", stream, dgc_count_kernel<CPW><<<cand_grid, kBlock, 0, stream>>>(P, w));
    GC_LAUNCH("dgc_scan", stream, dgc_scan_kernel<<<segs, kBlock, 0, stream>>>(P, w, out->seg_off));
    GC_LAUNCH("dgc_emit", stream, dgc_emit_kernel<kMode, CPW><<<cand_grid, kBlock, 0, stream>>>(P, src, w, out->idx, out->val));
}

// Exact DGC selection in four launches after the clip norm.
template <int kMode>
void launch_exact(const gc_plan *plan, const PlanDev &P, const DgcWs &w, const Src &src, bool clip, float thr,
                  gc_sparse *out, hipStream_t stream) {
    const unsigned segs = static_cast<unsigned>(plan->nseg);
    if (clip)
        GC_LAUNCH("dgc_norm", stream, dgc_norm_kernel<<<plan->ndchunk, kBlock, 0, stream>>>(P, src.G, w));
    GC_LAUNCH("dgc_prepare", stream, dgc_prepare_kernel<kMode><<<segs, kSelBlock, 0, stream>>>(P, src, w, clip ? 1 : 0, thr));
    if (w.kden) GC_LAUNCH("dgc_sbase", stream, dgc_sbase_kernel<<<1, kBlock, 0, stream>>>(P, w, nullptr));
    GC_LAUNCH("dgc_update", stream, dgc_update_kernel<kMode, true><<<plan->ndchunk, kBlock, 0, stream>>>(P, src, w));
    GC_LAUNCH("dgc_collect", stream, dgc_xcollect_kernel<<<static_cast<unsigned>(plan->xblock.size()), kBlock, 0, stream>>>(P, w));
    GC_LAUNCH("dgc_select", stream, dgc_xselect_kernel<kMode, false><<<segs, kSelBlock, 0, stream>>>(P, src, w, out->seg_off, 0u));
    if (plan->ndchunk >= kWideChunks)
        GC_LAUNCH("dgc_emit", stream, dgc_xemit_kernel<kMode, kCpwWide, false><<<grid_1d(plan->ndchunk, kWaves * kCpwWide), kBlock, 0, stream>>>(P, src, w, out->idx, out->val));
    else
        GC_LAUNCH("dgc_emit", stream, dgc_xemit_kernel<kMode, 1, false><<<grid_1d(plan->ndchunk, kWaves), kBlock, 0, stream>>>(P, src, w, out->idx, out->val));
}

// The selection pipeline for one key source: (clip), prep, sample + bound
// (exact) or ssample + squant (sampled), update, radix select, ordered emit.
// Sampled DGC selection on plans of the exact path's densities goes on from
// the estimate with the exact path's kernels instead: the update stages the
// keys at or above it, collect and select settle each segment (all of them
// sent, or the exact top-k among them), sbase lays the segments out, emit.
template <int kMode>
void launch_select(const gc_plan *plan, const PlanDev &P, const DgcWs &w, const Src &src, bool clip, float thr,
                   bool sampled, uint32_t period, uint32_t over, gc_sparse *out, hipStream_t stream) {
    const unsigned segs = static_cast<unsigned>(plan->nseg);
    const unsigned wave_grid = grid_1d(plan->ndchunk, kWaves);
    if (clip)
        GC_LAUNCH("dgc_norm", stream, dgc_norm_kernel<<<plan->ndchunk, kBlock, 0, stream>>>(P, src.G, w));
    // sampled selection: one workgroup per segment finds the sample quantile
    // unless a segment has more samples than kQuantOneBlock
    bool multi_q = false;
    if (sampled)
        for (const SegDev &d : plan->seg) multi_q = multi_q || sample_count(d.len, period) > kQuantOneBlock;
    const bool fine = sampled && plan->dgc_fast;
    GC_LAUNCH("dgc_prep", stream, dgc_prep_kernel<<<segs, kBlock, 0, stream>>>(P, w, clip ? 1 : 0, thr, multi_q ? 1 : 0,
                                                                               fine ? 1 : 0));
    if constexpr (kMode == kVanilla || kMode == kNesterov) {
        if (sampled) {
            GC_LAUNCH("dgc_ssample", stream, dgc_ssample_kernel<kMode><<<wave_grid, kBlock, 0, stream>>>(P, src, period, w));
            if (multi_q) {
                const unsigned qgrid = segs * kQBlocks;
                GC_LAUNCH("dgc_squant", stream, dgc_qhist_kernel<0><<<qgrid, kBlock, 0, stream>>>(P, period, w));
                GC_LAUNCH("dgc_squant", stream, dgc_qfind_kernel<0><<<segs, kBlock, 0, stream>>>(P, period, w));
                GC_LAUNCH("dgc_squant", stream, dgc_qhist_kernel<1><<<qgrid, kBlock, 0, stream>>>(P, period, w));
                GC_LAUNCH("dgc_squant", stream, dgc_qfind_kernel<1><<<segs, kBlock, 0, stream>>>(P, period, w));
                GC_LAUNCH("dgc_squant", stream, dgc_qhist_kernel<2><<<qgrid, kBlock, 0, stream>>>(P, period, w));
                GC_LAUNCH("dgc_squant", stream, dgc_qfind_kernel<2><<<segs, kBlock, 0, stream>>>(P, period, w));
            } else {
                GC_LAUNCH("dgc_squant", stream, dgc_squant_kernel<<<segs, kBlock, 0, stream>>>(P, period, w));
            }
        }
        if (fine) {
            GC_LAUNCH("dgc_update", stream, dgc_update_kernel<kMode, true><<<plan->ndchunk, kBlock, 0, stream>>>(P, src, w));
            GC_LAUNCH("dgc_collect", stream, dgc_xcollect_kernel<<<static_cast<unsigned>(plan->xblock.size()), kBlock, 0, stream>>>(P, w));
            GC_LAUNCH("dgc_select", stream, dgc_xselect_kernel<kMode, true><<<segs, kSelBlock, 0, stream>>>(P, src, w, out->seg_off, over));
            GC_LAUNCH("dgc_sbase", stream, dgc_sbase_kernel<<<1, kBlock, 0, stream>>>(P, w, out->seg_off));
            if (plan->ndchunk >= kWideChunks)
                GC_LAUNCH("dgc_emit", stream, dgc_xemit_kernel<kMode, kCpwWide, true><<<grid_1d(plan->ndchunk, kWaves * kCpwWide), kBlock, 0, stream>>>(P, src, w, out->idx, out->val));
            else
                GC_LAUNCH("dgc_emit", stream, dgc_xemit_kernel<kMode, 1, true><<<grid_1d(plan->ndchunk, kWaves), kBlock, 0, stream>>>(P, src, w, out->idx, out->val));
            return;
        }
    }
    if (!sampled) {
        GC_LAUNCH("dgc_sample", stream, dgc_sample_kernel<kMode><<<grid_1d(plan->ndchunk, 2 * kWaves), kBlock, 0, stream>>>(P, src, w));
        GC_LAUNCH("dgc_bound", stream, dgc_bound_kernel<<<segs, kBlock, 0, stream>>>(P, w));
    }
    // One workgroup per chunk: with non-temporal streaming this measured 15%
    // faster than an occupancy-sized persistent grid walking chunk ranges
    // (the explorer, bound by its Philox keys, runs the same in either shape).
    GC_LAUNCH("dgc_update", stream, dgc_update_kernel<kMode><<<plan->ndchunk, kBlock, 0, stream>>>(P, src, w));
    if (plan->ndchunk >= kWideChunks)
        launch_candidates<kMode, kCpwWide>(plan, P, w, src, sampled, over, out, stream);
    else
        launch_candidates<kMode, 1>(plan, P, w, src, sampled, over, out, stream);
}
}  // namespace

extern "C" uint64_t gc_dgc_message_cap(const gc_plan *plan, const gc_dgc_options *opt) {
    if (!plan) return 0;
    if (!opt) return plan->total_k;
    if (opt->select == GC_SELECT_SAMPLED) return dgc_capacity(plan, GC_SELECT_SAMPLED, opt->over);
    return dgc_capacity(plan, GC_SELECT_EXACT, 0, opt->density_num, opt->density_den);
}

extern "C" gc_status gc_dgc_step_ex(const gc_plan *plan, const float *G, float *U, float *V,
                                    const gc_dgc_options *opt, gc_sparse *out, void *ws,
                                    size_t ws_bytes, hipStream_t stream) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_dgc_step: plan is null");
    if (!opt) return set_error(GC_EINVAL, "gc_dgc_step: options are null");
    if (!G || !U || !V) return set_error(GC_EINVAL, "gc_dgc_step: G, U and V must be non-null");
    const float momentum = opt->momentum, thr_G = opt->thr_G;
    const int num_nodes = opt->num_nodes;
    if (!(momentum >= 0.0f && momentum < 1.0f))
        return set_error(GC_EINVAL, "gc_dgc_step: momentum must be in [0, 1)");
    if (std::isnan(thr_G) || std::isinf(thr_G))
        return set_error(GC_EINVAL, "gc_dgc_step: thr_G must be finite");
    if (num_nodes < 1) return set_error(GC_EINVAL, "gc_dgc_step: num_nodes must be >= 1");
    if (opt->momentum_kind != GC_MOMENTUM_VANILLA && opt->momentum_kind != GC_MOMENTUM_NESTEROV)
        return set_error(GC_EINVAL, "gc_dgc_step: momentum_kind must be GC_MOMENTUM_VANILLA or GC_MOMENTUM_NESTEROV");
    if (opt->select != GC_SELECT_EXACT && opt->select != GC_SELECT_SAMPLED)
        return set_error(GC_EINVAL, "gc_dgc_step: select must be GC_SELECT_EXACT or GC_SELECT_SAMPLED");
    const bool sampled = opt->select == GC_SELECT_SAMPLED;
    if (sampled && (opt->sample_period < 1 || opt->sample_period > GC_MAX_SAMPLE_PERIOD))
        return set_error(GC_EINVAL, "gc_dgc_step: sample_period must be in [1, GC_MAX_SAMPLE_PERIOD]");
    if (sampled && opt->over < 1) return set_error(GC_EINVAL, "gc_dgc_step: over must be >= 1");
    if (opt->reserved != 0) return set_error(GC_EINVAL, "gc_dgc_step: reserved must be 0");
    const uint32_t knum = opt->density_num, kden = opt->density_den;
    if (kden != 0 && (knum < 1 || knum > kden))
        return set_error(GC_EINVAL, "gc_dgc_step: density_num must be in [1, density_den] when density_den > 0");
    if (kden != 0 && sampled)
        return set_error(GC_ENOTSUP, "gc_dgc_step: a per-call density needs GC_SELECT_EXACT");
    gc_status st = check_select_io("gc_dgc_step", plan, out, dgc_capacity(plan, opt->select, opt->over, knum, kden),
                                   ws, ws_bytes);
    if (st != GC_OK) return st;
    PlanDev P;
    st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    DgcWs w = dgc_layout(plan, ws, nullptr);
    w.knum = knum;
    w.kden = kden;
    const bool clip = thr_G > 0.0f;
    const float thr = clip ? static_cast<float>(static_cast<double>(thr_G) /
                                                std::sqrt(static_cast<double>(num_nodes)))
                           : 0.0f;
    Src src{G, U, V, momentum, 0u, 0u, 0u, 0u, nullptr};
    const bool nesterov = opt->momentum_kind == GC_MOMENTUM_NESTEROV;
    const bool fast = !sampled && (kden == 0 ? plan->dgc_fast : dgc_exact_fast(plan, knum, kden));
    if (fast && nesterov)
        launch_exact<kNesterov>(plan, P, w, src, clip, thr, out, stream);
    else if (fast)
        launch_exact<kVanilla>(plan, P, w, src, clip, thr, out, stream);
    else if (nesterov)
        launch_select<kNesterov>(plan, P, w, src, clip, thr, sampled, opt->sample_period, opt->over, out, stream);
    else
        launch_select<kVanilla>(plan, P, w, src, clip, thr, sampled, opt->sample_period, opt->over, out, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_dgc_step launch");
    return GC_OK;
}

extern "C" gc_status gc_dgc_step(const gc_plan *plan, const float *G, float *U, float *V,
                                 float momentum, float thr_G, int num_nodes, gc_sparse *out,
                                 void *ws, size_t ws_bytes, hipStream_t stream) {
    gc_dgc_options o{};
    o.momentum = momentum;
    o.thr_G = thr_G;
    o.num_nodes = num_nodes;
    o.momentum_kind = GC_MOMENTUM_VANILLA;
    o.select = GC_SELECT_EXACT;
    return gc_dgc_step_ex(plan, G, U, V, &o, out, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ Slim-DP
extern "C" uint64_t gc_slimdp_mask_words(const gc_plan *plan) { return plan ? plan->mask_words : 0; }

extern "C" gc_status gc_slimdp_core(const gc_plan *plan, const float *w_param, const float *g, float c,
                                    gc_sparse *core, uint32_t *core_mask, void *ws, size_t ws_bytes,
                                    hipStream_t stream) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_slimdp_core: plan is null");
    if (!w_param || !g || !core_mask) return set_error(GC_EINVAL, "gc_slimdp_core: w, g and core_mask must be non-null");
    if (!(c > 0.0f) || std::isinf(c)) return set_error(GC_EINVAL, "gc_slimdp_core: c must be positive and finite");
    gc_status st = check_select_io("gc_slimdp_core", plan, core, plan->total_k, ws, ws_bytes);
    if (st != GC_OK) return st;
    PlanDev P;
    st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    DgcWs w = dgc_layout(plan, ws, nullptr);
    Src src{g, const_cast<float *>(w_param), nullptr, c, 0u, 0u, 0u, 0u, core_mask};
    launch_select<kSignif>(plan, P, w, src, false, 0.0f, false, 0u, 0u, core, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_slimdp_core launch");
    return GC_OK;
}

extern "C" gc_status gc_slimdp_explore(const gc_plan *plan, const gc_plan *core_plan, const float *delta,
                                       const uint32_t *core_mask, uint64_t seed, uint64_t step, gc_sparse *out,
                                       void *ws, size_t ws_bytes, hipStream_t stream) {
    clear_error();
    if (!plan || !core_plan) return set_error(GC_EINVAL, "gc_slimdp_explore: plans must be non-null");
    if (!delta || !core_mask) return set_error(GC_EINVAL, "gc_slimdp_explore: delta and core_mask must be non-null");
    if (core_plan->nseg != plan->nseg || core_plan->n_total != plan->n_total)
        return set_error(GC_EINVAL, "gc_slimdp_explore: plans must describe the same segments");
    for (int s = 0; s < plan->nseg; ++s) {
        const SegDev &a = plan->seg[s], &b = core_plan->seg[s];
        if (a.off != b.off || a.len != b.len)
            return set_error(GC_EINVAL, "gc_slimdp_explore: plans must describe the same segments");
        if (uint64_t(a.k) + b.k > a.len)
            return set_error(GC_EINVAL, "gc_slimdp_explore: core plus explorer exceeds a segment");
    }
    gc_status st = check_select_io("gc_slimdp_explore", plan, out, plan->total_k, ws, ws_bytes);
    if (st != GC_OK) return st;
    PlanDev P;
    st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    DgcWs w = dgc_layout(plan, ws, nullptr);
    Src src{delta, nullptr, nullptr, 0.0f, static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32),
            static_cast<uint32_t>(step), static_cast<uint32_t>(step >> 32), const_cast<uint32_t *>(core_mask)};
    launch_select<kExplore>(plan, P, w, src, false, 0.0f, false, 0u, 0u, out, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_slimdp_explore launch");
    return GC_OK;
}

namespace {
// Indices at or past n are clamped, so a malformed message stays in bounds.
__global__ __launch_bounds__(kBlock) void gather_kernel(const uint32_t *__restrict__ idx, uint32_t count,
                                                        const float *__restrict__ src, uint32_t n,
                                                        float *__restrict__ dst) {
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    if (i < count) dst[i] = src[min(idx[i], n - 1)];
}
}  // namespace

extern "C" gc_status gc_slimdp_core_values(const gc_plan *core_plan, const gc_sparse *core, const float *delta,
                                           float *values, hipStream_t stream) {
    clear_error();
    if (!core_plan || !core || !core->idx || !delta || !values)
        return set_error(GC_EINVAL, "gc_slimdp_core_values: arguments must be non-null");
    if (core->cap < core_plan->total_k)
        return set_error(GC_ECAPACITY, "gc_slimdp_core_values: core message smaller than the plan's total k");
    const uint64_t K = core_plan->total_k;
    GC_LAUNCH("slimdp_values", stream, gather_kernel<<<grid_1d(K, kBlock), kBlock, 0, stream>>>(
        core->idx, static_cast<uint32_t>(K), delta, static_cast<uint32_t>(core_plan->n_total), values));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_slimdp_core_values launch");
    return GC_OK;
}
