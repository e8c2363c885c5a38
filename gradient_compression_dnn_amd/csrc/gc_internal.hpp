// Internal definitions shared by the libgradcomp translation units:
// plan tables, workspace layouts, error state and block-level device
// primitives for gfx950 (wave64, 256-thread workgroups).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <string>
#include <vector>

#include "gradcomp.h"

namespace gc {

// ------------------------------------------------------------ launch shape
constexpr int kBlock = 256;            // threads per workgroup (4 waves)
constexpr int kWave = 64;
constexpr int kWaves = kBlock / kWave;
constexpr int kEPT = 16;               // elements per thread in dense passes
constexpr int kChunk = kBlock * kEPT;  // 4096 elements per workgroup tile
constexpr int kChunkLog2 = 12;

// Radix-select digits over the 31-bit magnitude key: 11 + 11 + 9 bits.
constexpr int kDigit1Bits = 11, kDigit2Bits = 11, kDigit3Bits = 9;
constexpr int kHist1 = 1 << kDigit1Bits;
constexpr int kHist2 = 1 << kDigit2Bits;
constexpr int kHist3 = 1 << kDigit3Bits;

// ------------------------------------------------------------ plan tables
// One segment as the kernels see it.  DGC chunks are aligned kChunk-element
// tiles from the segment start (so pairwise-tree nodes line up with them);
// AdaComp chunks hold a whole number of bins.
struct SegDev {
    uint64_t off;        // first element in the flat buffer
    uint32_t len;        // n_s
    uint32_t bin_len;    // L_T
    uint32_t k;          // top-k count
    uint32_t nbins;      // ceil(len / bin_len)
    uint32_t dchunk0;    // first DGC chunk
    uint32_t dnchunk;    // DGC chunks in this segment
    uint32_t achunk0;    // first AdaComp chunk
    uint32_t anchunk;    // AdaComp chunks in this segment
    uint32_t achunk_len; // elements per AdaComp chunk (multiple of bin_len)
    uint32_t bin0;       // first bin of the segment in the plan-wide bin array
    uint32_t kbase;      // first message slot of the segment in a DGC message
    uint32_t bgroup0;    // first 4096-bin group of the segment (AdaComp scale sum)
    uint32_t nbgroup;    // 4096-bin groups in the segment
    uint32_t mbase;      // first word of the segment's run in a selection bitmap
};

// Exact DGC: the collect kernel's workgroups each take up to kXBlockChunks
// chunks of one segment.
constexpr uint32_t kXBlockChunks = 32;

constexpr int kBinGroupLog2 = 12;  // bins per group of the scale's pairwise tree
constexpr uint32_t kBinGroup = 1u << kBinGroupLog2;

// One chunk of a segment, fetched with a single 16-byte load:
//   x = first flat element, y = elements, z = segment, w = aux (AdaComp:
//   first bin of the chunk in the plan-wide bin array; DGC: chunk number
//   inside the segment).
using ChunkRec = uint4;

struct PlanDev {
    const SegDev *seg;          // [nseg]
    const ChunkRec *dchunk_rec; // [ndchunk]
    const ChunkRec *achunk_rec; // [nachunk]
    const uint32_t *dchunk_seg; // [ndchunk]
    const uint32_t *achunk_seg; // [nachunk]
    const uint64_t *seg_start;  // [nseg] offsets, for searching an index
    const uint32_t *bgroup_seg; // [nbgroup] segment of each bin group
    const uint2 *xblock;        // [nxblock] exact DGC collect blocks: segment, first DGC chunk
    int nseg;
    uint32_t ndchunk;
    uint32_t nachunk;
    uint32_t nbgroup;
    uint32_t nxblock;
    uint64_t n_total;
};

}  // namespace gc

struct gc_plan {
    int nseg = 0;
    uint64_t n_total = 0;
    uint64_t total_k = 0;
    uint64_t total_bins = 0;
    uint32_t ndchunk = 0;
    uint32_t nachunk = 0;
    uint32_t nbgroup = 0;
    uint64_t mask_words = 0;  // sum over segments of ceil(length / 32)
    uint64_t seg_elems = 0;   // sum over segments of the length
    bool dgc_fast = false;    // exact DGC at the plan's k takes the four-launch path
    std::vector<gc::SegDev> seg;
    std::vector<uint32_t> dchunk_seg;
    std::vector<uint32_t> achunk_seg;
    std::vector<uint64_t> seg_start;
    std::vector<uint32_t> bgroup_seg;
    std::vector<uint2> xblock;  // exact DGC collect blocks (kXBlockChunks chunks of one segment at most)
    std::vector<gc::ChunkRec> dchunk_rec;
    std::vector<gc::ChunkRec> achunk_rec;
    // device copies, one per device, uploaded on first use
    std::mutex mu;
    std::vector<std::pair<int, void *>> dev_blob;
};

namespace gc {

// --------------------------------------------------------------- errors
gc_status set_error(gc_status code, const std::string &msg);
gc_status hip_error(hipError_t e, const char *what);
void clear_error();

// Device tables of a plan on the current device (uploads on first use).
gc_status plan_device(const gc_plan *plan, PlanDev *out);
// The same, for tables already on the current device (gc_plan_upload);
// GC_EINVAL otherwise, without allocating.
gc_status plan_device_resident(const gc_plan *plan, PlanDev *out);

// Workgroups of kBlock threads of `kernel` that the current device holds at
// once (its occupancy times the compute units), cached per device and kernel.
unsigned resident_blocks(const void *kernel);

// Whether exact DGC selection at these densities takes the four-launch path
// (knum = kden = 0: the plan's own k).
bool dgc_exact_fast(const gc_plan *plan, uint32_t knum, uint32_t kden);

// Workspace bytes per operation (each op's translation unit lays out its own).
size_t dgc_workspace_bytes(const gc_plan *plan);
size_t adacomp_workspace_bytes(const gc_plan *plan);
size_t pack_workspace_bytes(const gc_plan *plan);
size_t decode_workspace_bytes(const gc_plan *plan);
size_t unpack_workspace_bytes(const gc_plan *plan);

// --------------------------------------------------------------- workspace
// Bump allocator over the caller's workspace; every region 256-byte aligned.
struct WsCursor {
    uintptr_t base;
    size_t used = 0;
    explicit WsCursor(void *p) : base(reinterpret_cast<uintptr_t>(p)) {}
    template <class T>
    T *take(size_t count) {
        used = (used + 255) & ~size_t(255);
        T *p = reinterpret_cast<T *>(base + used);
        used += sizeof(T) * count;
        return p;
    }
};

// Minimum of two u64 by comparison (the device min<uint64_t> overload goes
// through double).
__host__ __device__ constexpr uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// ceil(a / b) in 64 bits (lengths near 2^32 overflow u32 round-ups).
__host__ __device__ constexpr uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

inline unsigned grid_1d(uint64_t n, unsigned per_block) {
    return static_cast<unsigned>((n + per_block - 1) / per_block);
}

// Kernel timing (see gc_timing_enable): returns an event to record before
// the launch (or nullptr when the kernel is not selected) and records the
// closing event after it.
hipEvent_t timing_begin(const char *kernel, hipStream_t s);
void timing_end(const char *kernel, hipEvent_t start, hipStream_t s);

struct TimedLaunch {
    const char *name;
    hipStream_t stream;
    hipEvent_t start;
    TimedLaunch(const char *n, hipStream_t s) : name(n), stream(s), start(timing_begin(n, s)) {}
    ~TimedLaunch() {
        if (start) timing_end(name, start, stream);
    }
};
#define GC_LAUNCH(name, stream, ...)                  \
    do {                                              \
        ::gc::TimedLaunch gc_timed_launch_(name, stream); \
        __VA_ARGS__;                                  \
    } while (0)

inline uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }

// ===================================================================== device
#if defined(__HIPCC__)

__device__ __forceinline__ uint32_t dev_f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float dev_u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Number of set bits of a wave mask below this lane.
__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}

// Wave-wide integer scans and reductions by DPP moves (CDNA data-parallel
// primitives): row_shr 1, 2, 4 and 8 inside each 16-lane row, then
// row_bcast 15 and row_bcast 31 carry the row totals into the rows above.  A
// lane whose source lies outside its row, or a row the broadcast skips,
// reads 0, the identity of + and of an unsigned max.  Every lane of the wave
// must be active.  (A wave scan by ds_bpermute shuffles measured about 8x
// slower: six dependent LDS round trips.)
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
constexpr int kDppWaveShr1 = 0x138;  // lane l reads lane l - 1 across the whole wave
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), kCtrl, kRowMask, 0xF, false));
}
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    x += dpp_u32<kDppRowShr1>(x);
    x += dpp_u32<kDppRowShr2>(x);
    x += dpp_u32<kDppRowShr4>(x);
    x += dpp_u32<kDppRowShr8>(x);
    x += dpp_u32<kDppRowBcast15, 0xA>(x);
    x += dpp_u32<kDppRowBcast31, 0xC>(x);
    return x;
}
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ void dpp_add_u64(uint32_t &lo, uint32_t &hi) {
    const uint32_t l = dpp_u32<kCtrl, kRowMask>(lo), h = dpp_u32<kCtrl, kRowMask>(hi);
    const uint32_t n = lo + l;
    hi = hi + h + (n < lo ? 1u : 0u);
    lo = n;
}
__device__ __forceinline__ uint64_t wave_inclusive_scan(uint64_t x) {
    uint32_t lo = static_cast<uint32_t>(x), hi = static_cast<uint32_t>(x >> 32);
    dpp_add_u64<kDppRowShr1>(lo, hi);
    dpp_add_u64<kDppRowShr2>(lo, hi);
    dpp_add_u64<kDppRowShr4>(lo, hi);
    dpp_add_u64<kDppRowShr8>(lo, hi);
    dpp_add_u64<kDppRowBcast15, 0xA>(lo, hi);
    dpp_add_u64<kDppRowBcast31, 0xC>(lo, hi);
    return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint32_t wave_inclusive_max(uint32_t x) {
    x = max(x, dpp_u32<kDppRowShr1>(x));
    x = max(x, dpp_u32<kDppRowShr2>(x));
    x = max(x, dpp_u32<kDppRowShr4>(x));
    x = max(x, dpp_u32<kDppRowShr8>(x));
    x = max(x, dpp_u32<kDppRowBcast15, 0xA>(x));
    x = max(x, dpp_u32<kDppRowBcast31, 0xC>(x));
    return x;
}
// The wave's sum and maximum, in every lane.
__device__ __forceinline__ uint32_t wave_total(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_inclusive_scan(x)), kWave - 1));
}
__device__ __forceinline__ uint32_t wave_max_all(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_inclusive_max(x)), kWave - 1));
}

// Exclusive scan of one value per thread, in thread order, over a workgroup
// of BS threads (T: uint32_t or uint64_t).  Returns the exclusive prefix;
// *total receives the sum.
template <class T, int BS = kBlock>
__device__ __forceinline__ T block_exclusive_scan(T v, T *total) {
    constexpr int NW = BS / kWave;
    __shared__ T wsum[NW];
    const T x = wave_inclusive_scan(v);
    if (lane_id() == kWave - 1) wsum[wave_id()] = x;
    __syncthreads();
    T before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        T s = wsum[w];
        if (w < wave_id()) before += s;
        all += s;
    }
    __syncthreads();
    *total = all;
    return before + x - v;
}

// Ordered compaction of kEPT flags per thread, where element (j, t) has rank
// j * kBlock + t in index order.  pos[j] receives the output slot of flagged
// elements; returns the number of flagged elements in the block.
template <int EPT>
__device__ __forceinline__ uint32_t block_compact(const bool (&flag)[EPT], uint32_t (&pos)[EPT]) {
    __shared__ uint32_t cnt[EPT * kWaves];
    __shared__ uint32_t tot;
    uint32_t rank[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
        uint64_t m = __ballot(flag[j]);
        rank[j] = lane_rank(m);
        if (lane_id() == 0) cnt[j * kWaves + wave_id()] = static_cast<uint32_t>(__popcll(m));
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        // one wave scans the EPT*kWaves (<= 64) counters in (j, wave) order
        uint32_t v = threadIdx.x < EPT * kWaves ? cnt[threadIdx.x] : 0u;
        const uint32_t x = wave_inclusive_scan(v);
        if (threadIdx.x < EPT * kWaves) cnt[threadIdx.x] = x - v;
        if (threadIdx.x == kWave - 1) tot = x;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EPT; ++j) pos[j] = cnt[j * kWaves + wave_id()] + rank[j];
    uint32_t t = tot;
    __syncthreads();
    return t;
}

// ------------------------------------------------------ 4-wide lane layout
// Dense chunk kernels give every lane 4 consecutive elements per row:
// element e = row * 1024 + 4 * threadIdx.x + u (u = 0..3), rows 0..3, so a
// 4096-element chunk is 4 rows.  When the chunk starts on a 16-byte boundary
// the four elements move as one float4; otherwise (or at a ragged tail) each
// element is accessed on its own.
constexpr int kRows = kChunk / (4 * kBlock);

__device__ __forceinline__ uint32_t row_elem(int row) { return row * (4 * kBlock) + 4u * threadIdx.x; }

// Chunk access through a raw buffer resource that covers exactly the chunk,
// [p, p + cnt): the hardware checks each dword against that range, so loads
// past cnt return 0 and stores past it are dropped.  Every lane then issues
// one 16-byte access with no branch (divergent load paths into the same
// registers would force waits that serialize a prefetch), p needs only dword
// alignment, and the base lives in scalar registers.  The resource must be
// wave-uniform: p and cnt depend on the chunk only.
//
// The accesses carry the non-temporal hint: every dense array here is
// streamed once per call and not reused within it, and letting it allocate
// in L2 and the Infinity Cache only evicts other data and defers write-backs
// into later kernels (measured: the step ran 13% faster with the hint).
using BufRsrc = __amdgpu_buffer_rsrc_t;
constexpr int kBufWord3 = 0x00020000;  // raw 32-bit data format, gfx9 resource word 3
constexpr int kBufNT = 2;              // cache policy operand: non-temporal
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ BufRsrc chunk_buf(const float *p, uint32_t cnt) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(p), static_cast<short>(0),
                                             static_cast<int>(cnt * 4u), kBufWord3);
}

// Elements [e0, e0 + 4) of the chunk; 0 past its end.
__device__ __forceinline__ void load4(BufRsrc r, uint32_t e0, float (&v)[4]) {
    const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(e0 * 4u), 0, kBufNT);
    v[0] = dev_u2f(t.x);
    v[1] = dev_u2f(t.y);
    v[2] = dev_u2f(t.z);
    v[3] = dev_u2f(t.w);
}

// Writes elements [e0, e0 + 4) of the chunk; those past its end are dropped.
__device__ __forceinline__ void store4(BufRsrc r, uint32_t e0, const float (&v)[4]) {
    const u32x4 t = {dev_f2u(v[0]), dev_f2u(v[1]), dev_f2u(v[2]), dev_f2u(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(t, r, static_cast<int>(e0 * 4u), 0, kBufNT);
}

// Ordered compaction in the 4-wide layout: element (row, u) of thread t has
// rank row * 1024 + 4 t + u.  pos receives the output slot of flagged
// elements; returns the block's flagged count.
__device__ __forceinline__ uint32_t block_compact4(const bool (&flag)[kRows][4],
                                                   uint32_t (&pos)[kRows][4]) {
    __shared__ uint32_t cnt[kRows * kWaves];
    __shared__ uint32_t tot;
    uint32_t rank[kRows][4];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        uint32_t before = 0, total = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint64_t m = __ballot(flag[j][u]);
            before += lane_rank(m);
            total += static_cast<uint32_t>(__popcll(m));
        }
        uint32_t within = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            rank[j][u] = before + within;
            within += flag[j][u] ? 1u : 0u;
        }
        if (lane_id() == 0) cnt[j * kWaves + wave_id()] = total;
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        uint32_t v = threadIdx.x < kRows * kWaves ? cnt[threadIdx.x] : 0u;
        const uint32_t x = wave_inclusive_scan(v);
        if (threadIdx.x < kRows * kWaves) cnt[threadIdx.x] = x - v;
        if (threadIdx.x == kWave - 1) tot = x;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) pos[j][u] = cnt[j * kWaves + wave_id()] + rank[j][u];
    uint32_t t = tot;
    __syncthreads();
    return t;
}

// Full 64-bit product of two u32 in one VALU op (v_mad_u64_u32 with a zero
// addend); on gfx950 this is faster than the separate low and high multiplies.
__device__ __forceinline__ uint64_t mul_wide(uint32_t a, uint32_t b) {
    uint64_t r, carry;
    asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(r), "=s"(carry) : "v"(a), "v"(b));
    return r;
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): ten rounds of two 32x32 -> 64-bit products, the
// key advanced by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kM0 = 0xD2511F53u, kM1 = 0xCD9E8D57u;
    constexpr uint32_t kW0 = 0x9E3779B9u, kW1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = mul_wide(kM0, c.x);
        const uint64_t p1 = mul_wide(kM1, c.z);
        c = make_uint4(uint32_t(p1 >> 32) ^ c.y ^ k0, uint32_t(p1), uint32_t(p0 >> 32) ^ c.w ^ k1,
                       uint32_t(p0));
        k0 += kW0;
        k1 += kW1;
    }
    return c;
}

// Perfect binary tree sum of one double per thread of a BS-thread
// workgroup, leaves in thread order.  Butterfly adds are bit-identical on
// both lanes because IEEE addition is commutative, so every lane ends with
// the wave's subtree sum; the wave sums are then added as a perfect tree.
template <int BS = kBlock>
__device__ __forceinline__ double block_tree_sum(double v) {
    constexpr int NW = BS / kWave;
    static_assert((NW & (NW - 1)) == 0, "power-of-two wave count");
    __shared__ double ws[NW];
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) v = v + __shfl_xor(v, d, kWave);
    if (lane_id() == 0) ws[wave_id()] = v;
    __syncthreads();
    double t[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) t[w] = ws[w];
#pragma unroll
    for (int half = NW / 2; half >= 1; half >>= 1)
#pragma unroll
        for (int w = 0; w < half; ++w) t[w] = t[2 * w] + t[2 * w + 1];
    __syncthreads();
    return t[0];
}

// Canonical pairwise sum of x[0..m) (zero-padded to a power of two) by one
// workgroup of BS threads.  load(i) returns term i as double for i < m.
// Thread t owns an aligned sub-block of B = max(1, M/BS) leaves.  Below 8 leaves it adds
// them as their perfect tree; otherwise it adds each run of 8 as a fixed
// 8-leaf tree and combines those nodes in order with the binary-counter stack
// (which forms exactly the perfect subtree over them).  The BS subtree sums
// are combined by block_tree_sum.  Sub-blocks past m are +0.0 subtrees, and
// adding +0.0 to a non-negative value is exact, so the result equals the tree
// over M leaves.  (A stack step per leaf cost 26 predicated adds each; per
// 8-leaf node the 5,063-chunk clip tree finishes in a fraction of that.)
constexpr int kTreeDepth = 23;  // levels of 8-leaf nodes: sub-blocks of up to 2^26 leaves per thread

template <int BS = kBlock, class Load>
__device__ double block_pairwise_sum(uint64_t m, Load load) {
    uint64_t M = 1;
    while (M < m) M <<= 1;
    const uint64_t B = M > uint64_t(BS) ? M / BS : 1;
    const uint64_t lo = static_cast<uint64_t>(threadIdx.x) * B;
    // leaf g, +0.0 past the terms (the index is clamped, so the load is in
    // bounds; m >= 1)
    auto leaf = [&](uint64_t g) {
        const double v = load(g < m ? g : m - 1);
        return g < m ? v : 0.0;
    };
    double carry;
    if (B < 8) {
        double l[4];
#pragma unroll
        for (uint64_t u = 0; u < 4; ++u) l[u] = u < B ? leaf(lo + u) : 0.0;
        carry = B == 1 ? l[0] : B == 2 ? l[0] + l[1] : (l[0] + l[1]) + (l[2] + l[3]);
    } else {
        double stack[kTreeDepth];
        for (uint64_t i = 0; i < B / 8; ++i) {
            double l[8];
#pragma unroll
            for (uint64_t u = 0; u < 8; ++u) l[u] = leaf(lo + 8 * i + u);
            carry = ((l[0] + l[1]) + (l[2] + l[3])) + ((l[4] + l[5]) + (l[6] + l[7]));
            bool done = false;
#pragma unroll
            for (int lv = 0; lv < kTreeDepth; ++lv) {
                if (!done) {
                    if ((i >> lv) & 1) {
                        carry = stack[lv] + carry;
                    } else {
                        stack[lv] = carry;
                        done = true;
                    }
                }
            }
        }
    }
    // after B/8 (a power of two) nodes the full subtree sum is the last carry
    return block_tree_sum<BS>(carry);
}

// Given NB bucket counts (read through `count(b)`), and 1 <= k <= total, find
// the bucket d holding the k-th largest element: sum_{b>d} < k <= sum_{b>=d}.
// Returns d and writes sum_{b>d} to *above.  Called by the whole workgroup
// of BS threads.
template <int NB, int BS = kBlock, class Count>
__device__ uint32_t block_find_bucket(uint32_t k, Count count, uint32_t *above) {
    constexpr int per = NB >= BS ? NB / BS : 1;
    static_assert(NB >= BS ? NB % BS == 0 : true, "bucket count");
    __shared__ uint32_t res_d, res_above;
    if (threadIdx.x == 0) {
        res_d = 0;
        res_above = 0;
    }
    uint32_t c[per];
    uint32_t tsum = 0;
    // thread t owns buckets NB-1-t*per down to NB-(t+1)*per (descending);
    // threads past the buckets own none
#pragma unroll
    for (int i = 0; i < per; ++i) {
        const int b = NB - 1 - int(threadIdx.x) * per - i;
        c[i] = b >= 0 ? count(b) : 0u;
        tsum += c[i];
    }
    uint32_t total;
    uint32_t pre = block_exclusive_scan<uint32_t, BS>(tsum, &total);
    if (pre < k && pre + tsum >= k) {
        uint32_t cum = pre;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (cum + c[i] >= k) {
                res_d = NB - 1 - threadIdx.x * per - i;
                res_above = cum;
                break;
            }
            cum += c[i];
        }
    }
    __syncthreads();
    *above = res_above;
    uint32_t d = res_d;
    __syncthreads();
    return d;
}

#endif  // __HIPCC__

}  // namespace gc
