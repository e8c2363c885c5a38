// The receiving side of the packed exchange: a run-length stream read back
// into a message.  "Deep Gradient Compression" (Lin et al.) §3.1: 32-bit
// values with 16-bit zero-run lengths (AdaComp codes carry a sign bit and one
// layer scale instead).
//
// The stream's block table gives every block's offset, codes and entries, and
// each block carries a checkpoint (entries read, reader position) before
// every 4096th code, so the blocks and their tiles of 4096 codes are read
// independently:
//   layout (one workgroup) check the stream header, the table and every
//          block header against the plan and against one another; segment
//          offsets of the message, tiles, scales
//   write  (tile) codes from the tile's checkpoint: block scans of steps and
//          entries give every entry's position and slot; the tile's end must
//          meet the next checkpoint (or the block's entry count); idx, val
// Anything that does not fit the plan sets a bit in *status and is not
// written; the message stays within its capacity and its segments.  A stream
// whose layout is wrong anywhere is read as empty.
#include <algorithm>

#include "gc_internal.hpp"

namespace gc {

namespace {

constexpr uint32_t kUTile = 4096;            // codes per tile, and between checkpoints
constexpr uint32_t kUPer = kUTile / kBlock;  // codes per thread in a tile

// status bits
constexpr uint32_t kBadStream = 1u, kBadBlock = 2u, kBadEntry = 4u, kOverCap = 8u, kBadCount = 16u;

struct UnpackWs {
    uint64_t *blk_off;     // [nseg] byte offset of each block
    uint32_t *seg_E;       // [nseg] codes of each block (0 when the stream is bad)
    uint32_t *seg_cnt;     // [nseg] entries of each block (0 when the stream is bad)
    uint32_t *tile_base;   // [nseg + 1] first tile of each block
    uint32_t *slot_base;   // [nseg + 1] first message slot of each block (before clamping to cap)
    size_t max_tiles;
};

// Codes a well-formed block of a segment of n elements holds at most.
__host__ __device__ __forceinline__ uint64_t max_codes(uint32_t n, uint32_t MAX) {
    return uint64_t(n) + n / MAX + 1;
}

UnpackWs unpack_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    UnpackWs w{};
    size_t tiles = 0;
    for (const auto &s : p->seg) tiles += (max_codes(s.len, 32767u) + kUTile - 1) / kUTile;
    w.max_tiles = tiles + 1;
    w.blk_off = c.take<uint64_t>(p->nseg);
    w.seg_E = c.take<uint32_t>(p->nseg);
    w.seg_cnt = c.take<uint32_t>(p->nseg);
    w.tile_base = c.take<uint32_t>(p->nseg + 1);
    w.slot_base = c.take<uint32_t>(p->nseg + 1);
    if (bytes) *bytes = c.used + 256;
    return w;
}

constexpr uint32_t magic(char a, char b, char c, char d) {
    return uint32_t(uint8_t(a)) | uint32_t(uint8_t(b)) << 8 | uint32_t(uint8_t(c)) << 16 |
           uint32_t(uint8_t(d)) << 24;
}

__device__ __forceinline__ uint64_t block_bytes(uint64_t E, bool dgc) {
    return 16 + 2 * E + 2 * (E & 1u) + (dgc ? 4 * E : 0) + 8 * ((E + kUTile - 1) / kUTile);
}

__device__ __forceinline__ uint64_t ld_u64(const uint8_t *p) {
    const uint32_t *q = reinterpret_cast<const uint32_t *>(p);
    return uint64_t(q[0]) | uint64_t(q[1]) << 32;
}

// Block s as the table and its header give it: table entry (offset, E, cnt)
// and whether the block fits the plan and the stream on its own (its header
// inside the stream, magic, length, codes and count agree with the table, its
// bytes inside the stream).  w3 is the header's last word.
struct BlockView {
    uint64_t off;
    uint32_t E, cnt, w3;
    bool ok;
};
__device__ __forceinline__ BlockView view_block(const PlanDev &P, bool dgc, uint32_t MAX, uint32_t bmagic,
                                                const uint8_t *in, uint64_t nbytes, int s) {
    BlockView b{};
    const uint8_t *t = in + 16 + 16 * uint64_t(s);
    b.off = ld_u64(t);
    b.E = reinterpret_cast<const uint32_t *>(t)[2];
    b.cnt = reinterpret_cast<const uint32_t *>(t)[3];
    const uint32_t len = P.seg[s].len;
    b.ok = b.off % 4 == 0 && b.off <= nbytes && nbytes - b.off >= 16 && b.E <= max_codes(len, MAX) && b.cnt <= b.E &&
           block_bytes(b.E, dgc) <= nbytes - b.off;
    if (b.ok) {
        const uint32_t *h = reinterpret_cast<const uint32_t *>(in + b.off);
        b.w3 = h[3];
        b.ok = h[0] == bmagic && h[1] == len && h[2] == b.E && (!dgc || h[3] == b.cnt);
    }
    return b;
}

// One workgroup.  Pass 1 checks every block and that each lies where the
// blocks before it end; pass 2 lays out the tiles and slots (every block
// empty when anything failed) and writes the message's segment offsets and
// scales.
__global__ __launch_bounds__(kBlock) void unpack_layout_kernel(PlanDev P, int kind, const uint8_t *__restrict__ in,
                                                               uint64_t nbytes, uint64_t cap, UnpackWs w,
                                                               uint32_t *__restrict__ seg_off, float *seg_scale,
                                                               uint32_t *status) {
    const bool dgc = kind == GC_KIND_DGC;
    const uint32_t MAX = dgc ? 65535u : 32767u;
    const uint32_t bmagic = dgc ? magic('D', 'G', 'C', '1') : magic('A', 'D', 'C', '1');
    const uint64_t head = 16 + 16 * uint64_t(P.nseg);
    uint32_t st = 0;
    {
        const uint32_t *h = reinterpret_cast<const uint32_t *>(in);
        if (nbytes < head || h[0] != magic('G', 'C', 'P', '2') || h[1] != uint32_t(kind) ||
            h[2] != uint32_t(P.nseg) || h[3] != 0u)
            st = kBadStream;
    }
    // pass 1
    uint64_t at = head;
    uint32_t bad = 0;
    if (!st) {
        for (int r = 0; r < P.nseg; r += kBlock) {
            const int s = r + int(threadIdx.x);
            uint64_t sz = 0;
            bool ok = true;
            uint64_t off = 0;
            if (s < P.nseg) {
                const BlockView b = view_block(P, dgc, MAX, bmagic, in, nbytes, s);
                ok = b.ok;
                off = b.off;
                sz = ok ? block_bytes(b.E, dgc) : 0;  // a bad block's size is unknown: the stream fails anyway
            }
            uint64_t tot;
            const uint64_t pre = block_exclusive_scan<uint64_t>(sz, &tot);
            if (s < P.nseg && (!ok || off != at + pre)) bad = 1u;
            at += tot;
        }
        if (__syncthreads_or(bad != 0u) || at != nbytes) st = kBadBlock;
    }
    // pass 2
    uint32_t tile_run = 0;
    uint64_t slot_run = 0;
    for (int r = 0; r < P.nseg; r += kBlock) {
        const int s = r + int(threadIdx.x);
        BlockView b{};
        if (s < P.nseg && !st) b = view_block(P, dgc, MAX, bmagic, in, nbytes, s);
        const uint32_t E = st ? 0u : b.E, cnt = st ? 0u : b.cnt;
        uint32_t ttot;
        uint64_t ctot;
        const uint32_t tpre = block_exclusive_scan<uint32_t>((E + kUTile - 1) / kUTile, &ttot);
        const uint64_t cpre = block_exclusive_scan<uint64_t>(cnt, &ctot);
        if (s < P.nseg) {
            w.blk_off[s] = st ? 0 : b.off;
            w.seg_E[s] = E;
            w.seg_cnt[s] = cnt;
            w.tile_base[s] = tile_run + tpre;
            const uint64_t sb = slot_run + cpre;
            w.slot_base[s] = static_cast<uint32_t>(min<uint64_t>(sb, 0xFFFFFFFFull));
            seg_off[s] = static_cast<uint32_t>(min<uint64_t>(sb, cap));
            if (seg_scale) seg_scale[s] = dgc || st ? 0.0f : dev_u2f(b.w3);
        }
        tile_run += ttot;
        slot_run += ctot;
    }
    if (threadIdx.x == 0) {
        w.tile_base[P.nseg] = tile_run;
        w.slot_base[P.nseg] = static_cast<uint32_t>(min<uint64_t>(slot_run, 0xFFFFFFFFull));
        seg_off[P.nseg] = static_cast<uint32_t>(min<uint64_t>(slot_run, cap));
        if (slot_run > cap) st |= kOverCap;
        *status = st;
    }
}

// Segment of tile t (the last s with tile_base[s] <= t), from an LDS copy of
// the table when it fits.
constexpr int kLdsSegs = 4096;
struct TileOf {
    const uint32_t *tb;
    int nseg;
    __device__ void init(const uint32_t *tile_base, int n, uint32_t *lds) {
        nseg = n;
        if (n <= kLdsSegs) {
            for (int i = threadIdx.x; i < n; i += kBlock) lds[i] = tile_base[i];
            __syncthreads();
            tb = lds;
        } else {
            tb = tile_base;
        }
    }
    __device__ uint32_t segment(uint32_t t) const {
        int lo = 0, hi = nseg - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (tb[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        return static_cast<uint32_t>(lo);
    }
};

// Exclusive prefix of one value per element in the tile's order, element
// (row i, thread t) being code i * kBlock + t: a wave scan per row, then one
// wave scans the kUPer * kWaves (row, wave) totals.  Returns the tile's total.
__device__ __forceinline__ uint32_t block_row_scan(const uint32_t (&v)[kUPer], uint32_t (&ex)[kUPer]) {
    static_assert(kUPer * kWaves <= kWave, "one wave scans the row totals");
    __shared__ uint32_t tot[kUPer * kWaves + 1];
    uint32_t incl[kUPer];
#pragma unroll
    for (uint32_t i = 0; i < kUPer; ++i) {
        const uint32_t x = wave_inclusive_scan(v[i]);
        incl[i] = x;
        if (lane_id() == kWave - 1) tot[i * kWaves + wave_id()] = x;
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
        const uint32_t t = threadIdx.x < kUPer * kWaves ? tot[threadIdx.x] : 0u;
        const uint32_t x = wave_inclusive_scan(t);
        if (threadIdx.x < kUPer * kWaves) tot[threadIdx.x] = x - t;
        if (threadIdx.x == kWave - 1) tot[kUPer * kWaves] = x;
    }
    __syncthreads();
#pragma unroll
    for (uint32_t i = 0; i < kUPer; ++i) ex[i] = tot[i * kWaves + wave_id()] + incl[i] - v[i];
    const uint32_t all = tot[kUPer * kWaves];
    __syncthreads();
    return all;
}

// Code i * kBlock + t of the tile is thread t's i-th: loads and the entries'
// stores are coalesced along a row; the row-order scans give every code its
// position and slot from the tile's checkpoint.
__global__ __launch_bounds__(kBlock) void unpack_write_kernel(PlanDev P, int kind, const uint8_t *__restrict__ in,
                                                              UnpackWs w, uint64_t cap,
                                                              const float *__restrict__ seg_scale,
                                                              uint32_t *__restrict__ out_idx,
                                                              float *__restrict__ out_val, uint32_t *status) {
    const uint32_t ntiles = w.tile_base[P.nseg];
    if (blockIdx.x >= ntiles) return;
    const bool dgc = kind == GC_KIND_DGC;
    const uint32_t MAX = dgc ? 65535u : 32767u;
    const uint32_t rmask = dgc ? 0xFFFFu : 0x7FFFu;
    __shared__ uint32_t lds[kLdsSegs];
    TileOf table;
    table.init(w.tile_base, P.nseg, lds);
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint32_t s = table.segment(t);
        const SegDev seg = P.seg[s];
        const uint32_t E = w.seg_E[s], cnt = w.seg_cnt[s];
        const uint32_t c = t - w.tile_base[s];
        const uint32_t j0 = c * kUTile;
        const uint32_t nck = (E + kUTile - 1) / kUTile;
        const uint8_t *blk = in + w.blk_off[s];
        const uint16_t *runs = reinterpret_cast<const uint16_t *>(blk + 16);
        const float *vals = reinterpret_cast<const float *>(blk + 16 + 2ull * E + 2ull * (E & 1u));
        const uint32_t *ck = reinterpret_cast<const uint32_t *>(blk + 16 + 2ull * E + 2ull * (E & 1u) + (dgc ? 4ull * E : 0));
        const float scale = dgc ? 0.0f : seg_scale[s];
        // the tile's start and, unless it is the block's last, the next tile's
        const uint32_t e0 = ck[2 * c], p0 = ck[2 * c + 1];
        const bool last = c + 1 >= nck;
        const uint32_t e1 = last ? cnt : ck[2 * c + 2], p1 = last ? 0u : ck[2 * c + 3];
        uint32_t code[kUPer], steps[kUPer], ent[kUPer];
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i) code[i] = runs[min(j0 + i * kBlock + threadIdx.x, E - 1)];
        float v[kUPer] = {};
        if (dgc) {  // an AdaComp block has no value array: never read past its codes
#pragma unroll
            for (uint32_t i = 0; i < kUPer; ++i) v[i] = vals[min(j0 + i * kBlock + threadIdx.x, E - 1)];
        }
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i) {
            const bool in_tile = j0 + i * kBlock + threadIdx.x < E;
            const uint32_t r = code[i] & rmask;
            ent[i] = in_tile && r != MAX ? 1u : 0u;
            steps[i] = !in_tile ? 0u : (r == MAX ? MAX : r + 1);
        }
        uint32_t spre[kUPer], epre[kUPer];
        const uint32_t stot = block_row_scan(steps, spre);
        const uint32_t etot = block_row_scan(ent, epre);
        uint32_t bad = 0;
        // the tile must end where the next checkpoint (or the block's count) says
        if (uint64_t(e0) + etot != e1 || (!last && uint64_t(p0) + stot != p1)) bad |= kBadCount;
        // slots of this block's entries stay inside its range of the message
        const uint64_t slot_end = min<uint64_t>(uint64_t(w.slot_base[s]) + cnt, cap);
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i) {
            if (!ent[i]) continue;
            const uint64_t rel = uint64_t(p0) + spre[i] + (code[i] & rmask);
            const uint64_t slot = uint64_t(w.slot_base[s]) + e0 + epre[i];
            if (rel >= seg.len) {
                bad |= kBadEntry;
            } else if (slot < slot_end) {
                __builtin_nontemporal_store(static_cast<uint32_t>(seg.off + rel), out_idx + slot);
                __builtin_nontemporal_store(dgc ? v[i] : ((code[i] & 0x8000u) ? -scale : scale), out_val + slot);
            }
        }
        if (bad) atomicOr(status, bad);
    }
}

}  // namespace

size_t unpack_workspace_bytes(const gc_plan *plan) {
    size_t b = 0;
    (void)unpack_layout(plan, nullptr, &b);
    return b;
}

}  // namespace gc

using namespace gc;

extern "C" gc_status gc_unpack(const gc_plan *plan, int kind, const uint8_t *in, uint64_t in_bytes,
                               gc_sparse *out, uint32_t *status, void *ws, size_t ws_bytes,
                               hipStream_t stream) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_unpack: plan is null");
    if (kind != GC_KIND_DGC && kind != GC_KIND_ADACOMP)
        return set_error(GC_EINVAL, "gc_unpack: kind must be GC_KIND_DGC or GC_KIND_ADACOMP");
    if (!in || !status) return set_error(GC_EINVAL, "gc_unpack: in and status must be non-null");
    if (reinterpret_cast<uintptr_t>(in) % 4) return set_error(GC_EINVAL, "gc_unpack: in must be 4-byte aligned");
    if (in_bytes < 16) return set_error(GC_EINVAL, "gc_unpack: a stream holds at least its 16-byte header");
    if (!out || !out->idx || !out->val || !out->seg_off || (kind == GC_KIND_ADACOMP && !out->seg_scale))
        return set_error(GC_EINVAL, "gc_unpack: message pointers must be non-null");
    if (!ws || ws_bytes < unpack_workspace_bytes(plan))
        return set_error(GC_ECAPACITY, "gc_unpack: workspace smaller than gc_plan_workspace_bytes(GC_OP_UNPACK)");
    if (reinterpret_cast<uintptr_t>(ws) % 256) return set_error(GC_EINVAL, "gc_unpack: workspace must be 256-byte aligned");
    PlanDev P;
    gc_status st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    UnpackWs w = unpack_layout(plan, ws, nullptr);
    constexpr size_t kTileGrid = 8192;
    const unsigned grid = static_cast<unsigned>(std::min<size_t>(w.max_tiles, kTileGrid));
    GC_LAUNCH("unpack_layout", stream, unpack_layout_kernel<<<1, kBlock, 0, stream>>>(P, kind, in, in_bytes, out->cap, w,
                                                                                     out->seg_off, out->seg_scale, status));
    GC_LAUNCH("unpack_write", stream, unpack_write_kernel<<<grid, kBlock, 0, stream>>>(P, kind, in, w, out->cap,
                                                                                       out->seg_scale, out->idx,
                                                                                       out->val, status));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_unpack launch");
    return GC_OK;
}
