// Byte-exact run-length packing of a sparse message.
// "Deep Gradient Compression" (Lin et al.) §3.1: 32-bit values with 16-bit
// zero-run lengths; AdaComp messages carry only a sign per entry plus one
// layer scale, so their 16-bit code holds the sign in bit 15.
//
// Entries of a segment are processed in tiles of 4096 (16 per thread).  A run longer than the code can hold is split with escapes; an
// entry's slot in its block is its rank in the segment plus the escapes
// emitted before it.  Escapes are rare (a gap of 32767+ unsent elements), so
// the count pass adds per-segment totals with integer atomics, and the write
// pass scans escape counts only in segments and tiles that have any.
#include <algorithm>

#include "gc_internal.hpp"

namespace gc {

namespace {

constexpr uint32_t kTile = 4096;
constexpr uint32_t kPerThread = kTile / kBlock;

struct PackWs {
    uint32_t *tile_base;  // [nseg + 1] first tile of each segment
    uint32_t *tile_esc;   // [max_tiles] escapes per tile
    uint32_t *seg_esc;    // [nseg] escapes per segment
    uint64_t *blk_off;    // [nseg] byte offset of each block
    uint32_t *seg_E;      // [nseg]
    size_t max_tiles;
};

PackWs pack_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    PackWs w{};
    size_t tiles = 0;
    for (const auto &s : p->seg) tiles += ceil_div(s.len, kTile);
    w.max_tiles = tiles + 1;
    w.tile_base = c.take<uint32_t>(p->nseg + 1);
    w.tile_esc = c.take<uint32_t>(w.max_tiles + 1);
    w.seg_esc = c.take<uint32_t>(p->nseg);
    w.blk_off = c.take<uint64_t>(p->nseg);
    w.seg_E = c.take<uint32_t>(p->nseg);
    if (bytes) *bytes = c.used + 256;
    return w;
}

constexpr uint32_t magic(char a, char b, char c, char d) {
    return uint32_t(uint8_t(a)) | uint32_t(uint8_t(b)) << 8 | uint32_t(uint8_t(c)) << 16 |
           uint32_t(uint8_t(d)) << 24;
}

struct EntryCtx {
    uint32_t s, first, end;  // segment and its entry range
    uint64_t off;            // segment offset
    uint32_t len;            // segment length
};

// Entries of segment s, clamped so that a malformed message can never make
// the packer read past the message or write past gc_pack_bound: at most
// max_entries (k for DGC, the length for AdaComp) and never past cap.
__device__ __forceinline__ uint32_t seg_entries(const uint32_t *seg_off, int s, uint32_t max_entries,
                                                uint64_t cap) {
    uint32_t a = seg_off[s], b = seg_off[s + 1];
    if (b <= a || a >= cap) return 0;
    uint64_t n = b - a;
    if (n > max_entries) n = max_entries;
    if (a + n > cap) n = cap - a;
    return static_cast<uint32_t>(n);
}

__device__ __forceinline__ uint32_t seg_max_entries(const SegDev &s, int kind) {
    return kind == GC_KIND_DGC ? s.k : s.len;
}

__device__ __forceinline__ EntryCtx entry_ctx(const PlanDev &P, const uint32_t *seg_off, int kind,
                                              uint64_t cap, uint32_t s) {
    EntryCtx x;
    x.s = s;
    x.first = seg_off[s];
    x.end = x.first + seg_entries(seg_off, s, seg_max_entries(P.seg[s], kind), cap);
    x.off = P.seg[s].off;
    x.len = P.seg[s].len;
    return x;
}

// Gap before entry j (unsent elements since the previous entry) from the
// loaded indices cur = idx[j] and prv = idx[j - 1]; out-of-order or
// out-of-segment indices count as gap 0.  Escapes before the entry are
// floor(gap / MAX).
__device__ __forceinline__ uint32_t entry_gap(const EntryCtx &x, uint32_t j, uint32_t cur, uint32_t prv) {
    const uint64_t rel = cur >= x.off ? uint64_t(cur) - x.off : uint64_t(x.len);
    const uint64_t prev_next = j > x.first ? (prv >= x.off ? uint64_t(prv) - x.off + 1 : 0) : 0;
    return (rel < x.len && rel >= prev_next) ? static_cast<uint32_t>(rel - prev_next) : 0u;
}

// Loads idx[j] and idx[j - 1] for entries j = j0 + i * stride of one tile,
// all issued before any is used: addresses are clamped into the segment's
// entries (which the tile's existence makes non-empty), so no load sits
// behind a branch.
template <uint32_t N>
__device__ __forceinline__ void load_ids(const uint32_t *__restrict__ idx, const EntryCtx &x, uint32_t j0,
                                         uint32_t stride, uint32_t (&cur)[N], uint32_t (&prv)[N]) {
    const uint32_t last = x.end > x.first ? x.end - 1 : x.first;
#pragma unroll
    for (uint32_t i = 0; i < N; ++i) {
        const uint32_t j = min(j0 + i * stride, last);
        cur[i] = idx[j];
        prv[i] = idx[j > x.first ? j - 1 : j];
    }
}

// One workgroup: tile counts per segment -> tile_base.
__global__ __launch_bounds__(kBlock) void pack_tiles_kernel(PlanDev P, int kind,
                                                            const uint32_t *__restrict__ seg_off,
                                                            uint64_t cap, PackWs w) {
    const int nseg = P.nseg;
    uint32_t run = 0;
    for (int r = 0; r < nseg; r += kBlock) {
        int s = r + threadIdx.x;
        uint32_t v = 0;
        if (s < nseg) v = (seg_entries(seg_off, s, seg_max_entries(P.seg[s], kind), cap) + kTile - 1) / kTile;
        uint32_t tot;
        uint32_t pre = block_exclusive_scan(v, &tot);
        if (s < nseg) {
            w.tile_base[s] = run + pre;
            w.seg_esc[s] = 0u;
        }
        run += tot;
    }
    if (threadIdx.x == 0) w.tile_base[nseg] = run;
}

// Segment of tile t: the last s with tile_base[s] <= t.  Workgroups copy the
// table to LDS once when it fits, so the searches cost no global round trips.
constexpr int kLdsSegs = 4096;

struct TileTable {
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
            int mid = (lo + hi + 1) / 2;
            if (tb[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        return static_cast<uint32_t>(lo);
    }
};

__global__ __launch_bounds__(kBlock) void pack_count_kernel(PlanDev P, int kind,
                                                            const uint32_t *__restrict__ idx,
                                                            const uint32_t *__restrict__ seg_off,
                                                            uint64_t cap, uint32_t MAX, PackWs w) {
    const uint32_t ntiles = w.tile_base[P.nseg];
    if (blockIdx.x >= ntiles) return;
    __shared__ uint32_t lds[kLdsSegs];
    TileTable table;
    table.init(w.tile_base, P.nseg, lds);
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const EntryCtx x = entry_ctx(P, seg_off, kind, cap, table.segment(t));
    const uint32_t j0 = x.first + (t - w.tile_base[x.s]) * kTile;
    uint32_t cur[kPerThread], prv[kPerThread];
    load_ids(idx, x, j0 + threadIdx.x, kBlock, cur, prv);
    uint32_t esc = 0;
#pragma unroll
    for (uint32_t i = 0; i < kPerThread; ++i) {
        const uint32_t j = j0 + i * kBlock + threadIdx.x;
        if (j < x.end) esc += entry_gap(x, j, cur[i], prv[i]) / MAX;
    }
    uint32_t tot;
    (void)block_exclusive_scan(esc, &tot);
    if (threadIdx.x == 0) {
        w.tile_esc[t] = tot;
        if (tot) atomicAdd(&w.seg_esc[x.s], tot);
    }
    }
}

// One workgroup: size every block from its entries and escapes, write the
// stream header, block headers and pads, and the stream length.
__global__ __launch_bounds__(kBlock) void pack_layout_kernel(PlanDev P, int kind, uint64_t cap, uint32_t MAX,
                                                             const uint32_t *__restrict__ seg_off,
                                                             const float *__restrict__ seg_scale,
                                                             uint8_t *__restrict__ out,
                                                             uint64_t *__restrict__ out_bytes, PackWs w) {
    uint64_t byte_run = 16;
    const bool dgc = kind == GC_KIND_DGC;
    for (int r = 0; r < P.nseg; r += kBlock) {
        int s = r + threadIdx.x;
        uint64_t sz = 0;
        uint32_t E = 0, cnt = 0;
        if (s < P.nseg) {
            const SegDev sg = P.seg[s];
            const uint32_t maxe = seg_max_entries(sg, kind);
            cnt = seg_entries(seg_off, s, maxe, cap);
            uint32_t esc = w.seg_esc[s];
            // never more slots than gc_pack_bound reserves for the segment
            uint64_t cap_e = uint64_t(maxe) + sg.len / MAX + 1;
            uint64_t e64 = uint64_t(cnt) + esc;
            E = static_cast<uint32_t>(e64 < cap_e ? e64 : cap_e);
            sz = 16 + 2ull * E + 2ull * (E & 1u) + (dgc ? 4ull * E : 0ull);
        }
        uint64_t tot;
        uint64_t pre = block_exclusive_scan<uint64_t>(sz, &tot);
        if (s < P.nseg) {
            uint64_t at = byte_run + pre;
            w.blk_off[s] = at;
            w.seg_E[s] = E;
            uint32_t *h = reinterpret_cast<uint32_t *>(out + at);
            h[0] = dgc ? magic('D', 'G', 'C', '1') : magic('A', 'D', 'C', '1');
            h[1] = P.seg[s].len;
            h[2] = E;
            h[3] = dgc ? cnt : dev_f2u(seg_scale[s]);
            if (E & 1u) *reinterpret_cast<uint16_t *>(out + at + 16 + 2ull * E) = 0;
        }
        byte_run += tot;
    }
    if (threadIdx.x == 0) {
        uint32_t *h = reinterpret_cast<uint32_t *>(out);
        h[0] = magic('G', 'C', 'P', '1');
        h[1] = static_cast<uint32_t>(kind);
        h[2] = static_cast<uint32_t>(P.nseg);
        h[3] = 0u;
        *out_bytes = byte_run;
    }
}

__global__ __launch_bounds__(kBlock) void pack_write_kernel(PlanDev P, int kind, uint64_t cap,
                                                            const uint32_t *__restrict__ idx,
                                                            const float *__restrict__ val,
                                                            const uint32_t *__restrict__ seg_off,
                                                            uint32_t MAX, uint8_t *__restrict__ out,
                                                            PackWs w) {
    const uint32_t ntiles = w.tile_base[P.nseg];
    if (blockIdx.x >= ntiles) return;
    const bool dgc = kind == GC_KIND_DGC;
    __shared__ uint32_t lds[kLdsSegs];
    TileTable table;
    table.init(w.tile_base, P.nseg, lds);
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const EntryCtx x = entry_ctx(P, seg_off, kind, cap, table.segment(t));
    const uint32_t tile0 = w.tile_base[x.s];
    const uint32_t j0 = x.first + (t - tile0) * kTile;
    const uint32_t E = w.seg_E[x.s];
    uint8_t *blk = out + w.blk_off[x.s];
    uint16_t *runs = reinterpret_cast<uint16_t *>(blk + 16);
    float *vals = reinterpret_cast<float *>(blk + 16 + 2ull * E + 2ull * (E & 1u));
    // escapes emitted before this tile in its segment
    uint32_t esc_base = 0;
    if (w.seg_esc[x.s] != 0) {
        uint32_t part = 0;
        for (uint32_t u = tile0 + threadIdx.x; u < t; u += kBlock) part += w.tile_esc[u];
        uint32_t all;
        (void)block_exclusive_scan(part, &all);
        esc_base = all;
    }
    if (w.tile_esc[t] == 0) {
        // no escape in this tile: entry j goes to slot (j - first) + esc_base
        uint32_t cur[kPerThread], prv[kPerThread];
        load_ids(idx, x, j0 + threadIdx.x, kBlock, cur, prv);
        float v[kPerThread];
        const uint32_t last = x.end > x.first ? x.end - 1 : x.first;
#pragma unroll
        for (uint32_t i = 0; i < kPerThread; ++i) v[i] = val[min(j0 + i * kBlock + threadIdx.x, last)];
#pragma unroll
        for (uint32_t i = 0; i < kPerThread; ++i) {
            const uint32_t j = j0 + i * kBlock + threadIdx.x;
            const uint32_t slot = (j - x.first) + esc_base;
            if (j >= x.end || slot >= E) continue;  // slot >= E only for malformed messages
            const uint32_t gap = entry_gap(x, j, cur[i], prv[i]);
            // the packed stream is not read again here: non-temporal stores
            if (dgc) {
                __builtin_nontemporal_store(static_cast<uint16_t>(gap), runs + slot);
                __builtin_nontemporal_store(v[i], vals + slot);
            } else {
                const uint16_t sign = (dev_f2u(v[i]) >> 31) ? 0x8000u : 0u;
                __builtin_nontemporal_store(static_cast<uint16_t>(sign | gap), runs + slot);
            }
        }
        continue;
    }
    // tile with escapes: thread-contiguous entries and an in-tile scan
    uint32_t esc[kPerThread], gap[kPerThread];
    {
        uint32_t cur[kPerThread], prv[kPerThread];
        load_ids(idx, x, j0 + threadIdx.x * kPerThread, 1u, cur, prv);
#pragma unroll
        for (uint32_t i = 0; i < kPerThread; ++i) {
            const uint32_t j = j0 + threadIdx.x * kPerThread + i;
            gap[i] = j < x.end ? entry_gap(x, j, cur[i], prv[i]) : 0u;
            esc[i] = gap[i] / MAX;
        }
    }
    uint32_t mine = 0;
#pragma unroll
    for (uint32_t i = 0; i < kPerThread; ++i) mine += esc[i];
    uint32_t tot;
    uint32_t before = esc_base + block_exclusive_scan(mine, &tot);
#pragma unroll
    for (uint32_t i = 0; i < kPerThread; ++i) {
        const uint32_t j = j0 + threadIdx.x * kPerThread + i;
        if (j >= x.end) continue;
        uint32_t slot = (j - x.first) + before;
        uint32_t g = gap[i];
        for (uint32_t q = 0; q < esc[i] && slot < E; ++q) {
            runs[slot] = static_cast<uint16_t>(MAX);
            if (dgc) vals[slot] = 0.0f;
            ++slot;
            g -= MAX;
        }
        if (slot >= E) continue;  // only for malformed messages
        if (dgc) {
            runs[slot] = static_cast<uint16_t>(g);
            vals[slot] = val[j];
        } else {
            const uint16_t sign = (dev_f2u(val[j]) >> 31) ? 0x8000u : 0u;
            runs[slot] = static_cast<uint16_t>(sign | g);
        }
        before += esc[i];
    }
    }
}

}  // namespace

size_t pack_workspace_bytes(const gc_plan *plan) {
    size_t b = 0;
    (void)pack_layout(plan, nullptr, &b);
    return b;
}

}  // namespace gc

using namespace gc;

extern "C" uint64_t gc_pack_bound(const gc_plan *plan, int kind) {
    if (!plan || (kind != GC_KIND_DGC && kind != GC_KIND_ADACOMP)) return 0;
    const uint64_t MAX = kind == GC_KIND_DGC ? 65535 : 32767;
    const uint64_t per = kind == GC_KIND_DGC ? 6 : 2;
    uint64_t b = 16;
    for (const auto &s : plan->seg) {
        uint64_t entries = kind == GC_KIND_DGC ? s.k : s.len;
        b += 16 + 2 + per * (entries + s.len / MAX + 1);
    }
    return b;
}

extern "C" gc_status gc_pack(const gc_plan *plan, int kind, const gc_sparse *in, uint8_t *out,
                             uint64_t out_cap, uint64_t *out_bytes, void *ws, size_t ws_bytes,
                             hipStream_t stream) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_pack: plan is null");
    if (kind != GC_KIND_DGC && kind != GC_KIND_ADACOMP)
        return set_error(GC_EINVAL, "gc_pack: kind must be GC_KIND_DGC or GC_KIND_ADACOMP");
    if (!in || !in->idx || !in->seg_off || (kind == GC_KIND_DGC && !in->val) ||
        (kind == GC_KIND_ADACOMP && (!in->val || !in->seg_scale)))
        return set_error(GC_EINVAL, "gc_pack: message pointers must be non-null");
    if (!out || !out_bytes) return set_error(GC_EINVAL, "gc_pack: out and out_bytes must be non-null");
    if (reinterpret_cast<uintptr_t>(out) % 4)
        return set_error(GC_EINVAL, "gc_pack: out must be 4-byte aligned");
    if (out_cap < gc_pack_bound(plan, kind))
        return set_error(GC_ECAPACITY, "gc_pack: out_cap below gc_pack_bound");
    size_t need = pack_workspace_bytes(plan);
    if (!ws || ws_bytes < need)
        return set_error(GC_ECAPACITY, "gc_pack: workspace smaller than gc_plan_workspace_bytes");
    if (reinterpret_cast<uintptr_t>(ws) % 256)
        return set_error(GC_EINVAL, "gc_pack: workspace must be 256-byte aligned");
    PlanDev P;
    gc_status st = plan_device(plan, &P);
    if (st != GC_OK) return st;
    PackWs w = pack_layout(plan, ws, nullptr);
    const uint32_t MAX = kind == GC_KIND_DGC ? 65535u : 32767u;
    const uint64_t cap = in->cap;
    // one tile per workgroup up to kTileGrid tiles (each tile is a chain of
    // dependent loads, so tiles run side by side rather than in sequence);
    // the grid follows the capacity, and workgroups past the actual tile
    // count exit at once
    constexpr size_t kTileGrid = 8192;
    const unsigned grid = static_cast<unsigned>(std::min<size_t>(w.max_tiles, kTileGrid));
    GC_LAUNCH("pack_tiles", stream, pack_tiles_kernel<<<1, kBlock, 0, stream>>>(P, kind, in->seg_off, cap, w));
    GC_LAUNCH("pack_count", stream, pack_count_kernel<<<grid, kBlock, 0, stream>>>(P, kind, in->idx, in->seg_off, cap, MAX, w));
    GC_LAUNCH("pack_layout", stream, pack_layout_kernel<<<1, kBlock, 0, stream>>>(P, kind, cap, MAX, in->seg_off, in->seg_scale, out,
                                                 out_bytes, w));
    GC_LAUNCH("pack_write", stream, pack_write_kernel<<<grid, kBlock, 0, stream>>>(P, kind, cap, in->idx, in->val, in->seg_off, MAX,
                                                   out, w));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_pack launch");
    return GC_OK;
}
