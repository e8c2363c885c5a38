// Byte-exact run-length packing of a sparse message.
// "Deep Gradient Compression" (Lin et al.) §3.1: 32-bit values with 16-bit
// zero-run lengths; AdaComp messages carry only a sign per entry plus one
// layer scale, so their 16-bit code holds the sign in bit 15.
//
// Entries of a segment are processed in tiles of 4096.  A run longer than
// the code can hold is split with escapes; an entry's slot in its block is
// its rank in the segment plus the escapes emitted before it.  Escapes are
// rare (a gap of 32767+ unsent elements), so the count pass adds per-segment
// totals with integer atomics, and the write pass scans escape counts only
// in segments and tiles that have any.  The count pass reads a tile in the
// 4-wide lane layout of the dense kernels (one 16-byte load per lane and
// row) and leaves a record of the tile (segment, entry range, segment
// geometry), so that a write workgroup starts its data loads after a single
// round trip; the write pass is lane-strided, so that each wave's 2-byte
// code stores cover contiguous bytes.
#include <algorithm>

#include "gc_internal.hpp"

namespace gc {

namespace {

constexpr uint32_t kTile = 4096;
constexpr int kTileRows = kTile / (4 * kBlock);

struct PackWs {
    uint32_t *tile_base;  // [nseg + 1] first tile of each segment; [nseg] = tile count
    uint32_t *tile_esc;   // [max_tiles] escapes per tile
    uint4 *tile_rec;      // [2 * max_tiles] per tile: {segment, first entry, entries, tile in segment},
                          //   {segment offset, length, first entry of the segment, 0}
    uint32_t *seg_esc;    // [nseg] escapes per segment
    uint64_t *blk_off;    // [nseg] byte offset of each block
    uint32_t *seg_E;      // [nseg]
    uint32_t *overflow;   // [1] set by the layout pass when the stream exceeds out_cap
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
    w.tile_rec = c.take<uint4>(2 * w.max_tiles);
    w.seg_esc = c.take<uint32_t>(p->nseg);
    w.blk_off = c.take<uint64_t>(p->nseg);
    w.seg_E = c.take<uint32_t>(p->nseg);
    w.overflow = c.take<uint32_t>(1);
    if (bytes) *bytes = c.used + 256;
    return w;
}

constexpr uint32_t magic(char a, char b, char c, char d) {
    return uint32_t(uint8_t(a)) | uint32_t(uint8_t(b)) << 8 | uint32_t(uint8_t(c)) << 16 |
           uint32_t(uint8_t(d)) << 24;
}

// The segment of an entry, as the gap computation needs it.
struct EntryCtx {
    uint32_t first;  // first entry of the segment
    uint32_t off;    // segment offset (below 2^32, as every index)
    uint32_t len;    // segment length
};

// Entries of segment s, clamped so that a malformed message can never make
// the packer read past the message: at most max_entries (the segment's
// length) and never past cap.
__device__ __forceinline__ uint32_t seg_entries(const uint32_t *seg_off, int s, uint32_t max_entries,
                                                uint64_t cap) {
    uint32_t a = seg_off[s], b = seg_off[s + 1];
    if (b <= a || a >= cap) return 0;
    uint64_t n = b - a;
    if (n > max_entries) n = max_entries;
    if (a + n > cap) n = cap - a;
    return static_cast<uint32_t>(n);
}

// A DGC message may hold more than the plan's k per segment (a per-call
// density, or the sampled selection's budget), an AdaComp one up to every
// element: either kind is bounded by the segment's length.
__device__ __forceinline__ uint32_t seg_max_entries(const SegDev &s, int) { return s.len; }

// Gap before entry j (unsent elements since the previous entry) from the
// loaded indices cur = idx[j] and prv = idx[j - 1]; out-of-order or
// out-of-segment indices count as gap 0.  Escapes before the entry are
// floor(gap / MAX).
// With rel = cur - off and p = prv - off (when prv >= off), the gap is
// rel - p - 1 when p < rel < len; rel when j is the segment's first entry or
// prv < off; 0 otherwise.  All in u32: no difference can wrap.
__device__ __forceinline__ uint32_t entry_gap(const EntryCtx &x, uint32_t j, uint32_t cur, uint32_t prv) {
    if (cur < x.off) return 0u;
    const uint32_t rel = cur - x.off;
    if (rel >= x.len) return 0u;
    if (j > x.first && prv >= x.off) {
        const uint32_t p = prv - x.off;
        return p < rel ? rel - p - 1 : 0u;
    }
    return rel;
}

// Message loads keep the default cache policy, unlike the dense streams: an
// entry's predecessor is read by a second load from the same lines, and the
// non-temporal hint had them fetched twice (measured: 8% more HBM reads and
// a 20% slower write pass).
constexpr int kKeep = 0;

// The tile's entries [j0, j0 + cnt) in the 4-wide layout: cur[r][q] =
// idx[j0 + 1024 r + 4 t + q] (0 past cnt, from the buffer's range check)
// and prv0[r] = the entry before the lane's first one of row r (clamped
// into the tile when that entry is the segment's first, where it is unused,
// or lies past the tile).  All loads are issued before any is used.
__device__ __forceinline__ void load_tile(const uint32_t *__restrict__ a, uint32_t first, uint32_t j0,
                                          uint32_t cnt, uint32_t (&cur)[kTileRows][4],
                                          uint32_t (&prv0)[kTileRows]) {
    const BufRsrc r = chunk_buf(reinterpret_cast<const float *>(a + j0), cnt);
#pragma unroll
    for (int row = 0; row < kTileRows; ++row) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(row_elem(row) * 4u), 0, kKeep);
        cur[row][0] = v.x;
        cur[row][1] = v.y;
        cur[row][2] = v.z;
        cur[row][3] = v.w;
        const uint32_t j = min(j0 + row_elem(row), j0 + cnt);
        prv0[row] = a[j > first ? j - 1 : first];
    }
}

__device__ __forceinline__ uint32_t prev_of(const uint32_t (&cur)[kTileRows][4], const uint32_t (&prv0)[kTileRows],
                                            int row, int q) {
    return q == 0 ? prv0[row] : cur[row][q - 1];
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
// table (and the tile count after it) to LDS once when it fits, so the
// searches cost no global round trips.
constexpr int kLdsSegs = 4096;

struct TileTable {
    const uint32_t *tb;
    int nseg;
    __device__ void init(const uint32_t *tile_base, int n, uint32_t *lds) {
        nseg = n;
        if (n <= kLdsSegs) {
            for (int i = threadIdx.x; i <= n; i += kBlock) lds[i] = tile_base[i];
            __syncthreads();
            tb = lds;
        } else {
            tb = tile_base;
        }
    }
    __device__ uint32_t count() const { return tb[nseg]; }
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
    __shared__ uint32_t lds[kLdsSegs + 1];
    TileTable table;
    table.init(w.tile_base, P.nseg, lds);
    const uint32_t ntiles = table.count();
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint32_t s = table.segment(t);
        const uint32_t ts = t - table.tb[s];
        const SegDev sg = P.seg[s];
        EntryCtx x;
        x.first = seg_off[s];
        x.off = static_cast<uint32_t>(sg.off);
        x.len = sg.len;
        const uint32_t end = x.first + seg_entries(seg_off, s, seg_max_entries(sg, kind), cap);
        const uint32_t j0 = x.first + ts * kTile;
        const uint32_t cnt = min(end - j0, kTile);
        uint32_t cur[kTileRows][4], prv0[kTileRows];
        load_tile(idx, x.first, j0, cnt, cur, prv0);
        uint32_t esc = 0;
#pragma unroll
        for (int row = 0; row < kTileRows; ++row)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t e = row_elem(row) + q;
                if (e < cnt) esc += entry_gap(x, j0 + e, cur[row][q], prev_of(cur, prv0, row, q)) / MAX;
            }
        uint32_t tot;
        (void)block_exclusive_scan(esc, &tot);
        if (threadIdx.x == 0) {
            w.tile_esc[t] = tot;
            w.tile_rec[2 * size_t(t)] = make_uint4(s, j0, cnt, ts);
            w.tile_rec[2 * size_t(t) + 1] =
                make_uint4(x.off, x.len, x.first, 0u);
            if (tot) atomicAdd(&w.seg_esc[s], tot);
        }
    }
}

// One workgroup: size every block from its entries and escapes; when the
// stream fits out_cap, write the stream header, block headers and pads;
// always the stream length, and the overflow flag the write pass reads.
__global__ __launch_bounds__(kBlock) void pack_layout_kernel(PlanDev P, int kind, uint64_t cap, uint32_t MAX,
                                                             const uint32_t *__restrict__ seg_off,
                                                             const float *__restrict__ seg_scale,
                                                             uint8_t *__restrict__ out, uint64_t out_cap,
                                                             uint64_t *__restrict__ out_bytes, PackWs w) {
    uint64_t byte_run = 16;
    const bool dgc = kind == GC_KIND_DGC;
    for (int r = 0; r < P.nseg; r += kBlock) {
        int s = r + threadIdx.x;
        uint64_t sz = 0;
        uint32_t E = 0;
        if (s < P.nseg) {
            const SegDev sg = P.seg[s];
            const uint32_t maxe = seg_max_entries(sg, kind);
            const uint32_t cnt = seg_entries(seg_off, s, maxe, cap);
            uint32_t esc = w.seg_esc[s];
            // never more codes than a segment of this length can need
            uint64_t cap_e = uint64_t(maxe) + sg.len / MAX + 1;
            uint64_t e64 = uint64_t(cnt) + esc;
            E = static_cast<uint32_t>(e64 < cap_e ? e64 : cap_e);
            sz = 16 + 2ull * E + 2ull * (E & 1u) + (dgc ? 4ull * E : 0ull);
        }
        uint64_t tot;
        uint64_t pre = block_exclusive_scan<uint64_t>(sz, &tot);
        if (s < P.nseg) {
            w.blk_off[s] = byte_run + pre;
            w.seg_E[s] = E;
        }
        byte_run += tot;
    }
    const bool fits = byte_run <= out_cap;
    __syncthreads();
    if (fits) {
        for (int s = threadIdx.x; s < P.nseg; s += kBlock) {
            const uint64_t at = w.blk_off[s];
            const uint32_t E = w.seg_E[s];
            uint32_t *h = reinterpret_cast<uint32_t *>(out + at);
            h[0] = dgc ? magic('D', 'G', 'C', '1') : magic('A', 'D', 'C', '1');
            h[1] = P.seg[s].len;
            h[2] = E;
            h[3] = dgc ? seg_entries(seg_off, s, seg_max_entries(P.seg[s], kind), cap) : dev_f2u(seg_scale[s]);
            if (E & 1u) *reinterpret_cast<uint16_t *>(out + at + 16 + 2ull * E) = 0;
        }
    }
    if (threadIdx.x == 0) {
        if (fits) {
            uint32_t *h = reinterpret_cast<uint32_t *>(out);
            h[0] = magic('G', 'C', 'P', '1');
            h[1] = static_cast<uint32_t>(kind);
            h[2] = static_cast<uint32_t>(P.nseg);
            h[3] = 0u;
        }
        *out_bytes = byte_run;
        *w.overflow = fits ? 0u : 1u;
    }
}

// Write pass.  Entries are lane-strided here (entry i * 256 + t of the tile
// in thread t), so that each 2-byte code store of a wave covers 128
// contiguous bytes.  The loads of a tile are issued before its escape count
// is known; a tile with escapes (rare) drops them and walks 16 contiguous
// entries per thread in two light passes (escapes, then slots), reloading
// what it needs, so that its registers do not add to the common path's.
constexpr uint32_t kPerThread = kTile / kBlock;

// A wave-uniform value moved to a scalar register (the tile geometry is read
// with vector loads; every lane holds the same value).
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

__global__ __launch_bounds__(kBlock) void pack_write_kernel(PlanDev P, int kind, size_t max_tiles,
                                                            const uint32_t *__restrict__ idx,
                                                            const float *__restrict__ val, uint32_t MAX,
                                                            uint8_t *__restrict__ out, PackWs w) {
    const bool dgc = kind == GC_KIND_DGC;
    if (*w.overflow) return;  // the stream does not fit out_cap: nothing is written
    for (uint32_t t = blockIdx.x; t < max_tiles; t += gridDim.x) {
        // the tile count and the tile's record in one round trip (records
        // past the count are never used)
        const uint32_t ntiles = uni(w.tile_base[P.nseg]);
        const uint4 ra = w.tile_rec[2 * size_t(t)], rb = w.tile_rec[2 * size_t(t) + 1];
        if (t >= ntiles) break;
        const uint32_t s = uni(ra.x), j0 = uni(ra.y), cnt = uni(ra.z);
        EntryCtx x;
        x.off = uni(rb.x);
        x.len = uni(rb.y);
        x.first = uni(rb.z);
        const uint32_t tile0 = t - uni(ra.w);
        // buffer resources over the tile (32-bit offsets; loads past the
        // range return 0): entries, values, and the entries shifted back by
        // one (from the entry before the tile unless the tile is the
        // segment's first, where entry 0's predecessor is unused)
        const uint32_t d = uni(j0 > x.first ? 1u : 0u);
        const BufRsrc ri = chunk_buf(reinterpret_cast<const float *>(idx + j0), cnt);
        const BufRsrc rp = chunk_buf(reinterpret_cast<const float *>(idx + j0 - d), cnt + d);
        const BufRsrc rv = chunk_buf(val + j0, cnt);
        uint32_t cur[kPerThread], prv[kPerThread];
        float v[kPerThread];
#pragma unroll
        for (uint32_t i = 0; i < kPerThread; ++i) {
            const uint32_t e = i * kBlock + threadIdx.x;
            const uint32_t ep = e + d > 0 ? e + d - 1 : 0u;
            cur[i] = __builtin_amdgcn_raw_buffer_load_b32(ri, static_cast<int>(4 * e), 0, kKeep);
            prv[i] = __builtin_amdgcn_raw_buffer_load_b32(rp, static_cast<int>(4 * ep), 0, kKeep);
            v[i] = dev_u2f(__builtin_amdgcn_raw_buffer_load_b32(rv, static_cast<int>(4 * e), 0, kKeep));
        }
        const uint32_t E = w.seg_E[s];
        const uint32_t tile_esc = w.tile_esc[t], seg_esc = w.seg_esc[s];
        uint8_t *blk = out + w.blk_off[s];
        uint16_t *runs = reinterpret_cast<uint16_t *>(blk + 16);
        float *vals = reinterpret_cast<float *>(blk + 16 + 2ull * E + 2ull * (E & 1u));
        // escapes emitted before this tile in its segment
        uint32_t esc_base = 0;
        if (seg_esc != 0) {
            uint32_t part = 0;
            for (uint32_t u = tile0 + threadIdx.x; u < t; u += kBlock) part += w.tile_esc[u];
            uint32_t all;
            (void)block_exclusive_scan(part, &all);
            esc_base = all;
        }
        auto put = [&](uint32_t slot, uint32_t gap, float value) {
            // the packed stream is not read again here: non-temporal stores
            if (dgc) {
                __builtin_nontemporal_store(static_cast<uint16_t>(gap), runs + slot);
                __builtin_nontemporal_store(value, vals + slot);
            } else {
                const uint16_t sign = (dev_f2u(value) >> 31) ? 0x8000u : 0u;
                __builtin_nontemporal_store(static_cast<uint16_t>(sign | gap), runs + slot);
            }
        };
        if (tile_esc == 0) {
            // no escape in this tile: entry j goes to slot (j - first) + esc_base
#pragma unroll
            for (uint32_t i = 0; i < kPerThread; ++i) {
                const uint32_t e = i * kBlock + threadIdx.x;
                const uint32_t slot = (j0 + e - x.first) + esc_base;
                if (e >= cnt || slot >= E) continue;  // slot >= E only for malformed messages
                put(slot, entry_gap(x, j0 + e, cur[i], prv[i]), v[i]);
            }
            continue;
        }
        // tile with escapes: thread t takes entries [16 t, 16 t + 16) of the tile
        const uint32_t e0 = threadIdx.x * kPerThread;
        auto gap_at = [&](uint32_t e) {
            const uint32_t j = j0 + e;
            return entry_gap(x, j, idx[j], idx[j > x.first ? j - 1 : j]);
        };
        uint32_t mine = 0;
#pragma unroll 1
        for (uint32_t e = e0; e < min(e0 + kPerThread, cnt); ++e) mine += gap_at(e) / MAX;
        uint32_t tot;
        uint32_t before = esc_base + block_exclusive_scan(mine, &tot);
#pragma unroll 1
        for (uint32_t e = e0; e < min(e0 + kPerThread, cnt); ++e) {
            uint32_t slot = (j0 + e - x.first) + before;
            uint32_t g = gap_at(e);
            const uint32_t esc = g / MAX;
            for (uint32_t z = 0; z < esc && slot < E; ++z) {
                runs[slot] = static_cast<uint16_t>(MAX);
                if (dgc) vals[slot] = 0.0f;
                ++slot;
                g -= MAX;
            }
            before += esc;
            if (slot >= E) continue;  // only for malformed messages
            put(slot, g, val[j0 + e]);
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

// Stream bytes at most for messages of at most entries(s) entries per segment.
template <class F>
static uint64_t pack_bound_for(const gc_plan *plan, int kind, F entries) {
    const uint64_t MAX = kind == GC_KIND_DGC ? 65535 : 32767;
    const uint64_t per = kind == GC_KIND_DGC ? 6 : 2;
    uint64_t b = 16;
    for (const auto &s : plan->seg) b += 16 + 2 + per * (entries(s) + s.len / MAX + 1);
    return b;
}

extern "C" uint64_t gc_pack_bound(const gc_plan *plan, int kind) {
    if (!plan || (kind != GC_KIND_DGC && kind != GC_KIND_ADACOMP)) return 0;
    return pack_bound_for(plan, kind, [&](const SegDev &s) -> uint64_t { return kind == GC_KIND_DGC ? s.k : s.len; });
}

extern "C" uint64_t gc_dgc_pack_bound(const gc_plan *plan, const gc_dgc_options *opt) {
    if (!plan) return 0;
    if (!opt) return gc_pack_bound(plan, GC_KIND_DGC);
    return pack_bound_for(plan, GC_KIND_DGC, [&](const SegDev &s) -> uint64_t {
        if (opt->select == GC_SELECT_SAMPLED) return std::min<uint64_t>(s.len, uint64_t(opt->over) * s.k);
        if (opt->density_den == 0) return s.k;
        const uint64_t k = (uint64_t(s.len) * opt->density_num + opt->density_den - 1) / opt->density_den;
        return std::max<uint64_t>(1, std::min<uint64_t>(k, s.len));
    });
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
                                                 out_cap, out_bytes, w));
    GC_LAUNCH("pack_write", stream, pack_write_kernel<<<grid, kBlock, 0, stream>>>(P, kind, w.max_tiles, in->idx, in->val, MAX,
                                                   out, w));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_pack launch");
    return GC_OK;
}
