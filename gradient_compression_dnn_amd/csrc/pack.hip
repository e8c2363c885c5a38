// Byte-exact run-length packing of a sparse message.
// "Deep Gradient Compression" (Lin et al.) §3.1: 32-bit values with 16-bit
// zero-run lengths; AdaComp messages carry only a sign per entry plus one
// layer scale, so their 16-bit code holds the sign in bit 15.
//
// Entries of a segment are processed in tiles of 4096.  A run longer than
// the code can hold is split with escapes; an entry's slot in its block is
// its rank in the segment plus the escapes emitted before it.  Escapes are
// rare (a gap of 32767 or 65535 unsent elements), so the stream is laid out
// first as if there were none, and written in one pass over the entries,
// which also counts each tile's escapes.  Plans of at most 512 segments take
// two passes:
//   main     every workgroup lays the stream out (escape-free) from the
//            message's segment counts in LDS; workgroup 0 writes the headers
//            and the length; every tile records its escapes and, when it has
//            none, writes its codes (and DGC values) at their slots
//   fix      returns unless some tile has escapes; otherwise lays the stream
//            out again with each segment's escapes and writes every tile
//            with the escapes before it
// Plans of more segments (a layout per workgroup would cost each of them a
// pass over every segment) take four:
//   plan     one workgroup: entries, tiles and block offsets with no escapes;
//            stream and block headers; the stream length
//   write    one workgroup per tile, as in main, from the plan's tables; a
//            flag when any tile has an escape
//   relayout one workgroup, only when flagged: blocks resized with their
//            escapes, headers and length written again
//   rewrite  one workgroup per tile, only when flagged, as in fix
// (A separate count pass reading every index before the write measured 51 us
// of 127 for the two packs of a DeepSpeech step.)  Messages are read in the
// lane-strided layout (entry i * 256 + t of the tile in thread t), so that
// each wave's 2-byte code stores cover contiguous bytes.
#include <algorithm>

#include "gc_internal.hpp"

namespace gc {

namespace {

constexpr uint32_t kTile = 4096;

struct PackWs {
    uint4 *srec;          // [nseg] {first entry, entries, E, first tile}
    uint64_t *blk_off;    // [nseg] byte offset of each block
    uint32_t *tile_seg;   // [max_tiles] segment of each tile
    uint32_t *tile_esc;   // [max_tiles] escapes per tile (write pass)
    uint8_t *tile_any;    // [max_tiles] 1 when the tile has escapes (write pass)
    uint32_t *flags;      // [0] tiles, [1] the stream exceeds out_cap, [2] some tile has an escape
    size_t max_tiles;
};

PackWs pack_layout(const gc_plan *p, void *base, size_t *bytes) {
    WsCursor c(base);
    PackWs w{};
    size_t tiles = 0;
    for (const auto &s : p->seg) tiles += ceil_div(s.len, kTile);
    w.max_tiles = tiles + 1;
    w.srec = c.take<uint4>(p->nseg);
    w.blk_off = c.take<uint64_t>(p->nseg);
    w.tile_seg = c.take<uint32_t>(w.max_tiles);
    w.tile_esc = c.take<uint32_t>(w.max_tiles);
    w.tile_any = c.take<uint8_t>(w.max_tiles);
    w.flags = c.take<uint32_t>(4);
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

constexpr uint32_t kCkpt = 4096;  // codes between a block's checkpoints

__device__ __forceinline__ uint64_t block_bytes(uint64_t E, bool dgc) {
    return 16 + 2 * E + 2 * (E & 1u) + (dgc ? 4 * E : 0) + 8 * ((E + kCkpt - 1) / kCkpt);
}

// The first block's offset: stream header and block table before it.
__device__ __forceinline__ uint64_t blocks_start(int nseg) { return 16 + 16 * uint64_t(nseg); }

// Table entry s: the block's offset, codes and entries.
__device__ __forceinline__ void write_table_entry(uint8_t *out, int s, uint64_t at, uint32_t E, uint32_t cnt) {
    uint32_t *t = reinterpret_cast<uint32_t *>(out + 16 + 16 * uint64_t(s));
    t[0] = static_cast<uint32_t>(at);
    t[1] = static_cast<uint32_t>(at >> 32);
    t[2] = E;
    t[3] = cnt;
}

// Headers of block s (at `at`, E codes, cnt entries) and its pad.
__device__ __forceinline__ void write_block_header(uint8_t *out, uint64_t at, bool dgc, uint32_t len, uint32_t E,
                                                   uint32_t cnt, float scale) {
    uint32_t *h = reinterpret_cast<uint32_t *>(out + at);
    h[0] = dgc ? magic('D', 'G', 'C', '1') : magic('A', 'D', 'C', '1');
    h[1] = len;
    h[2] = E;
    h[3] = dgc ? cnt : dev_f2u(scale);
    if (E & 1u) *reinterpret_cast<uint16_t *>(out + at + 16 + 2ull * E) = 0;
}

__device__ __forceinline__ void write_stream_header(uint8_t *out, int kind, int nseg) {
    uint32_t *h = reinterpret_cast<uint32_t *>(out);
    h[0] = magic('G', 'C', 'P', '2');
    h[1] = static_cast<uint32_t>(kind);
    h[2] = static_cast<uint32_t>(nseg);
    h[3] = 0u;
}

// Plan pass, one workgroup: per segment its entries (clamped as above), its
// tiles and, with E = entries, its block's offset; the tile -> segment table;
// when the stream fits out_cap, every header; always the stream length and
// the flags the later passes read.
__global__ __launch_bounds__(kBlock) void pack_plan_kernel(PlanDev P, int kind, uint64_t cap,
                                                           const uint32_t *__restrict__ seg_off,
                                                           const float *__restrict__ seg_scale,
                                                           uint8_t *__restrict__ out, uint64_t out_cap,
                                                           uint64_t *__restrict__ out_bytes, PackWs w) {
    const bool dgc = kind == GC_KIND_DGC;
    __shared__ uint32_t tstart[kBlock + 1];
    uint64_t byte_run = blocks_start(P.nseg);
    uint32_t tile_run = 0;
    for (int r = 0; r < P.nseg; r += kBlock) {
        const int s = r + int(threadIdx.x);
        uint32_t cnt = 0, first = 0;
        if (s < P.nseg) {
            cnt = seg_entries(seg_off, s, seg_max_entries(P.seg[s], kind), cap);
            first = seg_off[s];
        }
        const uint32_t nt = (cnt + kTile - 1) / kTile;
        uint64_t btot;
        uint32_t ttot;
        const uint64_t bpre = block_exclusive_scan<uint64_t>(block_bytes(cnt, dgc) * (s < P.nseg), &btot);
        const uint32_t tpre = block_exclusive_scan<uint32_t>(nt, &ttot);
        if (s < P.nseg) {
            w.srec[s] = make_uint4(first, cnt, cnt, tile_run + tpre);
            w.blk_off[s] = byte_run + bpre;
        }
        // the tile -> segment table of these segments' ttot tiles: thread t
        // fills an equal share, from the segment of its first tile on
        tstart[threadIdx.x] = tpre;
        if (threadIdx.x == 0) tstart[kBlock] = ttot;
        __syncthreads();
        const uint32_t per = (ttot + kBlock - 1) / kBlock;
        const uint32_t q0 = threadIdx.x * per, q1 = min(q0 + per, ttot);
        if (q0 < q1) {
            int lo = 0, hi = kBlock - 1;  // the last segment starting at or before q0
            while (lo < hi) {
                const int mid = (lo + hi + 1) / 2;
                if (tstart[mid] <= q0) lo = mid;
                else hi = mid - 1;
            }
            for (uint32_t q = q0; q < q1; ++q) {
                while (tstart[lo + 1] <= q) ++lo;
                w.tile_seg[tile_run + q] = static_cast<uint32_t>(r + lo);
            }
        }
        __syncthreads();
        byte_run += btot;
        tile_run += ttot;
    }
    const bool fits = byte_run <= out_cap;
    if (fits) {
        for (int s = threadIdx.x; s < P.nseg; s += kBlock) {
            const uint32_t cnt = seg_entries(seg_off, s, seg_max_entries(P.seg[s], kind), cap);
            // the block offset again, from this thread's own write above
            write_block_header(out, w.blk_off[s], dgc, P.seg[s].len, cnt, cnt, dgc ? 0.0f : seg_scale[s]);
            write_table_entry(out, s, w.blk_off[s], cnt, cnt);
        }
    }
    if (threadIdx.x == 0) {
        if (fits) write_stream_header(out, kind, P.nseg);
        *out_bytes = byte_run;
        w.flags[0] = tile_run;
        w.flags[1] = fits ? 0u : 1u;
        w.flags[2] = 0u;
    }
}

// Relayout, by one workgroup, when some tile has escapes: each segment's
// escapes (the sum over its tiles), blocks resized, headers, stream length
// and overflow written again.
__device__ void pack_relayout(const PlanDev &P, int kind, uint32_t MAX, const float *__restrict__ seg_scale,
                              uint8_t *__restrict__ out, uint64_t out_cap, uint64_t *__restrict__ out_bytes,
                              const PackWs &w) {
    const bool dgc = kind == GC_KIND_DGC;
    const uint32_t ntiles = w.flags[0];
    uint64_t byte_run = blocks_start(P.nseg);
    for (int r = 0; r < P.nseg; r += kBlock) {
        const int s = r + int(threadIdx.x);
        uint64_t sz = 0;
        if (s < P.nseg) {
            const uint4 sr = w.srec[s];
            const uint32_t t1 = s + 1 < P.nseg ? w.srec[s + 1].w : ntiles;
            uint64_t esc = 0;
            for (uint32_t u = sr.w; u < t1; ++u) esc += w.tile_esc[u];
            // never more codes than a segment of this length can need
            const uint64_t cap_e = uint64_t(P.seg[s].len) + P.seg[s].len / MAX + 1;
            const uint64_t e64 = uint64_t(sr.y) + esc;
            const uint32_t E = static_cast<uint32_t>(e64 < cap_e ? e64 : cap_e);
            w.srec[s].z = E;
            sz = block_bytes(E, dgc);
        }
        uint64_t tot;
        const uint64_t pre = block_exclusive_scan<uint64_t>(sz, &tot);
        if (s < P.nseg) w.blk_off[s] = byte_run + pre;
        byte_run += tot;
    }
    const bool fits = byte_run <= out_cap;
    if (fits)
        for (int s = threadIdx.x; s < P.nseg; s += kBlock) {
            const uint4 sr = w.srec[s];
            write_block_header(out, w.blk_off[s], dgc, P.seg[s].len, sr.z, sr.y, dgc ? 0.0f : seg_scale[s]);
            write_table_entry(out, s, w.blk_off[s], sr.z, sr.y);
        }
    if (threadIdx.x == 0) {
        *out_bytes = byte_run;
        w.flags[1] = fits ? 0u : 1u;
    }
}

// A wave-uniform value moved to a scalar register (the tile geometry is read
// with vector loads; every lane holds the same value).
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

constexpr uint32_t kPerThread = kTile / kBlock;

// Sum over the workgroup of one value per thread, in every thread.
__device__ __forceinline__ uint32_t block_total(uint32_t v) {
    __shared__ uint32_t wsum[kWaves];
    const uint32_t x = wave_total(v);
    if (lane_id() == 0) wsum[wave_id()] = x;
    __syncthreads();
    uint32_t all = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) all += wsum[i];
    return all;
}

// Tile t of segment s: entries [j0, j0 + cnt) of the message, the segment's
// tiles starting at tile0, its block of E codes at byte boff.
struct TileGeom {
    EntryCtx x;
    uint32_t E, j0, cnt, tile0;
    uint64_t boff;
};

// The tile's loads in the lane-strided layout (entry i * kBlock + t of the
// tile in thread t) and each entry's gap.  An entry's predecessor is the one
// in the lane before (a wave shift); lane 0 loads its own, from the entry
// before the tile unless the tile is the segment's first (where entry 0's
// predecessor is unused).  Buffer resources cover the tile: loads past it
// return 0.
__device__ __forceinline__ void tile_load(const TileGeom &g, const uint32_t *__restrict__ idx,
                                          const float *__restrict__ val, uint32_t (&gap)[kPerThread],
                                          float (&v)[kPerThread], uint32_t &cur0) {
    const uint32_t d = uni(g.j0 > g.x.first ? 1u : 0u);
    const BufRsrc ri = chunk_buf(reinterpret_cast<const float *>(idx + g.j0), g.cnt);
    const BufRsrc rp = chunk_buf(reinterpret_cast<const float *>(idx + g.j0 - d), g.cnt + d);
    const BufRsrc rv = chunk_buf(val + g.j0, g.cnt);
    uint32_t cur[kPerThread], p0[kPerThread];
    // lane 0 loads its predecessor (entry e - 1, at e + d - 1 in rp); the
    // other lanes, and the tile's first entry when it has none, load past the
    // resource's range (no memory access, 0) and take it from the lane before
    const bool lane0 = lane_id() == 0;
#pragma unroll
    for (uint32_t i = 0; i < kPerThread; ++i) {
        const uint32_t e = i * kBlock + threadIdx.x;
        const int vo = static_cast<int>(4 * threadIdx.x), so = static_cast<int>(4 * i * kBlock);
        cur[i] = __builtin_amdgcn_raw_buffer_load_b32(ri, vo, so, kKeep);
        v[i] = dev_u2f(__builtin_amdgcn_raw_buffer_load_b32(rv, vo, so, kKeep));
        const int po = lane0 && e + d > 0 ? static_cast<int>(4 * (e + d - 1)) : 0x7FFFFFF0;
        p0[i] = __builtin_amdgcn_raw_buffer_load_b32(rp, po, 0, kKeep);
    }
#pragma unroll
    for (uint32_t i = 0; i < kPerThread; ++i) {
        const uint32_t e = i * kBlock + threadIdx.x;
        // lane l takes lane l - 1's entry; lane 0 keeps its loaded one
        const uint32_t prv = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(static_cast<int>(p0[i]), static_cast<int>(cur[i]), kDppWaveShr1, 0xF, 0xF, false));
        gap[i] = e < g.cnt ? entry_gap(g.x, g.j0 + e, cur[i], prv) : 0u;
    }
    cur0 = cur[0];
}

// One code (and DGC value) at its slot of the block.  The packed stream is
// not read again here: non-temporal stores.
__device__ __forceinline__ void put_code(bool dgc, uint16_t *runs, float *vals, uint32_t slot, uint32_t gap,
                                         float value) {
    if (dgc) {
        __builtin_nontemporal_store(static_cast<uint16_t>(gap), runs + slot);
        __builtin_nontemporal_store(value, vals + slot);
    } else {
        const uint16_t sign = (dev_f2u(value) >> 31) ? 0x8000u : 0u;
        __builtin_nontemporal_store(static_cast<uint16_t>(sign | gap), runs + slot);
    }
}

__device__ __forceinline__ uint16_t *block_runs(uint8_t *out, const TileGeom &g) {
    return reinterpret_cast<uint16_t *>(out + g.boff + 16);
}
__device__ __forceinline__ float *block_vals(uint8_t *out, const TileGeom &g) {
    return reinterpret_cast<float *>(out + g.boff + 16 + 2ull * g.E + 2ull * (g.E & 1u));
}
// The block's checkpoints: (entries, reader position) before code kCkpt c.
__device__ __forceinline__ uint32_t *block_ckpt(uint8_t *out, const TileGeom &g, bool dgc) {
    return reinterpret_cast<uint32_t *>(out + g.boff + 16 + 2ull * g.E + 2ull * (g.E & 1u) + (dgc ? 4ull * g.E : 0));
}
__device__ __forceinline__ void put_ckpt(uint32_t *ck, uint32_t code, uint32_t entries, uint32_t pos) {
    ck[2 * (code / kCkpt)] = entries;
    ck[2 * (code / kCkpt) + 1] = pos;
}

// First pass over a tile: its escapes to tile_esc[t]; a tile without any is
// written at slot = rank in the segment.  Returns the tile's escapes.
template <bool kDgc>
__device__ __forceinline__ uint32_t tile_write(const TileGeom &g, uint32_t t, const uint32_t *__restrict__ idx,
                                               const float *__restrict__ val, uint8_t *__restrict__ out,
                                               const PackWs &w) {
    constexpr bool dgc = kDgc;
    constexpr uint32_t MAX = kDgc ? 65535u : 32767u;
    uint32_t gap[kPerThread], cur0;
    float v[kPerThread];
    tile_load(g, idx, val, gap, v, cur0);
    uint32_t mine = 0;
#pragma unroll
    for (uint32_t i = 0; i < kPerThread; ++i) mine += gap[i] / MAX;
    const uint32_t esc = block_total(mine);
    if (threadIdx.x == 0) {
        w.tile_esc[t] = esc;
        w.tile_any[t] = esc ? 1u : 0u;
    }
    if (esc) return esc;  // written by the rewrite pass
    // buffer resources over the tile's codes and values in the block (slots
    // j0 - first .. + cnt, inside the block's E): stores past them are dropped
    const uint32_t slot0 = g.j0 - g.x.first;
    const uint32_t room = slot0 < g.E ? min(g.cnt, g.E - slot0) : 0u;  // below cnt only for malformed messages
    const BufRsrc rr = __builtin_amdgcn_make_buffer_rsrc(block_runs(out, g) + slot0, static_cast<short>(0),
                                                         static_cast<int>(2 * room), kBufWord3);
    const BufRsrc rv = chunk_buf(block_vals(out, g) + slot0, dgc ? room : 0u);
#pragma unroll
    for (uint32_t i = 0; i < kPerThread; ++i) {
        const int vo = static_cast<int>(threadIdx.x), so = static_cast<int>(i * kBlock);
        if (dgc) {
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(gap[i]), rr, 2 * vo, 2 * so, kBufNT);
            __builtin_amdgcn_raw_buffer_store_b32(dev_f2u(v[i]), rv, 4 * vo, 4 * so, kBufNT);
        } else {
            const uint16_t sign = (dev_f2u(v[i]) >> 31) ? 0x8000u : 0u;
            __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(sign | gap[i]), rr, 2 * vo, 2 * so, kBufNT);
        }
    }
    // without escapes code c of the block is entry c: the tile's first entry
    // starts checkpoint t - tile0, with the reader standing at its position
    // minus its run
    if (threadIdx.x == 0 && g.j0 - g.x.first < g.E)
        put_ckpt(block_ckpt(out, g, dgc), g.j0 - g.x.first, g.j0 - g.x.first, (cur0 - g.x.off) - gap[0]);
    return 0;
}

// Rewrite pass over a tile, after the relayout: a tile without escapes at
// rank + the escapes of the segment's earlier tiles; a tile with escapes
// walks 16 contiguous entries per thread in two light passes (escapes, then
// slots), reloading what it needs, so that its registers do not add to the
// common path's.
template <bool kDgc>
__device__ __forceinline__ void tile_rewrite(const TileGeom &g, uint32_t t, const uint32_t *__restrict__ idx,
                                             const float *__restrict__ val, uint8_t *__restrict__ out,
                                             const PackWs &w) {
    constexpr bool dgc = kDgc;
    constexpr uint32_t MAX = kDgc ? 65535u : 32767u;
    uint32_t part = 0;
#pragma unroll 4
    for (uint32_t u = g.tile0 + threadIdx.x; u < t; u += kBlock) part += w.tile_esc[u];
    const uint32_t esc_base = block_total(part);
    uint16_t *runs = block_runs(out, g);
    float *vals = block_vals(out, g);
    uint32_t *ck = block_ckpt(out, g, dgc);
    if (uni(w.tile_esc[t]) == 0) {
        uint32_t gap[kPerThread], cur0;
        float v[kPerThread];
        tile_load(g, idx, val, gap, v, cur0);
#pragma unroll
        for (uint32_t i = 0; i < kPerThread; ++i) {
            const uint32_t e = i * kBlock + threadIdx.x;
            const uint32_t slot = (g.j0 + e - g.x.first) + esc_base;
            if (e < g.cnt && slot < g.E) {
                put_code(dgc, runs, vals, slot, gap[i], v[i]);
                // an entry of a tile without escapes: the code before it is
                // the previous entry's, so the reader stands at its position
                // minus its run
                if (slot % kCkpt == 0) put_ckpt(ck, slot, g.j0 + e - g.x.first, (idx[g.j0 + e] - g.x.off) - gap[i]);
            }
        }
        return;
    }
    const uint32_t e0 = threadIdx.x * kPerThread;
    auto gap_at = [&](uint32_t e) {
        const uint32_t j = g.j0 + e;
        return entry_gap(g.x, j, idx[j], idx[j > g.x.first ? j - 1 : j]);
    };
    uint32_t own = 0;
#pragma unroll 1
    for (uint32_t e = e0; e < min(e0 + kPerThread, g.cnt); ++e) own += gap_at(e) / MAX;
    uint32_t tot;
    uint32_t before = esc_base + block_exclusive_scan(own, &tot);
#pragma unroll 1
    for (uint32_t e = e0; e < min(e0 + kPerThread, g.cnt); ++e) {
        uint32_t slot = (g.j0 + e - g.x.first) + before;
        uint32_t gp = gap_at(e);
        const uint32_t esc = gp / MAX;
        const uint32_t rank = g.j0 + e - g.x.first;     // entries before this one in the segment
        uint32_t pos = (idx[g.j0 + e] - g.x.off) - gp;  // the reader's position before its first code
        for (uint32_t z = 0; z < esc && slot < g.E; ++z) {
            if (slot % kCkpt == 0) put_ckpt(ck, slot, rank, pos);
            runs[slot] = static_cast<uint16_t>(MAX);
            if (dgc) vals[slot] = 0.0f;
            ++slot;
            gp -= MAX;
            pos += MAX;
        }
        before += esc;
        if (slot >= g.E) continue;  // only for malformed messages
        if (slot % kCkpt == 0) put_ckpt(ck, slot, rank, pos);
        put_code(dgc, runs, vals, slot, gp, val[g.j0 + e]);
    }
}

// ------------------------------------------------- plans of many segments
// Geometry of tile t from the plan pass's tables.
__device__ __forceinline__ TileGeom table_tile(const PlanDev &P, const PackWs &w, uint32_t t) {
    const uint32_t s = uni(w.tile_seg[t]);
    const uint4 sr = w.srec[s];
    const SegDev sg = P.seg[s];
    TileGeom g;
    g.x.first = uni(sr.x);
    g.x.off = static_cast<uint32_t>(sg.off);
    g.x.len = sg.len;
    g.E = uni(sr.z);
    g.tile0 = uni(sr.w);
    g.j0 = g.x.first + (t - g.tile0) * kTile;
    g.cnt = uni(min(sr.y - (t - g.tile0) * kTile, kTile));
    g.boff = w.blk_off[s];
    return g;
}

// Write pass (kRedo false) and rewrite pass (kRedo true) after the plan pass.
template <bool kRedo, bool kDgc>
__global__ __launch_bounds__(kBlock) void pack_write_kernel(PlanDev P, const uint32_t *__restrict__ idx,
                                                            const float *__restrict__ val, uint8_t *__restrict__ out,
                                                            PackWs w) {
    if (w.flags[1]) return;  // the stream does not fit out_cap: nothing is written
    if (kRedo && !w.flags[2]) return;
    const uint32_t ntiles = uni(w.flags[0]);
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const TileGeom g = table_tile(P, w, t);
        if (kRedo) {
            tile_rewrite<kDgc>(g, t, idx, val, out, w);
        } else if (tile_write<kDgc>(g, t, idx, val, out, w) && threadIdx.x == 0) {
            atomicOr(&w.flags[2], 1u);
        }
        __syncthreads();
    }
}

// Relayout pass, one workgroup, only when some tile has escapes.  (Having
// the last write workgroup do it instead cost each of them a device-scope
// fence and an atomic on one counter: the write pass ran 10x slower.)
__global__ __launch_bounds__(kBlock) void pack_relayout_kernel(PlanDev P, int kind, uint32_t MAX,
                                                               const float *__restrict__ seg_scale,
                                                               uint8_t *__restrict__ out, uint64_t out_cap,
                                                               uint64_t *__restrict__ out_bytes, PackWs w) {
    if (w.flags[1] || !w.flags[2]) return;
    pack_relayout(P, kind, MAX, seg_scale, out, out_cap, out_bytes, w);
}

// ------------------------------------------------- plans of few segments
// Every workgroup lays the stream out itself (escape-free) from the message
// counts, in LDS, so that no plan pass runs before the write.
constexpr int kFuseSegs = 512;

struct FuseLds {
    uint32_t first[kFuseSegs], cnt[kFuseSegs], off[kFuseSegs], len[kFuseSegs];
    uint32_t tile0[kFuseSegs + 1];
    uint64_t boff[kFuseSegs];
    uint32_t cur;  // segment of the current tile
};

// Per segment its first entry, entries (clamped as in the plan pass),
// offset, length, first tile and block offset; returns the stream length,
// and the tile count in *ntiles.
__device__ uint64_t fused_layout(const PlanDev &P, bool dgc, uint64_t cap, const uint32_t *__restrict__ seg_off,
                                 FuseLds &L, uint32_t *ntiles) {
    uint64_t byte_run = blocks_start(P.nseg);
    uint32_t tile_run = 0;
    for (int r = 0; r < P.nseg; r += kBlock) {
        const int s = r + int(threadIdx.x);
        uint32_t cnt = 0;
        if (s < P.nseg) {
            const uint32_t len = P.seg[s].len;
            cnt = seg_entries(seg_off, s, len, cap);
            L.first[s] = seg_off[s];
            L.cnt[s] = cnt;
            L.off[s] = static_cast<uint32_t>(P.seg[s].off);
            L.len[s] = len;
        }
        uint64_t btot;
        uint32_t ttot;
        const uint64_t bpre = block_exclusive_scan<uint64_t>(block_bytes(cnt, dgc) * (s < P.nseg), &btot);
        const uint32_t tpre = block_exclusive_scan<uint32_t>((cnt + kTile - 1) / kTile, &ttot);
        if (s < P.nseg) {
            L.tile0[s] = tile_run + tpre;
            L.boff[s] = byte_run + bpre;
        }
        byte_run += btot;
        tile_run += ttot;
    }
    if (threadIdx.x == 0) L.tile0[P.nseg] = tile_run;
    __syncthreads();
    *ntiles = tile_run;
    return byte_run;
}

// Geometry of tile t: the segment whose tile range holds it (exactly one).
__device__ __forceinline__ TileGeom fused_tile(const PlanDev &P, FuseLds &L, uint32_t t, const uint32_t *E) {
    for (int s = threadIdx.x; s < P.nseg; s += kBlock)
        if (L.tile0[s] <= t && t < L.tile0[s + 1]) L.cur = static_cast<uint32_t>(s);
    __syncthreads();
    const uint32_t s = uni(L.cur);
    TileGeom g;
    g.x.first = uni(L.first[s]);
    g.x.off = uni(L.off[s]);
    g.x.len = uni(L.len[s]);
    g.E = uni(E ? E[s] : L.cnt[s]);
    g.tile0 = uni(L.tile0[s]);
    g.j0 = g.x.first + (t - g.tile0) * kTile;
    g.cnt = uni(min(L.cnt[s] - (t - g.tile0) * kTile, kTile));
    g.boff = L.boff[s];
    return g;
}

// Main pass: layout, then every tile as in the write pass.  Workgroup 0
// writes the headers, the stream length, the tile count (flags[0]) and
// whether the stream does not fit (flags[1]); every tile writes its escape
// count, so nothing has to be cleared before the pass.
template <bool kDgc>
__global__ __launch_bounds__(kBlock) void pack_main_kernel(PlanDev P, uint64_t cap, const uint32_t *__restrict__ seg_off,
                                                           const float *__restrict__ seg_scale,
                                                           const uint32_t *__restrict__ idx,
                                                           const float *__restrict__ val, uint8_t *__restrict__ out,
                                                           uint64_t out_cap, uint64_t *__restrict__ out_bytes,
                                                           PackWs w) {
    constexpr bool dgc = kDgc;
    constexpr int kind = kDgc ? GC_KIND_DGC : GC_KIND_ADACOMP;
    __shared__ FuseLds L;
    uint32_t ntiles;
    const uint64_t bytes = fused_layout(P, dgc, cap, seg_off, L, &ntiles);
    const bool fits = bytes <= out_cap;
    if (blockIdx.x == 0) {
        if (fits)
            for (int s = threadIdx.x; s < P.nseg; s += kBlock) {
                write_block_header(out, L.boff[s], dgc, L.len[s], L.cnt[s], L.cnt[s], dgc ? 0.0f : seg_scale[s]);
                write_table_entry(out, s, L.boff[s], L.cnt[s], L.cnt[s]);
            }
        if (threadIdx.x == 0) {
            if (fits) write_stream_header(out, kind, P.nseg);
            *out_bytes = bytes;
            w.flags[0] = ntiles;
            w.flags[1] = fits ? 0u : 1u;
        }
    }
    if (!fits) return;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const TileGeom g = fused_tile(P, L, t, nullptr);
        (void)tile_write<kDgc>(g, t, idx, val, out, w);
        __syncthreads();
    }
}

// Fix pass: returns unless some tile has escapes (each workgroup reads the
// tile counts).  Otherwise every workgroup lays the stream out again with
// each segment's escapes (the relayout of the plan path), workgroup 0
// rewrites the headers and the length, and the tiles are written again.
template <bool kDgc>
__global__ __launch_bounds__(kBlock) void pack_fix_kernel(PlanDev P, uint64_t cap, const uint32_t *__restrict__ seg_off,
                                                          const float *__restrict__ seg_scale,
                                                          const uint32_t *__restrict__ idx,
                                                          const float *__restrict__ val, uint8_t *__restrict__ out,
                                                          uint64_t out_cap, uint64_t *__restrict__ out_bytes,
                                                          PackWs w) {
    constexpr bool dgc = kDgc;
    constexpr uint32_t MAX = kDgc ? 65535u : 32767u;
    // the tiles' escape bytes (sixteen per load, over the workspace's whole
    // table) in the same round of loads as the tile count; bytes past the
    // count are not this call's
    const uint32_t ntiles = uni(w.flags[0]);
    const uint32_t nofit = w.flags[1];
    const uint4 *ta = reinterpret_cast<const uint4 *>(w.tile_any);  // 256-byte aligned region
    const uint32_t n16 = static_cast<uint32_t>((w.max_tiles + 15) / 16);
    uint32_t any = 0;
    for (uint32_t q0 = threadIdx.x; q0 < n16; q0 += 8 * kBlock) {
        uint4 x[8];
#pragma unroll
        for (uint32_t q = 0; q < 8; ++q) {
            const uint32_t i = q0 + q * kBlock;
            x[q] = i < n16 ? ta[i] : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (uint32_t q = 0; q < 8; ++q) {
            const uint32_t b = 16 * (q0 + q * kBlock);
            const uint32_t word[4] = {x[q].x, x[q].y, x[q].z, x[q].w};
#pragma unroll
            for (uint32_t k = 0; k < 4; ++k) {
                const uint32_t b0 = b + 4 * k;  // bytes [b0, b0 + 4) of the table
                const uint32_t keep = b0 + 4 <= ntiles ? 0xFFFFFFFFu
                                      : b0 >= ntiles   ? 0u
                                                       : (1u << (8 * (ntiles - b0))) - 1u;
                any |= word[k] & keep;
            }
        }
    }
    if (nofit) return;
    if (!__syncthreads_or(any != 0u)) return;
    __shared__ FuseLds L;
    __shared__ uint32_t esc[kFuseSegs];
    uint32_t nt2;
    (void)fused_layout(P, dgc, cap, seg_off, L, &nt2);  // the main pass's layout: nt2 == ntiles
    for (int s = threadIdx.x; s < P.nseg; s += kBlock) esc[s] = 0u;
    __syncthreads();
    for (uint32_t t = threadIdx.x; t < ntiles; t += kBlock) {
        const uint32_t e = w.tile_esc[t];
        if (!e) continue;
        int lo = 0, hi = P.nseg - 1;  // the last segment whose tiles start at or before t
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (L.tile0[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        atomicAdd(&esc[lo], e);
    }
    __syncthreads();
    uint64_t byte_run = blocks_start(P.nseg);
    for (int r = 0; r < P.nseg; r += kBlock) {
        const int s = r + int(threadIdx.x);
        uint64_t sz = 0;
        if (s < P.nseg) {
            // never more codes than a segment of this length can need
            const uint64_t cap_e = uint64_t(L.len[s]) + L.len[s] / MAX + 1;
            const uint64_t e64 = uint64_t(L.cnt[s]) + esc[s];
            const uint32_t E = static_cast<uint32_t>(e64 < cap_e ? e64 : cap_e);
            esc[s] = E;  // from here on: the block's codes
            sz = block_bytes(E, dgc);
        }
        uint64_t tot;
        const uint64_t pre = block_exclusive_scan<uint64_t>(sz, &tot);
        if (s < P.nseg) L.boff[s] = byte_run + pre;
        byte_run += tot;
    }
    __syncthreads();
    const bool fits = byte_run <= out_cap;
    if (blockIdx.x == 0) {
        if (fits)
            for (int s = threadIdx.x; s < P.nseg; s += kBlock) {
                write_block_header(out, L.boff[s], dgc, L.len[s], esc[s], L.cnt[s], dgc ? 0.0f : seg_scale[s]);
                write_table_entry(out, s, L.boff[s], esc[s], L.cnt[s]);
            }
        if (threadIdx.x == 0) *out_bytes = byte_run;
    }
    if (!fits) return;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const TileGeom g = fused_tile(P, L, t, esc);
        tile_rewrite<kDgc>(g, t, idx, val, out, w);
        __syncthreads();
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
    for (const auto &s : plan->seg) {
        const uint64_t codes = entries(s) + s.len / MAX + 1;  // at most
        b += 16 + 16 + 2 + per * codes + 8 * ceil_div(codes, kCkpt);  // table entry, header, pad, codes, checkpoints
    }
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

template <bool kDgc>
static gc_status pack_launch(const gc_plan *plan, const PlanDev &P, const gc_sparse *in, uint8_t *out,
                             uint64_t out_cap, uint64_t *out_bytes, const PackWs &w, uint32_t MAX, unsigned grid,
                             hipStream_t stream) {
    constexpr int kind = kDgc ? GC_KIND_DGC : GC_KIND_ADACOMP;
    const uint64_t cap = in->cap;
    if (plan->nseg <= kFuseSegs) {
        // few segments: every workgroup lays the stream out itself; the fix
        // pass only reads the tile counts unless a tile has escapes.  The
        // main pass keeps its workgroups resident: each lays the stream out
        // once, then loops over tiles.
        grid = std::min(grid, resident_blocks(reinterpret_cast<const void *>(pack_main_kernel<kDgc>)));
        const unsigned fgrid = static_cast<unsigned>(std::min<size_t>(w.max_tiles, 256));
        GC_LAUNCH("pack_main", stream, pack_main_kernel<kDgc><<<grid, kBlock, 0, stream>>>(P, cap, in->seg_off, in->seg_scale,
                                                                                           in->idx, in->val, out, out_cap,
                                                                                           out_bytes, w));
        GC_LAUNCH("pack_fix", stream, pack_fix_kernel<kDgc><<<fgrid, kBlock, 0, stream>>>(P, cap, in->seg_off, in->seg_scale,
                                                                                          in->idx, in->val, out, out_cap,
                                                                                          out_bytes, w));
    } else {
        GC_LAUNCH("pack_plan", stream, pack_plan_kernel<<<1, kBlock, 0, stream>>>(P, kind, cap, in->seg_off, in->seg_scale, out,
                                                                                 out_cap, out_bytes, w));
        GC_LAUNCH("pack_write", stream, pack_write_kernel<false, kDgc><<<grid, kBlock, 0, stream>>>(P, in->idx, in->val, out, w));
        GC_LAUNCH("pack_relayout", stream, pack_relayout_kernel<<<1, kBlock, 0, stream>>>(P, kind, MAX, in->seg_scale, out, out_cap,
                                                                                         out_bytes, w));
        GC_LAUNCH("pack_rewrite", stream, pack_write_kernel<true, kDgc><<<grid, kBlock, 0, stream>>>(P, in->idx, in->val, out, w));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_pack launch");
    return GC_OK;
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
    // One tile per workgroup up to kTileGrid tiles (each tile is a chain of
    // dependent loads, so tiles run side by side rather than in sequence);
    // workgroups past the actual tile count exit at once.  A DGC message
    // normally holds the plan's k per segment: its grid follows those tiles
    // (with room for denser messages, whose extra tiles the workgroups loop
    // over), not the capacity.
    constexpr size_t kTileGrid = 8192;
    size_t want = w.max_tiles;
    if (kind == GC_KIND_DGC) {
        size_t ktiles = 0;
        for (const auto &s : plan->seg) ktiles += ceil_div(s.k, kTile);
        want = std::max<size_t>(2 * ktiles, 256);
    }
    const unsigned grid = static_cast<unsigned>(std::min({w.max_tiles, want, kTileGrid}));
    if (kind == GC_KIND_DGC) return pack_launch<true>(plan, P, in, out, out_cap, out_bytes, w, MAX, grid, stream);
    return pack_launch<false>(plan, P, in, out, out_cap, out_bytes, w, MAX, grid, stream);
}

