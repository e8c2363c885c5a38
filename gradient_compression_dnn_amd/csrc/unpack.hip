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

// A wave-uniform value moved to scalar registers.
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uni64(uint64_t v) {
    return uint64_t(uni(static_cast<uint32_t>(v))) | uint64_t(uni(static_cast<uint32_t>(v >> 32))) << 32;
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

// One workgroup.  One pass checks every block, that each lies where the
// blocks before it end, and lays out the tiles and slots as the table gives
// them; when anything failed, a second pass lays out every block as empty.
// Then the message's segment offsets (clamped to cap) and scales.
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
    uint32_t over = 0;  // kOverCap, kept apart from st: st alone decides the second pass
    for (int pass = 0; pass < 2; ++pass) {
        if (pass == 1 && !st) break;  // the layout of the first pass stands (st is the same in every thread)
        uint64_t at = head, slot_run = 0;
        uint32_t tile_run = 0, bad = 0;
        for (int r = 0; r < P.nseg; r += kBlock) {
            const int s = r + int(threadIdx.x);
            BlockView b{};
            if (s < P.nseg && !st) {
                b = view_block(P, dgc, MAX, bmagic, in, nbytes, s);
                if (!b.ok) {
                    bad = 1u;
                    b.E = b.cnt = 0;  // a bad block's size is unknown: the stream fails anyway
                }
            }
            uint64_t btot, ctot;
            uint32_t ttot;
            const uint64_t bpre = block_exclusive_scan<uint64_t>(st ? 0 : block_bytes(b.E, dgc) * (s < P.nseg), &btot);
            const uint64_t cpre = block_exclusive_scan<uint64_t>(b.cnt, &ctot);
            const uint32_t tpre = block_exclusive_scan<uint32_t>((b.E + kUTile - 1) / kUTile, &ttot);
            if (s < P.nseg) {
                if (!st && b.off != at + bpre) bad = 1u;
                w.blk_off[s] = b.off;
                w.seg_E[s] = b.E;
                w.seg_cnt[s] = b.cnt;
                w.tile_base[s] = tile_run + tpre;
                const uint64_t sb = slot_run + cpre;
                w.slot_base[s] = static_cast<uint32_t>(umin64(sb, 0xFFFFFFFFull));
                seg_off[s] = static_cast<uint32_t>(umin64(sb, cap));
                if (seg_scale) seg_scale[s] = dgc || st ? 0.0f : dev_u2f(b.w3);
            }
            at += btot;
            slot_run += ctot;
            tile_run += ttot;
        }
        if (!st && (__syncthreads_or(bad != 0u) || at != nbytes)) st = kBadBlock;
        over = !st && slot_run > cap ? kOverCap : 0u;
        if (threadIdx.x == 0) {
            w.tile_base[P.nseg] = tile_run;
            w.slot_base[P.nseg] = static_cast<uint32_t>(umin64(slot_run, 0xFFFFFFFFull));
            seg_off[P.nseg] = static_cast<uint32_t>(umin64(slot_run, cap));
        }
    }
    if (threadIdx.x == 0) *status = st | over;
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

// Code i * kBlock + t of the tile is thread t's i-th: loads and the entries'
// stores are coalesced along a row.  One pass of row-order scans gives every
// code the steps and entries before it in the tile (one wave scan per row of
// both packed in a u32, then one wave scans the kUPer * kWaves (row, wave)
// totals of each), and so its position and slot from the tile's checkpoint.
// The steps and entry flags are derived from the codes where needed rather
// than kept, so that a thread holds two values per code (one more for DGC's
// values).
template <bool kDgc>
__global__ __launch_bounds__(kBlock) void unpack_write_kernel(PlanDev P, const uint8_t *__restrict__ in,
                                                              UnpackWs w, uint64_t cap,
                                                              const float *__restrict__ seg_scale,
                                                              uint32_t *__restrict__ out_idx,
                                                              float *__restrict__ out_val, uint32_t *status) {
    static_assert(kUPer * kWaves <= kWave, "one wave scans the row totals");
    const uint32_t ntiles = w.tile_base[P.nseg];
    if (blockIdx.x >= ntiles) return;
    constexpr uint32_t MAX = kDgc ? 65535u : 32767u;
    constexpr uint32_t rmask = kDgc ? 0xFFFFu : 0x7FFFu;
    __shared__ uint32_t lds[kLdsSegs];
    __shared__ uint32_t tot_s[kUPer * kWaves + 1], tot_e[kUPer * kWaves + 1];
    TileOf table;
    table.init(w.tile_base, P.nseg, lds);
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        // every value of the tile's geometry is the workgroup's: scalar registers
        const uint32_t s = uni(table.segment(t));
        const uint32_t seg_len = uni(P.seg[s].len);
        const uint64_t seg_off0 = uni64(P.seg[s].off);
        const uint32_t E = uni(w.seg_E[s]), cnt = uni(w.seg_cnt[s]);
        const uint32_t c = t - uni(w.tile_base[s]);
        const uint32_t j0 = c * kUTile;
        const uint32_t nck = (E + kUTile - 1) / kUTile;
        const uint32_t sbase = uni(w.slot_base[s]);
        const uint8_t *blk = in + uni64(w.blk_off[s]);
        const uint16_t *runs = reinterpret_cast<const uint16_t *>(blk + 16);
        const float *vals = reinterpret_cast<const float *>(blk + 16 + 2ull * E + 2ull * (E & 1u));
        const uint32_t *ck = reinterpret_cast<const uint32_t *>(blk + 16 + 2ull * E + 2ull * (E & 1u) + (kDgc ? 4ull * E : 0));
        const float scale = kDgc ? 0.0f : dev_u2f(uni(dev_f2u(seg_scale[s])));
        // the tile's start and, unless it is the block's last, the next tile's
        const uint32_t e0 = uni(ck[2 * c]), p0 = uni(ck[2 * c + 1]);
        const bool last = c + 1 >= nck;
        const uint32_t e1 = last ? cnt : uni(ck[2 * c + 2]), p1 = last ? 0u : uni(ck[2 * c + 3]);
        // buffer resources over the tile's codes and values: loads past the
        // block's last code return 0 (and are never used)
        const uint32_t ntile = min(E - j0, kUTile);
        const BufRsrc rr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(runs + j0), static_cast<short>(0),
                                                             static_cast<int>(2 * ntile), kBufWord3);
        uint32_t code[kUPer];
        float v[kDgc ? kUPer : 1];
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i)
            code[i] = __builtin_amdgcn_raw_buffer_load_b16(rr, static_cast<int>(2 * threadIdx.x),
                                                           static_cast<int>(2 * i * kBlock), 0);
        if (kDgc) {  // an AdaComp block has no value array
            const BufRsrc rv = chunk_buf(vals + j0, ntile);
#pragma unroll
            for (uint32_t i = 0; i < kUPer; ++i)
                v[kDgc ? i : 0] = dev_u2f(__builtin_amdgcn_raw_buffer_load_b32(rv, static_cast<int>(4 * threadIdx.x),
                                                                                static_cast<int>(4 * i * kBlock), 0));
        }
        auto in_tile = [&](uint32_t i) { return j0 + i * kBlock + threadIdx.x < E; };
        auto step_of = [&](uint32_t i) {
            const uint32_t r = code[i] & rmask;
            return !in_tile(i) ? 0u : (r == MAX ? MAX : r + 1);
        };
        auto ent_of = [&](uint32_t i) { return in_tile(i) && (code[i] & rmask) != MAX ? 1u : 0u; };
        // a row of one wave holds at most 64 entries (8 bits) and 64 * 65535
        // steps (22 bits): one scan of (steps << 8 | entries) gives both
        uint32_t pre[kUPer], rowtot[kUPer];
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i) {
            const uint32_t x = step_of(i) << 8 | ent_of(i);
            const uint32_t xi = wave_inclusive_scan(x);
            pre[i] = xi - x;
            rowtot[i] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(xi), kWave - 1));
        }
        if (lane_id() < kUPer) {  // lane i writes row i's totals (the wave's own)
            uint32_t x = 0;
#pragma unroll
            for (uint32_t i = 0; i < kUPer; ++i) x = lane_id() == int(i) ? rowtot[i] : x;
            tot_s[lane_id() * kWaves + wave_id()] = x >> 8;
            tot_e[lane_id() * kWaves + wave_id()] = x & 0xFFu;
        }
        __syncthreads();
        if (threadIdx.x < kWave) {
            const uint32_t ts = threadIdx.x < kUPer * kWaves ? tot_s[threadIdx.x] : 0u;
            const uint32_t te = threadIdx.x < kUPer * kWaves ? tot_e[threadIdx.x] : 0u;
            const uint32_t xs = wave_inclusive_scan(ts), xe = wave_inclusive_scan(te);
            if (threadIdx.x < kUPer * kWaves) {
                tot_s[threadIdx.x] = xs - ts;
                tot_e[threadIdx.x] = xe - te;
            }
            if (threadIdx.x == kWave - 1) {
                tot_s[kUPer * kWaves] = xs;
                tot_e[kUPer * kWaves] = xe;
            }
        }
        __syncthreads();
        const uint32_t stot = tot_s[kUPer * kWaves], etot = tot_e[kUPer * kWaves];
        uint32_t bad = 0;
        // the tile must end where the next checkpoint (or the block's count) says
        if (uint64_t(e0) + etot != e1 || (!last && uint64_t(p0) + stot != p1)) bad |= kBadCount;
        // the tile's entries go to slots first_slot + (entries before them in
        // the tile), kept inside the block's range of the message and the
        // capacity by the range of the stores' buffer resources (stores past
        // it are dropped)
        const uint64_t first_slot = uint64_t(sbase) + e0;
        const uint64_t slot_end = umin64(uint64_t(sbase) + cnt, cap);
        const uint32_t room = first_slot < slot_end ? static_cast<uint32_t>(umin64(slot_end - first_slot, kUTile)) : 0u;
        const BufRsrc oi = chunk_buf(reinterpret_cast<const float *>(out_idx + (room ? first_slot : 0)), room);
        const BufRsrc ov = chunk_buf(out_val + (room ? first_slot : 0), room);
        // positions in 32 bits: p0 + (steps before the code in the tile, below
        // 2^28) + run wraps only for a checkpoint near 2^32, which then fails
        // the segment-length test like any position past the segment
        uint32_t far = 0;
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i) {
            const uint32_t row = i * kWaves + wave_id();
            const uint32_t ts = tot_s[row], te = tot_e[row];
            const uint32_t d = ts + (pre[i] >> 8) + (code[i] & rmask);
            const uint32_t rel = p0 + d;
            const bool en = ent_of(i) != 0u;
            const bool out = rel < d || rel >= seg_len;  // wrapped, or past the segment
            far |= en && out ? 1u : 0u;
            // a code that is no entry, or an entry outside its segment, is
            // stored past the resources' range: dropped.  Cached stores: a
            // wave's 256 bytes start anywhere in a line, and the L2 merges
            // the two waves' parts of a shared line (non-temporal stores
            // measured 16% slower on the AdaComp stream)
            const uint32_t o = en && !out ? 4 * (te + (pre[i] & 0xFFu)) : 0x7FFFFFF0u;
            __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(seg_off0) + rel, oi, static_cast<int>(o), 0, 0);
            const float x = kDgc ? v[kDgc ? i : 0] : ((code[i] & 0x8000u) ? -scale : scale);
            __builtin_amdgcn_raw_buffer_store_b32(dev_f2u(x), ov, static_cast<int>(o), 0, 0);
        }
        if (far) bad |= kBadEntry;
        if (bad) atomicOr(status, bad);
        __syncthreads();  // tot_s / tot_e are rewritten by the next tile
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
    if (kind == GC_KIND_DGC)
        GC_LAUNCH("unpack_write", stream, unpack_write_kernel<true><<<grid, kBlock, 0, stream>>>(P, in, w, out->cap, out->seg_scale,
                                                                                                 out->idx, out->val, status));
    else
        GC_LAUNCH("unpack_write", stream, unpack_write_kernel<false><<<grid, kBlock, 0, stream>>>(P, in, w, out->cap, out->seg_scale,
                                                                                                  out->idx, out->val, status));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_unpack launch");
    return GC_OK;
}
