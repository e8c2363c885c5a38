// The receiving side of the packed exchange: a run-length stream read back
// into a message.  "Deep Gradient Compression" (Lin et al.) §3.1: 32-bit
// values with 16-bit zero-run lengths (AdaComp codes carry a sign bit and one
// layer scale instead).
//
// A segment's codes are read in tiles of 4096.  An element position is the
// sum of the steps before the code plus its run (a step is run + 1 for an
// entry and MAX for an escape); an entry's slot is the count of entries
// before it.  Both sums are prefix scans, so the path is
//   walk  (one workgroup) follow the block headers from the stream start
//         (each block's size depends on its entry count), check them against
//         the plan, and lay out the tiles
//   count (tile) entries and summed steps per tile
//   scan  (one workgroup) entry slots (over all tiles) and step prefixes
//   write (tile) block scans of steps and entries; idx, val
// Anything that does not fit the plan sets a bit in *status and is not
// written; the message stays within its capacity and its segments.
#include <algorithm>

#include "gc_internal.hpp"

namespace gc {

namespace {

constexpr uint32_t kUTile = 4096;
constexpr uint32_t kUPer = kUTile / kBlock;  // codes per thread in a tile

// status bits
constexpr uint32_t kBadStream = 1u, kBadBlock = 2u, kBadEntry = 4u, kOverCap = 8u, kBadCount = 16u;

struct UnpackWs {
    uint64_t *blk_off;    // [nseg] byte offset of each block
    uint32_t *seg_E;      // [nseg] codes of each block (0 for a bad block)
    uint32_t *seg_w3;     // [nseg] the header's last word (DGC count, AdaComp scale bits)
    uint32_t *tile_base;  // [nseg + 1]
    uint32_t *tile_cnt;   // [max_tiles] entries per tile
    uint32_t *tile_steps; // [max_tiles] summed steps per tile
    uint32_t *tile_out;   // [max_tiles + 1] first slot of each tile
    uint64_t *tile_gpos;  // [max_tiles + 1] steps before each tile, over all tiles
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
    w.seg_w3 = c.take<uint32_t>(p->nseg);
    w.tile_base = c.take<uint32_t>(p->nseg + 1);
    w.tile_cnt = c.take<uint32_t>(w.max_tiles);
    w.tile_steps = c.take<uint32_t>(w.max_tiles);
    w.tile_out = c.take<uint32_t>(w.max_tiles + 1);
    w.tile_gpos = c.take<uint64_t>(w.max_tiles + 1);
    if (bytes) *bytes = c.used + 256;
    return w;
}

constexpr uint32_t magic(char a, char b, char c, char d) {
    return uint32_t(uint8_t(a)) | uint32_t(uint8_t(b)) << 8 | uint32_t(uint8_t(c)) << 16 |
           uint32_t(uint8_t(d)) << 24;
}

__device__ __forceinline__ uint64_t block_bytes(uint64_t E, bool dgc) {
    return 16 + 2 * E + 2 * (E & 1u) + (dgc ? 4 * E : 0);
}

// One block header read at `at` by one thread, with the checks of the
// sequential walk: on a bad header the block counts as empty (E = 0) and st
// gets kBadBlock; once st is set no header is read.  Returns the block's
// bytes.
__device__ __forceinline__ uint64_t walk_one(const PlanDev &P, bool dgc, uint32_t MAX, uint32_t bmagic,
                                             const uint8_t *in, uint64_t nbytes, int s, uint64_t at, uint32_t &st,
                                             UnpackWs &w, float *seg_scale) {
    uint32_t E = 0, w3 = 0;
    if (!st && at + 16 <= nbytes) {
        const uint32_t *b = reinterpret_cast<const uint32_t *>(in + at);
        const uint32_t m = b[0], n = b[1];
        E = b[2];
        w3 = b[3];
        if (m != bmagic || n != P.seg[s].len || E > max_codes(n, MAX) || at + block_bytes(E, dgc) > nbytes) {
            st |= kBadBlock;
            E = 0;
        }
    } else if (!st) {
        st |= kBadBlock;
    }
    w.blk_off[s] = at;
    w.seg_E[s] = E;
    w.seg_w3[s] = w3;
    if (seg_scale) seg_scale[s] = dgc || st ? 0.0f : dev_u2f(w3);
    return block_bytes(E, dgc);
}

// One workgroup; the headers are a chain (each block's size comes from its
// own header), then the workgroup lays out the tiles.  AdaComp: thread 0
// follows the chain.  DGC: a block normally holds exactly k_s codes (an
// escape needs a gap of 65535 unsent elements), so wave 0 predicts the next
// 64 headers' offsets from k, reads them at once, and keeps the prefix whose
// headers are valid with E = k (what the sequential walk computes for them);
// the first block that differs is read at its now known offset by the
// sequential rule, and the next round predicts from there.
__global__ __launch_bounds__(kBlock) void unpack_walk_kernel(PlanDev P, int kind, const uint8_t *__restrict__ in,
                                                             uint64_t nbytes, UnpackWs w, float *seg_scale,
                                                             uint32_t *status) {
    const bool dgc = kind == GC_KIND_DGC;
    const uint32_t MAX = dgc ? 65535u : 32767u;
    const uint32_t bmagic = dgc ? magic('D', 'G', 'C', '1') : magic('A', 'D', 'C', '1');
    if (threadIdx.x < kWave) {
        const int lane = lane_id();
        uint32_t st = 0;
        const uint32_t *h = reinterpret_cast<const uint32_t *>(in);
        if (nbytes < 16 || h[0] != magic('G', 'C', 'P', '1') || h[1] != uint32_t(kind) || h[2] != uint32_t(P.nseg))
            st |= kBadStream;
        uint64_t at = 16;
        if (!dgc) {
            if (lane == 0)
                for (int s = 0; s < P.nseg; ++s) at += walk_one(P, dgc, MAX, bmagic, in, nbytes, s, at, st, w, seg_scale);
        } else {
            int s = 0;
            while (s < P.nseg && !st) {
                const int sl = s + lane;
                const bool live = sl < P.nseg;
                const uint32_t k = live ? P.seg[sl].k : 0u;
                const uint32_t len = live ? P.seg[sl].len : 0u;
                const uint64_t sz = live ? block_bytes(k, true) : 0;
                uint64_t incl = sz;  // inclusive scan of the predicted sizes
#pragma unroll
                for (int d = 1; d < kWave; d <<= 1) {
                    const uint64_t y = __shfl_up(incl, d, kWave);
                    if (lane >= d) incl += y;
                }
                const uint64_t my_at = at + incl - sz;
                bool ok = false;
                uint32_t w3 = 0;
                if (live && my_at + 16 <= nbytes) {
                    const uint32_t *b = reinterpret_cast<const uint32_t *>(in + my_at);
                    w3 = b[3];
                    ok = b[0] == bmagic && b[1] == len && b[2] == k && my_at + sz <= nbytes;
                }
                const uint64_t bad = __ballot(live && !ok);
                const int nlive = P.nseg - s < kWave ? P.nseg - s : kWave;
                const int f = bad ? __ffsll(static_cast<long long>(bad)) - 1 : nlive;  // confirmed blocks
                if (lane < f) {
                    w.blk_off[sl] = my_at;
                    w.seg_E[sl] = k;
                    w.seg_w3[sl] = w3;
                    if (seg_scale) seg_scale[sl] = 0.0f;
                }
                if (f > 0) at = __shfl(my_at + sz, f - 1, kWave);
                s += f;
                if (f < nlive) {
                    // block s differs from the prediction: the sequential rule
                    uint64_t add = 0;
                    if (lane == 0) add = walk_one(P, dgc, MAX, bmagic, in, nbytes, s, at, st, w, seg_scale);
                    at += __shfl(add, 0, kWave);
                    st = __shfl(st, 0, kWave);
                    ++s;
                }
            }
            // after a bad block the rest are read as empty, as in the sequential walk
            for (int r = s + lane; r < P.nseg; r += kWave) {
                w.blk_off[r] = at + 16ull * uint64_t(r - s);
                w.seg_E[r] = 0;
                w.seg_w3[r] = 0;
                if (seg_scale) seg_scale[r] = 0.0f;
            }
            if (s < P.nseg) at += 16ull * uint64_t(P.nseg - s);
        }
        if (lane == 0) {
            if (!st && at != nbytes) st |= kBadBlock;
            *status = st;
        }
    }
    __syncthreads();
    uint32_t run = 0;
    for (int r = 0; r < P.nseg; r += kBlock) {
        const int s = r + int(threadIdx.x);
        const uint32_t v = s < P.nseg ? (w.seg_E[s] + kUTile - 1) / kUTile : 0u;
        uint32_t tot;
        const uint32_t pre = block_exclusive_scan(v, &tot);
        if (s < P.nseg) w.tile_base[s] = run + pre;
        run += tot;
    }
    if (threadIdx.x == 0) w.tile_base[P.nseg] = run;
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

__device__ __forceinline__ const uint16_t *block_runs(const uint8_t *in, const UnpackWs &w, uint32_t s) {
    return reinterpret_cast<const uint16_t *>(in + w.blk_off[s] + 16);
}

__global__ __launch_bounds__(kBlock) void unpack_count_kernel(PlanDev P, int kind, const uint8_t *__restrict__ in,
                                                              UnpackWs w) {
    const uint32_t ntiles = w.tile_base[P.nseg];
    if (blockIdx.x >= ntiles) return;
    const uint32_t MAX = kind == GC_KIND_DGC ? 65535u : 32767u;
    const uint32_t rmask = kind == GC_KIND_DGC ? 0xFFFFu : 0x7FFFu;
    __shared__ uint32_t lds[kLdsSegs];
    TileOf table;
    table.init(w.tile_base, P.nseg, lds);
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint32_t s = table.segment(t);
        const uint32_t E = w.seg_E[s];
        const uint32_t j0 = (t - w.tile_base[s]) * kUTile;
        const uint16_t *runs = block_runs(in, w, s);
        uint32_t code[kUPer];
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i) code[i] = runs[min(j0 + i * kBlock + threadIdx.x, E - 1)];
        uint32_t cnt = 0, steps = 0;
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i) {
            if (j0 + i * kBlock + threadIdx.x >= E) continue;
            const uint32_t r = code[i] & rmask;
            const bool esc = r == MAX;
            cnt += esc ? 0u : 1u;
            steps += esc ? MAX : r + 1;
        }
        uint32_t tc, ts;
        (void)block_exclusive_scan(cnt, &tc);
        (void)block_exclusive_scan(steps, &ts);
        if (threadIdx.x == 0) {
            w.tile_cnt[t] = tc;
            w.tile_steps[t] = ts;
        }
    }
}

// One workgroup: slots and step prefixes over all tiles, segment offsets, the
// capacity and the DGC header counts.
constexpr uint32_t kScanRun = 16;

__global__ __launch_bounds__(kBlock) void unpack_scan_kernel(PlanDev P, int kind, UnpackWs w, uint64_t cap,
                                                             uint32_t *__restrict__ seg_off, uint32_t *status) {
    const uint32_t ntiles = w.tile_base[P.nseg];
    uint32_t out_run = 0;
    uint64_t pos_run = 0;
    for (uint32_t r0 = 0; r0 < ntiles; r0 += kBlock * kScanRun) {
        const uint32_t t0 = r0 + threadIdx.x * kScanRun;
        uint32_t c[kScanRun], st[kScanRun];
        uint32_t csum = 0;
        uint64_t ssum = 0;
#pragma unroll
        for (uint32_t u = 0; u < kScanRun; ++u) {
            const bool in = t0 + u < ntiles;
            c[u] = in ? w.tile_cnt[t0 + u] : 0u;
            st[u] = in ? w.tile_steps[t0 + u] : 0u;
            csum += c[u];
            ssum += st[u];
        }
        uint32_t ctot;
        uint64_t stot;
        uint32_t cpre = out_run + block_exclusive_scan(csum, &ctot);
        uint64_t spre = pos_run + block_exclusive_scan<uint64_t>(ssum, &stot);
#pragma unroll
        for (uint32_t u = 0; u < kScanRun; ++u) {
            if (t0 + u >= ntiles) break;
            w.tile_out[t0 + u] = cpre;
            w.tile_gpos[t0 + u] = spre;
            cpre += c[u];
            spre += st[u];
        }
        out_run += ctot;
        pos_run += stot;
    }
    if (threadIdx.x == 0) {
        w.tile_out[ntiles] = out_run;
        w.tile_gpos[ntiles] = pos_run;
    }
    __syncthreads();
    uint32_t bad = 0;
    for (int s = threadIdx.x; s <= P.nseg; s += kBlock) {
        const uint32_t o = w.tile_out[w.tile_base[s]];
        seg_off[s] = static_cast<uint32_t>(min<uint64_t>(o, cap));
        if (s < P.nseg && kind == GC_KIND_DGC) {
            const uint32_t cnt = w.tile_out[w.tile_base[s + 1]] - o;
            if (w.seg_E[s] && cnt != w.seg_w3[s]) bad |= kBadCount;
        }
    }
    if (out_run > cap) bad |= kOverCap;
    if (bad) atomicOr(status, bad);
}

// Exclusive prefix of one value per element in the tile's order, element
// (row i, thread t) being code i * kBlock + t: a wave scan per row, then one
// wave scans the kUPer * kWaves (row, wave) totals.
__device__ __forceinline__ void block_row_scan(const uint32_t (&v)[kUPer], uint32_t (&ex)[kUPer]) {
    static_assert(kUPer * kWaves <= kWave, "one wave scans the row totals");
    __shared__ uint32_t tot[kUPer * kWaves];
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
    }
    __syncthreads();
#pragma unroll
    for (uint32_t i = 0; i < kUPer; ++i) ex[i] = tot[i * kWaves + wave_id()] + incl[i] - v[i];
    __syncthreads();
}

// Code i * kBlock + t of the tile is thread t's i-th: loads and the entries'
// stores are coalesced along a row; the row-order scans give every code its
// position and slot.
__global__ __launch_bounds__(kBlock) void unpack_write_kernel(PlanDev P, int kind, const uint8_t *__restrict__ in,
                                                              UnpackWs w, uint64_t cap,
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
        const uint32_t E = w.seg_E[s];
        const uint32_t j0 = (t - w.tile_base[s]) * kUTile;
        const uint16_t *runs = block_runs(in, w, s);
        const float *vals = reinterpret_cast<const float *>(in + w.blk_off[s] + 16 + 2ull * E + 2ull * (E & 1u));
        const float scale = dev_u2f(w.seg_w3[s]);
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
        block_row_scan(steps, spre);
        block_row_scan(ent, epre);
        const uint64_t pos0 = w.tile_gpos[t] - w.tile_gpos[w.tile_base[s]];
        const uint32_t slot0 = w.tile_out[t];
        uint32_t bad = 0;
#pragma unroll
        for (uint32_t i = 0; i < kUPer; ++i) {
            if (!ent[i]) continue;
            const uint64_t rel = pos0 + spre[i] + (code[i] & rmask);
            const uint32_t slot = slot0 + epre[i];
            if (rel >= seg.len) {
                bad |= kBadEntry;
            } else if (slot < cap) {
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
    GC_LAUNCH("unpack_walk", stream, unpack_walk_kernel<<<1, kBlock, 0, stream>>>(P, kind, in, in_bytes, w, out->seg_scale, status));
    GC_LAUNCH("unpack_count", stream, unpack_count_kernel<<<grid, kBlock, 0, stream>>>(P, kind, in, w));
    GC_LAUNCH("unpack_scan", stream, unpack_scan_kernel<<<1, kBlock, 0, stream>>>(P, kind, w, out->cap, out->seg_off, status));
    GC_LAUNCH("unpack_write", stream, unpack_write_kernel<<<grid, kBlock, 0, stream>>>(P, kind, in, w, out->cap, out->idx,
                                                                                       out->val, status));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_unpack launch");
    return GC_OK;
}
