// Host side of libgradcomp: error state, segment-plan validation and tables,
// device upload of the tables, workspace sizing.
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "gc_internal.hpp"

namespace gc {

namespace {
thread_local std::string g_last_error;
}

gc_status set_error(gc_status code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

gc_status hip_error(hipError_t e, const char *what) {
    return set_error(GC_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

void clear_error() { g_last_error.clear(); }

// Layout of the per-device table blob.
struct BlobLayout {
    size_t seg, dchunk, achunk, start, bgroup, xblock, drec, arec, total;
};

static BlobLayout blob_layout(const gc_plan *p) {
    BlobLayout L{};
    size_t o = 0;
    auto take = [&](size_t bytes) {
        o = (o + 255) & ~size_t(255);
        size_t at = o;
        o += bytes;
        return at;
    };
    L.seg = take(sizeof(SegDev) * p->seg.size());
    L.dchunk = take(sizeof(uint32_t) * p->dchunk_seg.size());
    L.achunk = take(sizeof(uint32_t) * p->achunk_seg.size());
    L.start = take(sizeof(uint64_t) * p->seg_start.size());
    L.bgroup = take(sizeof(uint32_t) * p->bgroup_seg.size());
    L.xblock = take(sizeof(uint2) * p->xblock.size());
    L.drec = take(sizeof(ChunkRec) * p->dchunk_rec.size());
    L.arec = take(sizeof(ChunkRec) * p->achunk_rec.size());
    L.total = std::max<size_t>(o, 256);
    return L;
}

unsigned resident_blocks(const void *kernel) {
    static std::mutex mu;
    static std::vector<std::pair<std::pair<int, const void *>, unsigned>> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 1024;
    }
    std::lock_guard<std::mutex> lock(mu);
    for (const auto &c : cache)
        if (c.first.first == dev && c.first.second == kernel) return c.second;
    int per = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, kBlock, 0) != hipSuccess || per < 1) {
        (void)hipGetLastError();
        per = 1;
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        cus = 1;
    }
    const unsigned v = static_cast<unsigned>(per) * static_cast<unsigned>(cus);
    cache.push_back({{dev, kernel}, v});
    return v;
}

static gc_status plan_tables(const gc_plan *cplan, PlanDev *out, bool upload) {
    gc_plan *plan = const_cast<gc_plan *>(cplan);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_error(e, "hipGetDevice");
    BlobLayout L = blob_layout(plan);
    void *blob = nullptr;
    {
        std::lock_guard<std::mutex> lock(plan->mu);
        for (auto &pr : plan->dev_blob)
            if (pr.first == dev) blob = pr.second;
        if (!blob && !upload)
            return set_error(GC_EINVAL, "the plan's tables are not on the current device: call gc_plan_upload first");
        if (!blob) {
            e = hipMalloc(&blob, L.total);
            if (e != hipSuccess) return hip_error(e, "hipMalloc(plan tables)");
            std::vector<uint8_t> host(L.total, 0);
            std::memcpy(host.data() + L.seg, plan->seg.data(), sizeof(SegDev) * plan->seg.size());
            std::memcpy(host.data() + L.dchunk, plan->dchunk_seg.data(),
                        sizeof(uint32_t) * plan->dchunk_seg.size());
            std::memcpy(host.data() + L.achunk, plan->achunk_seg.data(),
                        sizeof(uint32_t) * plan->achunk_seg.size());
            std::memcpy(host.data() + L.start, plan->seg_start.data(),
                        sizeof(uint64_t) * plan->seg_start.size());
            std::memcpy(host.data() + L.bgroup, plan->bgroup_seg.data(),
                        sizeof(uint32_t) * plan->bgroup_seg.size());
            std::memcpy(host.data() + L.xblock, plan->xblock.data(), sizeof(uint2) * plan->xblock.size());
            std::memcpy(host.data() + L.drec, plan->dchunk_rec.data(),
                        sizeof(ChunkRec) * plan->dchunk_rec.size());
            std::memcpy(host.data() + L.arec, plan->achunk_rec.data(),
                        sizeof(ChunkRec) * plan->achunk_rec.size());
            e = hipMemcpy(blob, host.data(), L.total, hipMemcpyHostToDevice);
            if (e != hipSuccess) {
                (void)hipFree(blob);
                return hip_error(e, "hipMemcpy(plan tables)");
            }
            plan->dev_blob.emplace_back(dev, blob);
        }
    }
    auto *b = static_cast<uint8_t *>(blob);
    out->seg = reinterpret_cast<const SegDev *>(b + L.seg);
    out->dchunk_seg = reinterpret_cast<const uint32_t *>(b + L.dchunk);
    out->achunk_seg = reinterpret_cast<const uint32_t *>(b + L.achunk);
    out->seg_start = reinterpret_cast<const uint64_t *>(b + L.start);
    out->bgroup_seg = reinterpret_cast<const uint32_t *>(b + L.bgroup);
    out->xblock = reinterpret_cast<const uint2 *>(b + L.xblock);
    out->dchunk_rec = reinterpret_cast<const ChunkRec *>(b + L.drec);
    out->achunk_rec = reinterpret_cast<const ChunkRec *>(b + L.arec);
    out->nseg = plan->nseg;
    out->nbgroup = plan->nbgroup;
    out->nxblock = static_cast<uint32_t>(plan->xblock.size());
    out->ndchunk = plan->ndchunk;
    out->nachunk = plan->nachunk;
    out->n_total = plan->n_total;
    return GC_OK;
}

gc_status plan_device(const gc_plan *plan, PlanDev *out) { return plan_tables(plan, out, true); }

gc_status plan_device_resident(const gc_plan *plan, PlanDev *out) { return plan_tables(plan, out, false); }

}  // namespace gc

using namespace gc;

extern "C" {

const char *gc_last_error(void) { return g_last_error.c_str(); }

const char *gc_version(void) { return "libgradcomp 0.1.0 (gfx950)"; }

uint32_t gc_topk_count(uint32_t n) {
    uint64_t k = (static_cast<uint64_t>(n) + 999) / 1000;
    return static_cast<uint32_t>(k < 1 ? 1 : k);
}

gc_status gc_plan_create(const gc_segment *segs, int nseg, uint64_t n_total, gc_plan **out) {
    clear_error();
    if (!out) return set_error(GC_EINVAL, "gc_plan_create: out is null");
    if (nseg < 1) return set_error(GC_EINVAL, "gc_plan_create: nseg must be >= 1");
    if (!segs) return set_error(GC_EINVAL, "gc_plan_create: segs is null");
    if (n_total >= (uint64_t(1) << 32))
        return set_error(GC_ERANGE, "gc_plan_create: n_total must be < 2^32 (u32 indices)");
    uint64_t prev_end = 0, total_k = 0, total_bins = 0;
    uint64_t ndchunk = 0, nachunk = 0;
    for (int s = 0; s < nseg; ++s) {
        const gc_segment &g = segs[s];
        std::string at = "gc_plan_create: segment " + std::to_string(s) + ": ";
        if (g.reserved != 0) return set_error(GC_EINVAL, at + "reserved field must be 0");
        if (g.length < 1) return set_error(GC_EINVAL, at + "length must be >= 1");
        if (g.offset < prev_end)
            return set_error(GC_EINVAL, at + "segments must be ascending and non-overlapping");
        // compared without forming offset + length, which wraps for offsets
        // near 2^64
        if (g.offset >= n_total || g.length > n_total - g.offset)
            return set_error(GC_EINVAL, at + "segment extends past n_total");
        if (g.bin_len < 1) return set_error(GC_EINVAL, at + "bin_len must be >= 1");
        if (g.bin_len > GC_MAX_BIN_LEN)
            return set_error(GC_ENOTSUP, at + "bin_len above GC_MAX_BIN_LEN");
        if (g.length > GC_MAX_SEGMENT_LEN)
            return set_error(GC_ENOTSUP, at + "length above GC_MAX_SEGMENT_LEN");
        if (g.k < 1 || g.k > g.length) return set_error(GC_EINVAL, at + "k must be in [1, length]");
        prev_end = g.offset + g.length;
        total_k += g.k;
        total_bins += ceil_div(g.length, g.bin_len);
        ndchunk += ceil_div(g.length, kChunk);
        uint32_t per = (kChunk / g.bin_len) * g.bin_len;  // whole bins per AdaComp chunk
        nachunk += ceil_div(g.length, per);
    }
    if (ndchunk >= (uint64_t(1) << 31) || nachunk >= (uint64_t(1) << 31))
        return set_error(GC_ERANGE, "gc_plan_create: too many chunks");

    gc_plan *p = new (std::nothrow) gc_plan;
    if (!p) return set_error(GC_EINVAL, "gc_plan_create: out of host memory");
    p->nseg = nseg;
    p->n_total = n_total;
    p->total_k = total_k;
    p->total_bins = total_bins;
    p->seg.resize(nseg);
    p->seg_start.resize(nseg);
    p->dchunk_seg.reserve(ndchunk);
    p->achunk_seg.reserve(nachunk);
    uint32_t bin0 = 0, kbase = 0, mbase = 0;
    uint64_t seg_elems = 0;
    for (int s = 0; s < nseg; ++s) {
        const gc_segment &g = segs[s];
        SegDev d{};
        d.off = g.offset;
        d.len = g.length;
        d.bin_len = g.bin_len;
        d.k = g.k;
        d.nbins = static_cast<uint32_t>(ceil_div(g.length, g.bin_len));
        d.dchunk0 = static_cast<uint32_t>(p->dchunk_seg.size());
        d.dnchunk = static_cast<uint32_t>(ceil_div(g.length, kChunk));
        d.achunk_len = (kChunk / g.bin_len) * g.bin_len;
        d.achunk0 = static_cast<uint32_t>(p->achunk_seg.size());
        d.anchunk = static_cast<uint32_t>(ceil_div(g.length, d.achunk_len));
        d.bin0 = bin0;
        d.kbase = kbase;
        d.mbase = mbase;
        mbase += static_cast<uint32_t>(ceil_div(g.length, 32));
        d.bgroup0 = static_cast<uint32_t>(p->bgroup_seg.size());
        d.nbgroup = (d.nbins + kBinGroup - 1) / kBinGroup;
        for (uint32_t g2 = 0; g2 < d.nbgroup; ++g2) p->bgroup_seg.push_back(static_cast<uint32_t>(s));
        bin0 += d.nbins;
        kbase += g.k;
        for (uint32_t c = 0; c < d.dnchunk; c += kXBlockChunks)
            p->xblock.push_back(make_uint2(static_cast<uint32_t>(s), d.dchunk0 + c));
        for (uint32_t c = 0; c < d.dnchunk; ++c) {
            p->dchunk_seg.push_back(static_cast<uint32_t>(s));
            const uint32_t first = c * uint32_t(kChunk);
            const uint32_t cnt = std::min<uint32_t>(uint32_t(kChunk), g.length - first);
            p->dchunk_rec.push_back(make_uint4(static_cast<uint32_t>(g.offset + first), cnt,
                                               static_cast<uint32_t>(s), c));
        }
        for (uint32_t c = 0; c < d.anchunk; ++c) {
            p->achunk_seg.push_back(static_cast<uint32_t>(s));
            const uint32_t first = c * d.achunk_len;
            const uint32_t cnt = std::min<uint32_t>(d.achunk_len, g.length - first);
            p->achunk_rec.push_back(make_uint4(static_cast<uint32_t>(g.offset + first), cnt,
                                               static_cast<uint32_t>(s),
                                               d.bin0 + c * (d.achunk_len / g.bin_len)));
        }
        p->seg[s] = d;
        p->seg_start[s] = g.offset;
        seg_elems += g.length;
    }
    p->ndchunk = static_cast<uint32_t>(p->dchunk_seg.size());
    p->nachunk = static_cast<uint32_t>(p->achunk_seg.size());
    p->nbgroup = static_cast<uint32_t>(p->bgroup_seg.size());
    p->mask_words = mbase;
    p->seg_elems = seg_elems;
    p->dgc_fast = dgc_exact_fast(p, 0, 0);
    *out = p;
    return GC_OK;
}

gc_status gc_plan_upload(const gc_plan *plan) {
    clear_error();
    if (!plan) return set_error(GC_EINVAL, "gc_plan_upload: plan is null");
    PlanDev P;
    return plan_device(plan, &P);
}

void gc_plan_destroy(gc_plan *plan) {
    if (!plan) return;
    int cur = 0;
    bool have = hipGetDevice(&cur) == hipSuccess;
    for (auto &pr : plan->dev_blob) {
        if (hipSetDevice(pr.first) == hipSuccess) (void)hipFree(pr.second);
    }
    if (have) (void)hipSetDevice(cur);
    delete plan;
}

int gc_plan_num_segments(const gc_plan *plan) { return plan ? plan->nseg : 0; }
uint64_t gc_plan_num_elements(const gc_plan *plan) { return plan ? plan->n_total : 0; }
uint64_t gc_plan_total_k(const gc_plan *plan) { return plan ? plan->total_k : 0; }
uint64_t gc_plan_total_bins(const gc_plan *plan) { return plan ? plan->total_bins : 0; }

size_t gc_plan_workspace_bytes(const gc_plan *plan, int op) {
    if (!plan) return 0;
    switch (op) {
        case GC_OP_DGC: return dgc_workspace_bytes(plan);
        case GC_OP_ADACOMP: return adacomp_workspace_bytes(plan);
        case GC_OP_PACK: return pack_workspace_bytes(plan);
        case GC_OP_DECODE: return decode_workspace_bytes(plan);
        case GC_OP_UNPACK: return unpack_workspace_bytes(plan);
        default: return 0;
    }
}

}  // extern "C"
