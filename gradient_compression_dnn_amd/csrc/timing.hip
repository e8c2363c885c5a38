// Optional per-kernel timing with HIP events on the caller's stream, for
// measurement tools (gc_timing_enable / gc_timing_take).
#include <atomic>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "gc_internal.hpp"

namespace gc {

namespace {

struct Pair {
    hipEvent_t start, stop;
};

std::mutex g_mu;
std::atomic<bool> g_on{false};
bool g_all = false;
std::set<std::string> g_selected;
std::map<std::string, std::vector<Pair>> g_records;
std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
    if (!g_pool.empty()) {
        hipEvent_t e = g_pool.back();
        g_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

}  // namespace

hipEvent_t timing_begin(const char *kernel, hipStream_t s) {
    if (!g_on.load(std::memory_order_relaxed)) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_all && !g_selected.count(kernel)) return nullptr;
    hipEvent_t e = take_event();
    if (e && hipEventRecord(e, s) != hipSuccess) {
        g_pool.push_back(e);
        return nullptr;
    }
    return e;
}

void timing_end(const char *kernel, hipEvent_t start, hipStream_t s) {
    std::lock_guard<std::mutex> lock(g_mu);
    hipEvent_t e = take_event();
    if (!e || hipEventRecord(e, s) != hipSuccess) {
        g_pool.push_back(start);
        if (e) g_pool.push_back(e);
        return;
    }
    g_records[kernel].push_back({start, e});
}

}  // namespace gc

using namespace gc;

extern "C" gc_status gc_timing_enable(const char *kernels) {
    clear_error();
    std::lock_guard<std::mutex> lock(g_mu);
    g_selected.clear();
    g_all = false;
    if (!kernels || !*kernels) {
        g_on.store(false);
        return GC_OK;
    }
    std::string list(kernels);
    size_t at = 0;
    while (at <= list.size()) {
        size_t comma = list.find(',', at);
        if (comma == std::string::npos) comma = list.size();
        std::string name = list.substr(at, comma - at);
        if (name == "*") g_all = true;
        else if (!name.empty()) g_selected.insert(name);
        at = comma + 1;
    }
    g_on.store(true);
    return GC_OK;
}

extern "C" gc_status gc_timing_take(const char *kernel, double *total_ms, uint64_t *launches) {
    clear_error();
    if (!kernel || !total_ms || !launches)
        return set_error(GC_EINVAL, "gc_timing_take: null argument");
    std::vector<Pair> recs;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        auto it = g_records.find(kernel);
        if (it != g_records.end()) {
            recs.swap(it->second);
            g_records.erase(it);
        }
    }
    double sum = 0.0;
    gc_status st = GC_OK;
    for (const Pair &p : recs) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(p.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start, p.stop);
        if (e != hipSuccess && st == GC_OK) st = hip_error(e, "gc_timing_take");
        sum += ms;
    }
    {
        std::lock_guard<std::mutex> lock(g_mu);
        for (const Pair &p : recs) {
            g_pool.push_back(p.start);
            g_pool.push_back(p.stop);
        }
    }
    *total_ms = sum;
    *launches = recs.size();
    return st;
}
