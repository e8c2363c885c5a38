// A streaming reference for measurement tools: the DGC update's HBM traffic,
// three fp32 reads and two writes per element, with none of its selection
// work, in the dense kernels' chunk tiling, lane layout and cache hints (one
// workgroup per 4096-element chunk, 16-byte raw buffer accesses with the
// non-temporal hint).  Timed beside dgc_update it shows how close the update
// runs to the bandwidth this access pattern reaches on the device.
#include "gc_internal.hpp"

namespace gc {

namespace {

__global__ __launch_bounds__(kBlock) void stream_probe_kernel(const float *__restrict__ a,
                                                              const float *__restrict__ b,
                                                              const float *__restrict__ c, float *__restrict__ d,
                                                              float *__restrict__ e, uint64_t n) {
    const uint64_t lo = uint64_t(blockIdx.x) << kChunkLog2;
    const uint64_t left = n - lo;
    const uint32_t cnt = left < uint64_t(kChunk) ? static_cast<uint32_t>(left) : uint32_t(kChunk);
    const BufRsrc ra = chunk_buf(a + lo, cnt), rb = chunk_buf(b + lo, cnt), rc = chunk_buf(c + lo, cnt);
    const BufRsrc rd = chunk_buf(d + lo, cnt), re = chunk_buf(e + lo, cnt);
    float x[kRows][4], y[kRows][4], z[kRows][4];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        load4(ra, row_elem(j), x[j]);
        load4(rb, row_elem(j), y[j]);
        load4(rc, row_elem(j), z[j]);
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        float p[4], q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            p[k] = x[j][k] + y[j][k];
            q[k] = z[j][k] + p[k];
        }
        store4(rd, row_elem(j), p);
        store4(re, row_elem(j), q);
    }
}

}  // namespace

}  // namespace gc

using namespace gc;

extern "C" gc_status gc_stream_probe(const float *a, const float *b, const float *c, float *d, float *e,
                                     uint64_t n, hipStream_t stream) {
    clear_error();
    if (!a || !b || !c || !d || !e) return set_error(GC_EINVAL, "gc_stream_probe: null pointer");
    if (n >= (uint64_t(1) << 32)) return set_error(GC_ERANGE, "gc_stream_probe: n must be below 2^32");
    for (const void *p : {static_cast<const void *>(a), static_cast<const void *>(b), static_cast<const void *>(c),
                          static_cast<const void *>(d), static_cast<const void *>(e)})
        if (reinterpret_cast<uintptr_t>(p) % 4) return set_error(GC_EINVAL, "gc_stream_probe: pointers must be 4-byte aligned");
    if (n == 0) return GC_OK;
    const unsigned grid = static_cast<unsigned>(ceil_div(n, kChunk));
    GC_LAUNCH("stream_probe", stream, stream_probe_kernel<<<grid, kBlock, 0, stream>>>(a, b, c, d, e, n));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return hip_error(err, "gc_stream_probe launch");
    return GC_OK;
}
