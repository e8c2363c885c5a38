// Compressed model exchange with random quantization, "Communication
// Compression for Decentralized Training" (Tang et al.):
//   DCD-PSGD step 2  z = x_{t+1/2} - x_t, x_{t+1} = x_t + C(z)   (dcd_kernel<kDiff>)
//   DCD-PSGD step 3  replica x^_j <- x^_j + C(z_j)               (dcd_apply_kernel<false>)
//   DCD-PSGD step 1  x_{t+1/2} = sum_j W_ij x^_j - gamma grad    (dcd_mix_kernel)
//   ECD-PSGD Eq. 3   C((1 - t/2) x_{t-1} + (t/2) x_t)           (dcd_kernel<kExtrap>)
//   ECD-PSGD Eq. 4   x~ <- (1 - 2/t) x~ + (2/t) C(z)             (dcd_apply_kernel<true>)
// C is a random quantization; buckets of 512 and 8-bit codes are the
// Quant-DP setting in "Slim-DP" (experimental setup); the DCD page also runs
// 4 bits.
//
// One workgroup per 4096 elements; thread t of row j owns the 4 consecutive
// elements [base + 1024 j + 4 t, +4), which share one Philox4x32-10 block
// (counter = element / 4), so every random word is drawn exactly once.
// Bucket maxima: per-thread max of 4, butterfly max over the lanes of a
// bucket inside a wave, LDS max across waves.
#include <cmath>
#include <string>

#include "gc_internal.hpp"

namespace gc {

namespace {

// What the quantizer is applied to.  kDiff: z = xh - x, and xo = x + C(z) is
// written.  kExtrap: z = fl(a x) + fl(b xh) (x = x_{t-1}, xh = x_t), nothing
// but the codes and scales is written.
enum Source { kDiff, kExtrap };

template <Source kSrc>
__global__ __launch_bounds__(kBlock) void dcd_kernel(const float *x,  // may alias xo
                                                     const float *__restrict__ xh, float *xo,
                                                     uint32_t n, int bits, int blog2,
                                                     uint32_t k0, uint32_t k1, uint64_t step,
                                                     float a, float b,
                                                     float *__restrict__ scales,
                                                     uint8_t *__restrict__ codes) {
    const uint32_t base = blockIdx.x * uint32_t(kChunk);
    const uint32_t bucket = 1u << blog2;
    const int lanes_per_bucket = bucket >= 4 * kWave ? kWave : int(bucket / 4);
    __shared__ uint32_t smax[kChunk / 4];  // up to 1024 buckets of 4
    __shared__ float sinv[kChunk / 4], sstep[kChunk / 4];
    const uint32_t nbk = kChunk >> blog2;
    for (uint32_t b = threadIdx.x; b < nbk; b += kBlock) smax[b] = 0u;
    float xv[kRows][4], zv[kRows][4];
    // dense arrays through chunk-bounded buffer resources: branch-free tail,
    // any dword alignment, non-temporal
    const uint32_t cnt = min(n - base, uint32_t(kChunk));
    const BufRsrc rx = chunk_buf(x + base, cnt), rh = chunk_buf(xh + base, cnt);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        float h[4];
        load4(rx, row_elem(j), xv[j]);
        load4(rh, row_elem(j), h);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (kSrc == kDiff) {
                zv[j][u] = h[u] - xv[j][u];
            } else {
                const float p = a * xv[j][u];
                const float q = b * h[u];
                zv[j][u] = p + q;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t a = dev_f2u(zv[j][u]) & 0x7FFFFFFFu;
            if (a > 0x7F800000u) a = 0u;  // a NaN never counts toward the bucket max
            m = a > m ? a : m;
        }
        for (int d = 1; d < lanes_per_bucket; d <<= 1) {
            uint32_t o = __shfl_xor(m, d, kWave);
            m = m > o ? m : o;
        }
        if ((lane_id() & (lanes_per_bucket - 1)) == 0) atomicMax(&smax[row_elem(j) >> blog2], m);
    }
    __syncthreads();
    const uint32_t L = (1u << (bits - 1)) - 1u;
    const float Lf = static_cast<float>(L);
    // per bucket: inv = fl(L / s_b), step = fl(s_b / L), once
    for (uint32_t b = threadIdx.x; b < nbk; b += kBlock) {
        const float sb = dev_u2f(smax[b]);
        sinv[b] = sb > 0.0f ? Lf / sb : 0.0f;
        sstep[b] = sb > 0.0f ? sb / Lf : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        const uint32_t e0 = row_elem(j);
        const uint32_t i0 = base + e0;
        if (i0 >= n) continue;
        const uint32_t bk = e0 >> blog2;
        const float sb = dev_u2f(smax[bk]);
        const float inv = sinv[bk];
        const float stepq = sstep[bk];
        const uint32_t q = i0 >> 2;
        const uint4 r = philox4x32_10(make_uint4(q, 0u, uint32_t(step), uint32_t(step >> 32)), k0, k1);
        const uint32_t words[4] = {r.x, r.y, r.z, r.w};
        uint32_t code[4];
        float out[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            uint32_t level = 0;
            const float z = zv[j][u];
            float y = sb > 0.0f ? fabsf(z) * inv : 0.0f;
            if (y > Lf) y = Lf;
            // a NaN difference, and every difference in a bucket whose max is
            // infinite (|z| * 0), quantizes to level 0
            if (sb > 0.0f && y == y) {
                const float l0 = floorf(y);
                const float f = y - l0;
                const float uu = static_cast<float>(words[u] >> 8) * 0x1p-24f;
                level = static_cast<uint32_t>(l0) + (uu < f ? 1u : 0u);
            }
            float C = 0.0f;
            code[u] = 0;
            if (level > 0) {
                const float mag = static_cast<float>(level) * stepq;
                const bool neg = dev_f2u(z) >> 31;
                C = neg ? -mag : mag;
                code[u] = (neg ? 1u << (bits - 1) : 0u) | level;
            }
            out[u] = xv[j][u] + C;
        }
        if (kSrc == kDiff) store4(chunk_buf(xo + base, cnt), e0, out);
        if (bits == 8) {
            if (i0 + 3 < n) {
                __builtin_nontemporal_store(code[0] | code[1] << 8 | code[2] << 16 | code[3] << 24,
                                            reinterpret_cast<uint32_t *>(codes + i0));
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (i0 + u < n) codes[i0 + u] = static_cast<uint8_t>(code[u]);
            }
        } else {
            const uint32_t b0 = code[0] | code[1] << 4, b1 = code[2] | code[3] << 4;
            if (i0 + 3 < n) {
                __builtin_nontemporal_store(static_cast<uint16_t>(b0 | b1 << 8),
                                            reinterpret_cast<uint16_t *>(codes + i0 / 2));
            } else {
                // the stream ends inside this group: only bytes holding a
                // real element exist; missing high nibbles stay zero
                codes[i0 / 2] = static_cast<uint8_t>(i0 + 1 < n ? b0 : code[0]);
                if (i0 + 2 < n) codes[i0 / 2 + 1] = static_cast<uint8_t>(i0 + 3 < n ? b1 : code[2]);
            }
        }
    }
    const uint32_t b_first = base >> blog2;
    const uint32_t nb_total = static_cast<uint32_t>((uint64_t(n) + bucket - 1) >> blog2);
    for (uint32_t b = threadIdx.x; b < nbk; b += kBlock)
        if (b_first + b < nb_total) scales[b_first + b] = dev_u2f(smax[b]);
}

// ----------------------------------------------------------------- apply
// Decode C(z) from codes and scales and apply it to a dense model:
// kEcd == false: x <- fl(x + C) (a replica, DCD-PSGD step 3);
// kEcd == true:  x <- fl(fl(c1 x) + fl(c2 C)) (ECD-PSGD Eq. 4).
// One workgroup per 4096 elements in the 4-wide layout; a lane's 4 elements
// share one bucket (buckets are powers of two >= 4) and one 16- or 32-bit
// code word.
template <bool kEcd>
__global__ __launch_bounds__(kBlock) void dcd_apply_kernel(const float *__restrict__ scales,
                                                           const uint8_t *__restrict__ codes,
                                                           float *x, uint32_t n, int bits, int blog2,
                                                           float c1, float c2) {
    const uint32_t base = blockIdx.x * uint32_t(kChunk);
    const uint32_t cnt = min(n - base, uint32_t(kChunk));
    const BufRsrc rx = chunk_buf(x + base, cnt);
    const uint32_t L = (1u << (bits - 1)) - 1u;
    const float Lf = static_cast<float>(L);
    float xv[kRows][4];
    uint32_t word[kRows];
    float sb[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        load4(rx, row_elem(j), xv[j]);
        const uint32_t i0 = base + row_elem(j);
        word[j] = 0u;
        sb[j] = 0.0f;
        if (i0 >= n) continue;
        sb[j] = scales[i0 >> blog2];
        if (i0 + 3 < n) {
            word[j] = bits == 8 ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(codes + i0))
                                : __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(codes + i0 / 2));
        } else if (bits == 8) {
            for (uint32_t u = 0; i0 + u < n; ++u) word[j] |= uint32_t(codes[i0 + u]) << (8 * u);
        } else {
            // bytes exist only for elements below n
            word[j] = codes[i0 / 2];
            if (i0 + 2 < n) word[j] |= uint32_t(codes[i0 / 2 + 1]) << 8;
        }
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        const float stepq = sb[j] / Lf;
        float out[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t code = bits == 8 ? (word[j] >> (8 * u)) & 0xFFu : (word[j] >> (4 * u)) & 0xFu;
            const uint32_t level = code & L;
            float C = 0.0f;
            if (level) {
                const float mag = static_cast<float>(level) * stepq;
                C = (code >> (bits - 1)) ? -mag : mag;
            }
            if (kEcd) {
                const float p = c1 * xv[j][u];
                const float q = c2 * C;
                out[u] = p + q;
            } else {
                out[u] = xv[j][u] + C;
            }
        }
        store4(rx, row_elem(j), out);
    }
}

// ------------------------------------------------------------------- mix
struct MixArgs {
    const float *rep[GC_MAX_REPLICAS];
    float w[GC_MAX_REPLICAS];
};

// x_half = (((+0 + fl(w0 r0)) + fl(w1 r1)) + ...) - fl(lr g), one rounding per
// operation, replicas in the order given.
__global__ __launch_bounds__(kBlock) void dcd_mix_kernel(MixArgs A, int K, const float *__restrict__ g,
                                                         float lr, float *__restrict__ xh, uint32_t n) {
    const uint32_t base = blockIdx.x * uint32_t(kChunk);
    const uint32_t cnt = min(n - base, uint32_t(kChunk));
    float acc[kRows][4];
#pragma unroll
    for (int j = 0; j < kRows; ++j)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[j][u] = 0.0f;
    for (int r = 0; r < K; ++r) {
        const BufRsrc rr = chunk_buf(A.rep[r] + base, cnt);
        const float wr = A.w[r];
        float v[kRows][4];
#pragma unroll
        for (int j = 0; j < kRows; ++j) load4(rr, row_elem(j), v[j]);
#pragma unroll
        for (int j = 0; j < kRows; ++j)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float t = wr * v[j][u];
                acc[j][u] = acc[j][u] + t;
            }
    }
    const BufRsrc rg = chunk_buf(g + base, cnt), ro = chunk_buf(xh + base, cnt);
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        float gv[4], out[4];
        load4(rg, row_elem(j), gv);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float step = lr * gv[u];
            out[u] = acc[j][u] - step;
        }
        store4(ro, row_elem(j), out);
    }
}

}  // namespace

}  // namespace gc

using namespace gc;

namespace {
// Shared host checks of a quantized stream (scales + codes over n elements).
gc_status check_codes(const char *fn, uint64_t n, int bits, uint32_t bucket, const uint8_t *codes) {
    if (bits != 4 && bits != 8) return set_error(GC_EINVAL, std::string(fn) + ": bits must be 4 or 8");
    if (bucket == 0) return set_error(GC_EINVAL, std::string(fn) + ": bucket must be >= 1");
    if (bucket < 4 || bucket > uint32_t(kChunk) || (bucket & (bucket - 1)))
        return set_error(GC_ENOTSUP, std::string(fn) + ": bucket must be a power of two in [4, 4096]");
    if (n > (uint64_t(1) << 32) - 2 * uint64_t(kChunk))
        return set_error(GC_ERANGE, std::string(fn) + ": n must be <= 2^32 - 8192");
    if (reinterpret_cast<uintptr_t>(codes) % 4)
        return set_error(GC_EINVAL, std::string(fn) + ": codes must be 4-byte aligned");
    return GC_OK;
}

int bucket_log2(uint32_t bucket) {
    int b = 0;
    while ((1u << b) < bucket) ++b;
    return b;
}
}  // namespace

extern "C" gc_status gc_dcd_compress(const float *x, const float *x_half, float *x_out, uint64_t n,
                                     int bits, uint32_t bucket, uint64_t seed, uint64_t step,
                                     float *scales, uint8_t *codes, hipStream_t stream) {
    clear_error();
    if (!x || !x_half || !x_out || !scales || !codes)
        return set_error(GC_EINVAL, "gc_dcd_compress: buffers must be non-null");
    if (bits != 4 && bits != 8) return set_error(GC_EINVAL, "gc_dcd_compress: bits must be 4 or 8");
    if (bucket == 0) return set_error(GC_EINVAL, "gc_dcd_compress: bucket must be >= 1");
    if (bucket < 4 || bucket > uint32_t(kChunk) || (bucket & (bucket - 1)))
        return set_error(GC_ENOTSUP, "gc_dcd_compress: bucket must be a power of two in [4, 4096]");
    if (n > (uint64_t(1) << 32) - 2 * uint64_t(kChunk))
        return set_error(GC_ERANGE, "gc_dcd_compress: n must be <= 2^32 - 8192");
    if (reinterpret_cast<uintptr_t>(codes) % 4)
        return set_error(GC_EINVAL, "gc_dcd_compress: codes must be 4-byte aligned");
    if (x_half == x_out && x_half != x)
        return set_error(GC_EINVAL, "gc_dcd_compress: x_out may alias x only");
    if (n == 0) return GC_OK;
    int blog2 = 0;
    while ((1u << blog2) < bucket) ++blog2;
    const unsigned grid = grid_1d(n, kChunk);
    const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
    GC_LAUNCH("dcd", stream, dcd_kernel<kDiff><<<grid, kBlock, 0, stream>>>(x, x_half, x_out, static_cast<uint32_t>(n), bits,
                                                                           blog2, k0, k1, step, 0.0f, 0.0f, scales, codes));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_dcd_compress launch");
    return GC_OK;
}

extern "C" gc_status gc_dcd_decode(const float *scales, const uint8_t *codes, uint64_t n, int bits,
                                   uint32_t bucket, float *x_hat, hipStream_t stream) {
    clear_error();
    if (!scales || !codes || !x_hat) return set_error(GC_EINVAL, "gc_dcd_decode: buffers must be non-null");
    gc_status st = check_codes("gc_dcd_decode", n, bits, bucket, codes);
    if (st != GC_OK) return st;
    if (n == 0) return GC_OK;
    GC_LAUNCH("dcd_decode", stream, dcd_apply_kernel<false><<<grid_1d(n, kChunk), kBlock, 0, stream>>>(
        scales, codes, x_hat, static_cast<uint32_t>(n), bits, bucket_log2(bucket), 0.0f, 0.0f));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_dcd_decode launch");
    return GC_OK;
}

extern "C" gc_status gc_dcd_mix(const float *const *replicas, const float *weights, int K,
                                const float *grad, float lr, float *x_half, uint64_t n,
                                hipStream_t stream) {
    clear_error();
    if (!replicas || !weights || !grad || !x_half)
        return set_error(GC_EINVAL, "gc_dcd_mix: pointers must be non-null");
    if (K < 1 || K > GC_MAX_REPLICAS) return set_error(GC_EINVAL, "gc_dcd_mix: K must be in [1, GC_MAX_REPLICAS]");
    if (n > (uint64_t(1) << 32) - 2 * uint64_t(kChunk))
        return set_error(GC_ERANGE, "gc_dcd_mix: n must be <= 2^32 - 8192");
    MixArgs A{};
    for (int r = 0; r < K; ++r) {
        if (!replicas[r]) return set_error(GC_EINVAL, "gc_dcd_mix: replica pointer is null");
        if (replicas[r] == x_half) return set_error(GC_EINVAL, "gc_dcd_mix: x_half must not alias a replica");
        A.rep[r] = replicas[r];
        A.w[r] = weights[r];
    }
    if (grad == x_half) return set_error(GC_EINVAL, "gc_dcd_mix: x_half must not alias grad");
    if (n == 0) return GC_OK;
    GC_LAUNCH("dcd_mix", stream, dcd_mix_kernel<<<grid_1d(n, kChunk), kBlock, 0, stream>>>(
        A, K, grad, lr, x_half, static_cast<uint32_t>(n)));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_dcd_mix launch");
    return GC_OK;
}

extern "C" gc_status gc_ecd_compress(const float *x_prev, const float *x, uint64_t n, uint64_t t,
                                     int bits, uint32_t bucket, uint64_t seed, float *scales,
                                     uint8_t *codes, hipStream_t stream) {
    clear_error();
    if (!x_prev || !x || !scales || !codes)
        return set_error(GC_EINVAL, "gc_ecd_compress: buffers must be non-null");
    if (t < 1) return set_error(GC_EINVAL, "gc_ecd_compress: t must be >= 1");
    gc_status st = check_codes("gc_ecd_compress", n, bits, bucket, codes);
    if (st != GC_OK) return st;
    if (n == 0) return GC_OK;
    const float a = static_cast<float>(1.0 - 0.5 * static_cast<double>(t));
    const float b = static_cast<float>(0.5 * static_cast<double>(t));
    const uint32_t k0 = static_cast<uint32_t>(seed), k1 = static_cast<uint32_t>(seed >> 32);
    GC_LAUNCH("ecd_compress", stream, dcd_kernel<kExtrap><<<grid_1d(n, kChunk), kBlock, 0, stream>>>(
        x_prev, x, nullptr, static_cast<uint32_t>(n), bits, bucket_log2(bucket), k0, k1, t, a, b, scales, codes));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_ecd_compress launch");
    return GC_OK;
}

extern "C" gc_status gc_ecd_update(const float *scales, const uint8_t *codes, uint64_t n, int bits,
                                   uint32_t bucket, uint64_t t, float *x_tilde, hipStream_t stream) {
    clear_error();
    if (!scales || !codes || !x_tilde) return set_error(GC_EINVAL, "gc_ecd_update: buffers must be non-null");
    if (t < 1) return set_error(GC_EINVAL, "gc_ecd_update: t must be >= 1");
    gc_status st = check_codes("gc_ecd_update", n, bits, bucket, codes);
    if (st != GC_OK) return st;
    if (n == 0) return GC_OK;
    const float c1 = static_cast<float>(1.0 - 2.0 / static_cast<double>(t));
    const float c2 = static_cast<float>(2.0 / static_cast<double>(t));
    GC_LAUNCH("ecd_update", stream, dcd_apply_kernel<true><<<grid_1d(n, kChunk), kBlock, 0, stream>>>(
        scales, codes, x_tilde, static_cast<uint32_t>(n), bits, bucket_log2(bucket), c1, c2));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_error(e, "gc_ecd_update launch");
    return GC_OK;
}
