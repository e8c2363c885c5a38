/*
 * Oracle for libgradcomp — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of every result the
 * compression path computes.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may build, load or call it; the product path
 * never does.  It shares no code, header, table or helper with the HIP path.
 *
 * Arithmetic: gradients and states are fp32 (the DGC encoder carries 32-bit
 * values; residuals and momenta live in the same fp32 layout), so every
 * elementwise step is one correctly rounded fp32 IEEE operation, in the order
 * written, with no contraction (built with -ffp-contract=off).  Reductions are
 * in fp64 through orc_psum64's fixed pairwise tree.
 *
 * Parity pins: every function is pinned by tests that do not re-run it (hand
 * derived golden values, closed forms, invariants, brute force on tiny
 * inputs, published known-answer vectors).  See tests/test_oracle_*.py.
 */
#ifndef GC_ORACLE_H
#define GC_ORACLE_H
#include <stdint.h>

typedef struct orc_seg {
    uint64_t offset;
    uint32_t length;
    uint32_t bin_len;
    uint32_t k;
    uint32_t pad;
} orc_seg;

/* Number of threads the OpenMP runtime uses (1 when built without OpenMP). */
int orc_num_threads(void);
void orc_set_num_threads(int n);

/* Pairwise sum in fp64: pad x[0..m) with +0.0 to the next power of two and
 * add as a perfect binary tree in index order. */
double orc_psum64(const double *x, uint64_t m);

/* AdaComp step on every segment (see oracle.c for the steps).
 * gmax_out (optional) receives all bin maxima, segments in order. */
void orc_adacomp(const orc_seg *segs, int nseg, const float *dW, float *R,
                 float scale_factor, uint32_t *out_idx, float *out_val,
                 uint32_t *seg_off, float *seg_scale, float *gmax_out);
/* The same with the threshold rule chosen: 0 as orc_adacomp, 1 the factor on
 * the new gradient with the bin max always sent (see oracle.c). */
void orc_adacomp_rule(const orc_seg *segs, int nseg, const float *dW, float *R,
                      float scale_factor, int rule, uint32_t *out_idx, float *out_val,
                      uint32_t *seg_off, float *seg_scale, float *gmax_out);

/* DGC options.  nesterov: 0 vanilla momentum (Alg. 3), 1 Nesterov (Alg. 4).
 * sampled: 0 exact top-k; 1 threshold estimated from a sample of one
 * 32-element block per window of 32*sample_period elements, with the exact
 * top-k taken instead when more than over*k entries pass it. */
typedef struct orc_dgc_opts {
    float momentum;
    float thr_G;
    int num_nodes;
    int nesterov;
    int sampled;
    uint32_t sample_period;
    uint32_t over;
    uint32_t pad;
} orc_dgc_opts;

/* DGC step on every segment; the message is compact (seg_off[nseg] entries).
 * clip_out (optional) receives the per-segment clip coefficient. */
void orc_dgc_ex(const orc_seg *segs, int nseg, const float *G, float *U, float *V,
                const orc_dgc_opts *opts, uint32_t *out_idx, float *out_val,
                uint32_t *seg_off, float *clip_out);

/* DGC step, vanilla momentum, exact top-k. */
void orc_dgc(const orc_seg *segs, int nseg, const float *G, float *U, float *V,
             float momentum, float thr_G, int num_nodes, uint32_t *out_idx,
             float *out_val, uint32_t *seg_off, float *clip_out);

/* Run-length packing.  kind 1 = DGC, 2 = AdaComp.  Returns bytes written,
 * or 0 if cap is too small. */
uint64_t orc_pack(int kind, const orc_seg *segs, int nseg,
                  const uint32_t *idx, const float *val,
                  const uint32_t *seg_off, const float *seg_scale,
                  uint8_t *out, uint64_t cap);

/* Read a packed stream back into a message (idx, val, seg_off[nseg+1],
 * seg_scale[nseg]) of at most cap entries.  Returns 0, or nonzero for a
 * stream that does not fit the plan. */
int orc_unpack(int kind, const orc_seg *segs, int nseg, const uint8_t *buf, uint64_t nbytes,
               uint32_t *idx, float *val, uint32_t *seg_off, float *seg_scale, uint64_t cap);

/* Decompress-aggregate K messages (idx[k], val[k], count[k]) into dense.
 * mode 0 = sum, 1 = average; accumulate != 0 adds into dense. */
void orc_decode(const orc_seg *segs, int nseg, int K,
                const uint32_t *const *idx, const float *const *val,
                const uint64_t *count, float *dense, int mode, int accumulate);

/* Philox4x32-10 block: out = philox(ctr, key). */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                       uint32_t out[4]);

/* DCD difference + random quantization on a flat buffer. */
void orc_dcd(const float *x, const float *x_half, float *x_out, uint64_t n,
             int bits, uint32_t bucket, uint64_t seed, uint64_t step,
             float *scales, uint8_t *codes);
/* orc_dcd for the window [base, base + m) of a longer model: x, x_half,
 * x_out, scales and codes hold the window's elements and buckets; base is a
 * multiple of the bucket, and Philox counters use the model's indices. */
void orc_dcd_window(const float *x, const float *x_half, float *x_out, uint64_t m, uint64_t base,
                    int bits, uint32_t bucket, uint64_t seed, uint64_t step,
                    float *scales, uint8_t *codes);

/* DCD-PSGD step 3: x_hat <- x_hat + C(z) from codes and scales. */
void orc_dcd_decode(const float *scales, const uint8_t *codes, uint64_t n, int bits,
                    uint32_t bucket, float *x_hat);

/* DCD-PSGD step 1: x_half = sum_j weights[j] * replicas[j] - lr * grad. */
void orc_dcd_mix(int K, const float *const *replicas, const float *weights, const float *grad,
                 float lr, float *x_half, uint64_t n);

/* ECD-PSGD Eq. (3): codes and scales of C((1 - t/2) x_prev + (t/2) x). */
void orc_ecd_compress(const float *x_prev, const float *x, uint64_t n, uint64_t t, int bits,
                      uint32_t bucket, uint64_t seed, float *scales, uint8_t *codes);

/* ECD-PSGD Eq. (4): x_tilde <- (1 - 2/t) x_tilde + (2/t) C(z). */
void orc_ecd_update(const float *scales, const uint8_t *codes, uint64_t n, int bits,
                    uint32_t bucket, uint64_t t, float *x_tilde);

/* Slim-DP core: per segment the k_s entries of largest S = |w| + c|g|
 * (ties to the lower index), ascending; core_val = S.  mask receives one
 * word-aligned run of ceil(n_s/32) words per segment marking the core. */
void orc_slimdp_core(const orc_seg *segs, int nseg, const float *w, const float *g, float c,
                     uint32_t *core_idx, float *core_val, uint32_t *seg_off, uint32_t *mask);

/* Slim-DP explorer: per segment the k_s non-core entries with the largest
 * Philox keys, ascending, with val = delta at them. */
void orc_slimdp_explore(const orc_seg *segs, int nseg, const float *delta, const uint32_t *mask,
                        uint64_t seed, uint64_t step, uint32_t *idx, float *val, uint32_t *seg_off);

#endif
