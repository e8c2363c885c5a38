/*
 * libgradcomp — per-step gradient compression for data-parallel training on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow these pages:
 *   [AdaComp] "AdaComp: Adaptive Residual Gradient Compression for
 *             Data-Parallel Distributed Training" (Chen et al.), the review's
 *             "Proposed method" list and Abstract.
 *   [DGC]     "Deep Gradient Compression: Reducing the Communication Bandwidth
 *             for Distributed Training" (Lin et al.), §3.1–§3.3, §5, §6 and
 *             Appendices A–D.
 *   [DCD]     "Communication Compression for Decentralized Training"
 *             (Tang et al.), DCD-PSGD steps 1–3, the signal-to-noise
 *             parameter alpha of the compression operator, and ECD-PSGD's
 *             extrapolation and estimate (Eqs. 3 and 4).
 *   [SlimDP]  "Slim-DP: A Light Communication Data Parallelism for DNN",
 *             §3 (core and explorer selection, significance, key caching)
 *             and the experimental setup (Quant-DP baseline: random
 *             quantization with buckets of 512).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every buffer argument typed as a pointer to float / uint32_t / uint8_t /
 *    uint64_t / void is a DEVICE pointer owned by the caller.  Structs and
 *    arrays documented as "host" are read during the call and not retained.
 *  - A learner's model is one flat fp32 buffer of n_total elements.  Each
 *    layer tensor is a segment of it (gc_segment).  State buffers (AdaComp
 *    residual R, DGC momentum U and accumulator V) use the same flat layout.
 *  - Argument errors are detected on the host before anything is enqueued; on
 *    error no device buffer has been touched.  Errors are returned as negative
 *    gc_status codes; gc_last_error() gives a thread-local message.
 *  - Hot calls enqueue kernels on `stream` and return without synchronising.
 *    Counts and messages land in device memory.
 *  - Hot calls never allocate device memory, with one exception: the first
 *    call that uses a plan on a device uploads the plan's tables to that
 *    device (one hipMalloc + one synchronous copy per plan and device).
 *  - Results are bitwise deterministic: every floating-point operation is a
 *    single correctly rounded IEEE operation in a fixed order (no FMA
 *    contraction), and every reduction that feeds a decision uses a fixed
 *    pairwise tree (see gc_dgc_step and gc_adacomp_compress).
 *  - Non-finite inputs have defined results.  A NaN never counts toward a
 *    maximum (an AdaComp bin's, a DCD bucket's), is never selected by
 *    AdaComp (it stays in the residual) and quantizes to level 0 in DCD.
 *    +-Inf are magnitudes above every finite one: an Inf is its bin's
 *    maximum, and a DCD bucket whose maximum is Inf sends only level 0.  DGC
 *    ranks by the magnitude bits, where a NaN ranks above +Inf.  Every other
 *    step is the IEEE operation as written; NaNs that arithmetic makes carry
 *    no guaranteed sign or payload.
 *  - Input, state and output buffers must not alias each other (except
 *    x_out == x in gc_dcd_compress).
 *  - Calls on different streams are independent as long as they use
 *    different workspaces and outputs.
 */
#ifndef GRADCOMP_H
#define GRADCOMP_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ status */
typedef int gc_status;
#define GC_OK          0
#define GC_EINVAL     -1   /* malformed argument (null pointer, bad range)   */
#define GC_ECAPACITY  -2   /* output or workspace capacity too small         */
#define GC_ERANGE     -3   /* size outside the supported range (n >= 2^32)   */
#define GC_EHIP       -4   /* a HIP runtime call failed                      */
#define GC_ENOTSUP    -5   /* valid but unsupported parameter combination    */

/* Thread-local text of the last error raised on this thread ("" if none). */
const char *gc_last_error(void);
/* Library version string, e.g. "libgradcomp 0.1.0". */
const char *gc_version(void);

/* ------------------------------------------------------------------ layout */
/*
 * One layer tensor inside the flat buffer (host struct).
 * Both methods act on each layer on its own: [AdaComp] applies the scheme
 * layer by layer; [DGC] §3.1 thresholds each gradient tensor.
 *   offset  : index of the segment's first element in the flat buffer.
 *   length  : number of elements n_s (>= 1).
 *   bin_len : AdaComp bin length L_T (>= 1, <= GC_MAX_BIN_LEN); bins restart
 *             at the segment start and the last bin may be partial.
 *   k       : DGC top-k count (1 <= k <= length).  gc_topk_count() gives the
 *             0.1%-density value ceil(n_s/1000) used by [DGC] §3.3/§4.
 */
typedef struct gc_segment {
    uint64_t offset;
    uint32_t length;
    uint32_t bin_len;
    uint32_t k;
    uint32_t reserved;   /* must be 0 */
} gc_segment;

#define GC_MAX_BIN_LEN   4096u
#define GC_MAX_MESSAGES  64
/* Longest segment, 2^32 - 2^18: a packed block of n_s elements holds up to
 * n_s + n_s / 32767 + 1 codes (an AdaComp message that sends every element,
 * plus its escapes), and that count travels as the block's u32 E. */
#define GC_MAX_SEGMENT_LEN 0xFFFC0000u

/* Opaque, immutable plan: validated segment table + device tables. */
typedef struct gc_plan gc_plan;

/*
 * Validate a segment table and build a plan.  Host only: touches no device.
 *   segs[nseg] (host) must be ascending by offset, non-overlapping, and lie in
 *   [0, n_total); n_total must be < 2^32 (indices are u32).  Gaps between
 *   segments are allowed and are never read or written.
 * Returns GC_EINVAL (bad table), GC_ERANGE (n_total >= 2^32), GC_ENOTSUP
 * (bin_len > GC_MAX_BIN_LEN or length > GC_MAX_SEGMENT_LEN).  *out is set
 * only on GC_OK.
 */
gc_status gc_plan_create(const gc_segment *segs, int nseg, uint64_t n_total,
                         gc_plan **out);
void      gc_plan_destroy(gc_plan *plan);
/* Put the plan's tables on the current device now: one hipMalloc and one
 * synchronous copy, once per plan and device (a hot call does the same on
 * its first use there).  For callers that capture a plan's first calls in a
 * HIP graph, or allocate nothing inside their hot loop.  Returns GC_OK once
 * the tables are there, GC_EINVAL for a NULL plan, GC_EHIP on a HIP error. */
gc_status gc_plan_upload(const gc_plan *plan);
int       gc_plan_num_segments(const gc_plan *plan);
uint64_t  gc_plan_num_elements(const gc_plan *plan);
/* Sum over segments of k (the DGC message size). */
uint64_t  gc_plan_total_k(const gc_plan *plan);
/* Sum over segments of ceil(length/bin_len) (AdaComp bin count). */
uint64_t  gc_plan_total_bins(const gc_plan *plan);
/* ceil(n / 1000), the per-tensor count at 99.9% sparsity. */
uint32_t  gc_topk_count(uint32_t n);

#define GC_OP_DGC      1
#define GC_OP_ADACOMP  2
#define GC_OP_PACK     3
#define GC_OP_DECODE   4
#define GC_OP_UNPACK   5
/* Device workspace bytes a hot call with this plan needs (0 if none). */
size_t gc_plan_workspace_bytes(const gc_plan *plan, int op);

/* ----------------------------------------------------------------- message */
/*
 * Sparse message (host struct whose members are device pointers).
 *   idx[cap]        : flat element indices, ascending within the message
 *                     (segments in plan order, ascending inside a segment).
 *   val[cap]        : value to add at idx — V_i for DGC, +-scale_s for AdaComp.
 *   seg_off[nseg+1] : entries of segment s are [seg_off[s], seg_off[s+1]);
 *                     seg_off[nseg] is the message's entry count.
 *   seg_scale[nseg] : AdaComp layer scale per segment (unused by DGC; may be
 *                     NULL there).
 *   cap             : capacity of idx/val in entries.
 */
typedef struct gc_sparse {
    uint32_t *idx;
    float    *val;
    uint32_t *seg_off;
    float    *seg_scale;
    uint64_t  cap;
} gc_sparse;

/* --------------------------------------------------------------- AdaComp */
/*
 * One AdaComp step for one learner ([AdaComp] "Proposed method", Abstract):
 *   a1  G_i = fl32(R_i + dW_i)                                (residual + new gradient)
 *   a2  g_max(b) = max_{i in b} |G_i|   over bins of bin_len  (exact; max is order-free)
 *   a3  sel_i  <=>  g_max(b) > 0  and  fl32(scale_factor * |G_i|) >= g_max(b)
 *       (the bin's own max always qualifies when scale_factor >= 1; 2.0 is the
 *        empirical factor the page gives)
 *   a4  scale_s = fl32( PSUM64(g_max over the segment's bins) / nbins_s )
 *       (mean of the bin maxima across the whole layer)
 *   a5  q_i = copysign(scale_s, G_i) if selected, else 0;  R_i <- fl32(G_i - q_i)
 *   a6  out: per segment, ascending idx with val = q_i; out->seg_scale[s] = scale_s.
 * PSUM64(x_0..x_{m-1}) converts each term to double, pads with +0.0 to the
 * next power of two and adds as a perfect binary tree in index order.
 *
 * Residual storage.  A learner's residual is the pair (R, state):
 *   state == NULL : R holds the exact residual before and after the call.
 *   state != NULL : deferred mode.  `state` is a caller-owned, 256-byte
 *     aligned device buffer of at least gc_adacomp_state_bytes(plan) bytes,
 *     zero-filled before the learner's first step and used with this plan
 *     only.  After a call, R holds G and the state records which entries the
 *     call sent and the layer scales; the residual of such an entry is
 *     fl32(R_i - copysign(scale_s, R_i)) (step a5, exactly), which the next
 *     call applies before a1.  R and dW then cross HBM once per step instead
 *     of twice.  Messages are identical in both modes; gc_adacomp_residual()
 *     gives the exact residual of (R, state).
 *   dW  [n_total] in,  R [n_total] in/out,
 *   out : cap >= gc_adacomp_message_cap(plan), the sum of the segment
 *         lengths (the worst case: every element sent).
 *   ws  : at least gc_plan_workspace_bytes(plan, GC_OP_ADACOMP) bytes.
 * Errors: GC_EINVAL (null pointer, scale_factor not finite or < 1, state
 *         not 256-byte aligned), GC_ECAPACITY (out->cap below
 *         gc_adacomp_message_cap, ws or state too small).
 */
gc_status gc_adacomp_compress(const gc_plan *plan, const float *dW, float *R, void *state,
                              size_t state_bytes, float scale_factor, gc_sparse *out,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The same step with the reading of the adaptive threshold chosen.  The
 * AdaComp page ("Proposed method") builds the threshold from a scale factor
 * (empirically 2x) that picks entries near the bin's max, without fixing what
 * the factor multiplies; both readings are offered, and neither is pinned by
 * the page:
 *   GC_ADACOMP_RULE_RESIDUAL (gc_adacomp_compress): step a3 above;
 *   GC_ADACOMP_RULE_GRADIENT: the factor weighs the new gradient instead,
 *     a3' H_i = fl32(G_i + fl32((scale_factor - 1) * dW_i))
 *              (for the factor 2, fl32(G_i + dW_i), i.e. R + 2 dW rounded
 *               from G)
 *         sel_i <=> g_max(b) > 0 and (|H_i| >= g_max(b) or |G_i| = g_max(b))
 *         (every entry at the bin's max is sent, as under the default).
 *   Steps a1, a2, a4-a6 and both residual modes are unchanged; an entry with
 *   G_i = +-0 that H sends gets copysign(scale_s, G_i).
 * opt: scale_factor finite and >= 1; rule one of the two; reserved zero.
 * Arguments, layouts and the other errors as gc_adacomp_compress.
 * Errors: GC_EINVAL also for a null opt, an unknown rule or nonzero
 *         reserved fields.
 */
#define GC_ADACOMP_RULE_RESIDUAL 0
#define GC_ADACOMP_RULE_GRADIENT 1
typedef struct gc_adacomp_options {
    float    scale_factor;  /* >= 1; 2.0 in the pages  */
    int      rule;          /* GC_ADACOMP_RULE_*       */
    uint32_t reserved[2];   /* must be 0               */
} gc_adacomp_options;
gc_status gc_adacomp_compress_ex(const gc_plan *plan, const float *dW, float *R, void *state,
                                 size_t state_bytes, const gc_adacomp_options *opt, gc_sparse *out,
                                 void *ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of one learner's deferred-residual state for this plan (0 if plan
 * is NULL). */
size_t gc_adacomp_state_bytes(const gc_plan *plan);

/* Slots an AdaComp message needs for this plan: the sum of the segment
 * lengths (0 if plan is NULL).  Gaps between segments need none. */
uint64_t gc_adacomp_message_cap(const gc_plan *plan);

/* R_out[n_total] <- the exact residual held by (R, state): elements outside
 * every segment are copied, in-segment elements sent in the last deferred
 * step get fl32(R_i - copysign(scale_s, R_i)).  state == NULL copies R.
 * R_out must not overlap R; R and state are not modified.
 * Errors: GC_EINVAL (null R or R_out, overlap, misaligned state),
 *         GC_ECAPACITY (state smaller than gc_adacomp_state_bytes). */
gc_status gc_adacomp_residual(const gc_plan *plan, const float *R, const void *state,
                              size_t state_bytes, float *R_out, hipStream_t stream);

/* ------------------------------------------------------------------- DGC */
/*
 * One DGC step for one learner, vanilla momentum ([DGC] §3.1–§3.3, App. C, D):
 *   a7  local clipping (App. C), only if thr_G > 0:
 *         thr = fl32(thr_G / sqrt(num_nodes))            (in double)
 *         S_s = PSUM64(G_i^2 over the segment)            (squares exact in double)
 *         c_s = fl32(thr / sqrt(S_s)) if sqrt(S_s) > thr else 1
 *       G'_i = fl32(c_s * G_i)
 *   a8  momentum correction (§3.2):  U_i <- fl32(fl32(momentum*U_i) + G'_i)
 *                                    V_i <- fl32(V_i + U_i)
 *   a9  exact top-k (§3.1, §5): key_i = bits(V_i) & 0x7FFFFFFF; the k_s entries
 *       first in the order (key descending, index ascending) are sent.
 *   a10 momentum factor masking (§3.3): at sent indices V_i <- +0, U_i <- +0.
 *   out: per segment exactly k_s entries, ascending idx, val = V_i before masking.
 *   G [n_total] in;  U, V [n_total] in/out;  out->cap >= gc_plan_total_k(plan).
 *   0 <= momentum < 1;  num_nodes >= 1;  thr_G <= 0 disables clipping.
 * Errors: GC_EINVAL, GC_ECAPACITY (out->cap or ws too small).
 */
gc_status gc_dgc_step(const gc_plan *plan, const float *G, float *U, float *V,
                      float momentum, float thr_G, int num_nodes,
                      gc_sparse *out, void *ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * DGC step with the momentum kind and the selection mode chosen.
 * gc_dgc_step(plan, G, U, V, m, thr_G, N, ...) is this call with
 * {m, thr_G, N, GC_MOMENTUM_VANILLA, GC_SELECT_EXACT}.
 *
 * Momentum correction ([DGC] §3.2, App. B, App. D):
 *   GC_MOMENTUM_VANILLA  (Alg. 3)  U_i <- fl32(fl32(m*U_i) + G'_i);  V_i <- fl32(V_i + U_i)
 *   GC_MOMENTUM_NESTEROV (Alg. 4)  U_i <- fl32(fl32(m*U_i) + G'_i);
 *                                  V_i <- fl32(V_i + fl32(fl32(m*U_i) + G'_i))  (updated U_i)
 *   Nesterov SGD steps along m*U + G with U <- m*U + G; momentum correction
 *   accumulates that step direction in V instead of applying it.  Clipping
 *   (a7) and masking (a10) are as in gc_dgc_step.
 *
 * Selection ([DGC] §3.1, §5, §6):
 *   GC_SELECT_EXACT    exactly k_s entries per segment, as in gc_dgc_step.
 *   GC_SELECT_SAMPLED  the threshold is estimated from a sample and, when it
 *     lets through far more entries than k_s, the exact top-k is taken among
 *     those (hierarchical selection).  Per segment of n entries:
 *       sample: window w = 0, 1, ... covers entries [32*P*w, 32*P*(w+1)) of
 *         the segment; its block is the 32 entries starting at
 *         32*P*w + 32*((w * 2654435769 mod 2^32) mod P), those at or past n
 *         excluded (P = sample_period: 1/P of the entries; the page samples
 *         0.1% to 1%, P = 1000 to 100).  S = number of sampled entries.
 *       estimate: thr = the r-th largest key among the sampled entries'
 *         keys (of V after a8), r = ceil(S * k_s / n).
 *       C = #{ i : key_i >= thr }.  If C <= min(n, over * k_s), those C
 *         entries are sent; otherwise the exact top k_s (as GC_SELECT_EXACT).
 *     Segments' entries are laid end to end: seg_off[s+1] - seg_off[s] is
 *     the segment's count.  The call's cost grows with S (small P is slow).
 *   out->cap >= gc_dgc_message_cap(plan, opt).
 * Errors: as gc_dgc_step; GC_EINVAL also for an unknown momentum_kind or
 *         select, sample_period outside [1, GC_MAX_SAMPLE_PERIOD] or over < 1
 *         in sampled mode, reserved != 0.
 */
#define GC_MAX_SAMPLE_PERIOD  (1u << 26)
#define GC_MOMENTUM_VANILLA   0
#define GC_MOMENTUM_NESTEROV  1
#define GC_SELECT_EXACT       0
#define GC_SELECT_SAMPLED     1
typedef struct gc_dgc_options {
    float    momentum;       /* 0 <= m < 1                                   */
    float    thr_G;          /* clip threshold of the whole job; <= 0: none  */
    int      num_nodes;      /* N >= 1                                       */
    int      momentum_kind;  /* GC_MOMENTUM_*                                */
    int      select;         /* GC_SELECT_*                                  */
    uint32_t sample_period;  /* GC_SELECT_SAMPLED: 1 <= P <= GC_MAX_SAMPLE_PERIOD */
    uint32_t over;           /* GC_SELECT_SAMPLED: budget factor >= 1        */
    uint32_t reserved;       /* must be 0                                    */
    uint32_t density_num;    /* per-call density (warm-up): with             */
    uint32_t density_den;    /* density_den > 0, k_s = clamp(ceil(n_s *     */
                             /* density_num / density_den), 1, n_s) in place */
                             /* of the plan's k; 0 < num <= den; exact only  */
} gc_dgc_options;

/* Entries a message needs for these options: sum of k_s (exact), or sum of
 * min(n_s, over * k_s) (sampled).  0 if plan is NULL. */
uint64_t  gc_dgc_message_cap(const gc_plan *plan, const gc_dgc_options *opt);
gc_status gc_dgc_step_ex(const gc_plan *plan, const float *G, float *U, float *V,
                         const gc_dgc_options *opt, gc_sparse *out, void *ws,
                         size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ pack */
/*
 * Byte-exact run-length encoding of a message ([DGC] §3.1: 32-bit values and
 * 16-bit zero-run lengths).  Little-endian; every block 4-byte aligned.
 *   stream header : u32 'GCP2', u32 kind, u32 nseg, u32 0
 *   block table   : per segment u64 offset of its block from the stream
 *                   start, u32 E, u32 entries of the segment
 *   then the blocks in segment order, the first at 16 + 16 nseg:
 *   DGC block     : u32 'DGC1', u32 n_s, u32 E, u32 entries of the segment,
 *                   u16 run[E] (+ one u16 0 if E is odd), f32 val[E],
 *                   checkpoints
 *   AdaComp block : u32 'ADC1', u32 n_s, u32 E, f32 scale_s,
 *                   u16 code[E] (+ one u16 0 if E is odd), checkpoints;
 *                   code = sign << 15 | run  (sign 1 = negative)
 *   checkpoints   : for c = 0 .. ceil(E / 4096) - 1, u32 entries and u32
 *                   reader position p (as gc_unpack defines it) before code
 *                   4096 c
 * The table and the checkpoints let a receiver read blocks and tiles of
 * 4096 codes independently.
 * A run counts the unsent elements since the previous entry of the segment
 * (from the segment start for the first).  A run >= MAX is split: emit an
 * escape (run MAX; DGC value +0.0f), subtract MAX, repeat.  MAX is 65535 for
 * DGC and 32767 for AdaComp; E counts entries plus escapes.
 *   in       : a message produced for this plan (device counts are read;
 *              a segment's entries are taken up to its length).
 *   out      : device byte buffer of out_cap >= gc_pack_bound(plan, kind),
 *              which holds any AdaComp message and any DGC message of the
 *              plan's k per segment.  A DGC message with more entries per
 *              segment (a per-call density, or the sampled selection's
 *              budget) may need up to gc_dgc_pack_bound(plan, opt) bytes.
 *   out_bytes: device u64, receives the stream length.  When it exceeds
 *              out_cap the stream did not fit: out does not hold it (no
 *              byte past out_cap is written), and the message needs a
 *              buffer of at least *out_bytes bytes (the sizes above always
 *              suffice).
 * Errors: GC_EINVAL (bad kind / null), GC_ECAPACITY (out_cap or ws too small).
 */
#define GC_KIND_DGC      1
#define GC_KIND_ADACOMP  2
uint64_t  gc_pack_bound(const gc_plan *plan, int kind);
/* Stream bytes a DGC message of these selection options needs at most: the
 * bound above with k_s replaced by the call's entries per segment (a
 * per-call density's ceil(n_s num / den), or min(n_s, over k_s) sampled).
 * opt NULL: gc_pack_bound(plan, GC_KIND_DGC).  0 if plan is NULL. */
uint64_t  gc_dgc_pack_bound(const gc_plan *plan, const gc_dgc_options *opt);
gc_status gc_pack(const gc_plan *plan, int kind, const gc_sparse *in,
                  uint8_t *out, uint64_t out_cap, uint64_t *out_bytes,
                  void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * The receiver's inverse of gc_pack: a stream (as gc_pack wrote it, for this
 * plan and kind) read back into a message for gc_decompress_accumulate.  Per
 * segment, codes are read in order from position p = 0: a code whose run is
 * MAX (DGC 0xFFFF; AdaComp 0x7FFF, sign bit ignored) advances p by MAX;
 * any other code puts an entry at segment position p + run, with val = the
 * code's f32 value (DGC) or +-scale_s by the sign bit (AdaComp), then sets
 * p to that position + 1.
 *   in       : device stream of in_bytes bytes (4-byte aligned, >= 16).
 *   out      : idx/val (ascending per segment), seg_off[nseg+1] and, for
 *              AdaComp, seg_scale[nseg].  Entries at or past out->cap are
 *              not written (seg_off is clamped to cap).
 *   status   : device u32, set to 0 for a stream that fits the plan, else a
 *              bitmask: 1 bad stream header (or too short for its table),
 *              2 a block table entry or block header that disagrees with the
 *              plan, the stream's bytes or the blocks before it (or
 *              trailing bytes): the whole stream is then read as empty,
 *              4 an entry outside its segment (not written), 8 more entries
 *              than out->cap, 16 a tile whose entries or positions disagree
 *              with the next checkpoint or the block's entry count.
 *              Whatever the stream, every write stays inside the message,
 *              inside the range seg_off gives its segment, and inside the
 *              segment's elements.
 *   ws       : gc_plan_workspace_bytes(plan, GC_OP_UNPACK) bytes.
 * One workgroup checks the table and headers; then every tile of 4096 codes
 * is read from its checkpoint, independently of the others.
 * Errors: GC_EINVAL (bad kind, null pointers, misaligned or short stream),
 *         GC_ECAPACITY (ws).
 */
gc_status gc_unpack(const gc_plan *plan, int kind, const uint8_t *in, uint64_t in_bytes,
                    gc_sparse *out, uint32_t *status, void *ws, size_t ws_bytes,
                    hipStream_t stream);

/* ---------------------------------------------------------------- decode */
/*
 * Decompress-and-aggregate K messages into a dense update ([DGC] App. A: the
 * nodes' gradients are summed; [AdaComp]: the learners' compressed gradients
 * are averaged).  For every element i of the plan's segments:
 *   S_i = +0.0f, then S_i = fl32(S_i + v_{k,i}) for k = 0..K-1 in array order
 *         over the messages that hold i;
 *   r_i = fl32(S_i / K) (GC_AVG) or S_i (GC_SUM);
 *   dense_i = r_i (accumulate == 0) or fl32(dense_i + r_i) (accumulate != 0).
 *   msgs (host array of K <= GC_MAX_MESSAGES): messages for this plan with
 *   indices inside segments and ascending.  dense [n_total] out (in/out if
 *   accumulate).  Elements in gaps between segments are not touched.
 * Errors: GC_EINVAL (K out of range, bad mode, null), GC_ECAPACITY (ws).
 */
#define GC_SUM  0
#define GC_AVG  1
gc_status gc_decompress_accumulate(const gc_plan *plan, const gc_sparse *msgs,
                                   int K, float *dense, int mode,
                                   int accumulate, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * operation and results as gc_decompress_accumulate, with no workspace
 * argument: the index pass's table (K * (chunks + 1) u32, where chunks is
 * the plan's count of 4096-element tiles) lives in a fixed 8 MiB device
 * array inside the library.  Each GPU holds its own copy until the process
 * ends.  The call allocates nothing: it looks the array's address up once per
 * device (hipGetSymbolAddress) and requires the plan's tables to be on the
 * current device already (gc_plan_upload, outside the caller's hot loop).
 * Every call on one GPU shares that GPU's array, so calls that overlap on one
 * GPU (other streams, other threads) race and give undefined results; calls
 * in one stream are ordered and safe.  Nothing in the array needs to start at
 * any value: each call writes every entry it reads.
 * gc_decompress_noalloc_max_chunks(K) is the largest plan chunk count the
 * array holds for K messages (2,097,152 / K - 1; 0 for K out of range).
 * Errors: as gc_decompress_accumulate, plus GC_ECAPACITY when the plan has
 *         more chunks than that (checked on the host) and GC_EINVAL when the
 *         plan was not uploaded to the current device.
 */
uint64_t  gc_decompress_noalloc_max_chunks(int K);
gc_status gc_decompress_accumulate_noalloc(const gc_plan *plan, const gc_sparse *msgs,
                                           int K, float *dense, int mode,
                                           int accumulate, hipStream_t stream);

/* ------------------------------------------------------------------- DCD */
/*
 * Compressed model difference with random quantization ([DCD] DCD-PSGD step 2;
 * [SlimDP] Quant-DP: buckets of 512; 8-bit and 4-bit precisions).
 *   z_i = fl32(x_half_i - x_i); buckets of `bucket` elements over [0, n).
 *   s_b = max |z_i| in bucket b -> scales[b].
 *   L = 2^(bits-1) - 1.  If s_b == 0 every code is 0 and C_i = 0.  Otherwise
 *     inv = fl32(L / s_b); y = min(L, fl32(|z_i| * inv)); l0 = floor(y);
 *     f = y - l0; r = word (i mod 4) of Philox4x32-10(key = (seed lo, seed hi),
 *     counter = (lo(i/4), hi(i/4), lo(step), hi(step))); u = (r >> 8) * 2^-24;
 *     l = l0 + (u < f); C_i = +-fl32(l * fl32(s_b / L)) with the sign of z_i.
 *   code_i = l == 0 ? 0 : (sign << (bits-1)) | l.  4-bit codes are packed two
 *   per byte, even index in the low nibble; 8-bit codes one per byte.
 *   x_out_i = fl32(x_i + C_i)  (x_out may equal x: step 2's local update).
 *   scales [ceil(n/bucket)], codes [ceil(n*bits/8)] out.
 *   codes must be 4-byte aligned.
 * Errors: GC_EINVAL (bits not 4 or 8, bucket 0, null, misaligned codes),
 *         GC_ENOTSUP (bucket not a power of two in [4, 4096]),
 *         GC_ERANGE (n > 2^32 - 8192).
 */
gc_status gc_dcd_compress(const float *x, const float *x_half, float *x_out,
                          uint64_t n, int bits, uint32_t bucket, uint64_t seed,
                          uint64_t step, float *scales, uint8_t *codes,
                          hipStream_t stream);

/*
 * DCD-PSGD step 3 ([DCD] step 3): a neighbour's replica advances by the
 * received compressed difference, x_hat_i <- fl32(x_hat_i + C_i), with C_i
 * decoded from the stream gc_dcd_compress wrote:
 *   code_i = codes[i] (8 bits) or nibble i%2 of codes[i/2] (4 bits, even i in
 *   the low nibble); level = code & L, L = 2^(bits-1) - 1; sign = bit bits-1;
 *   C_i = level == 0 ? 0 : +-fl32(level * fl32(scales[i/bucket] / L)).
 * Applied to a copy of x_t this reproduces gc_dcd_compress's x_out bit for
 * bit, so every replica stays equal to its node's model.
 *   scales [ceil(n/bucket)], codes [ceil(n*bits/8)] in (codes 4-byte aligned);
 *   x_hat [n] in/out.
 * Errors: GC_EINVAL (null, bits not 4 or 8, bucket 0, misaligned codes),
 *         GC_ENOTSUP (bucket not a power of two in [4, 4096]),
 *         GC_ERANGE (n > 2^32 - 8192).
 */
gc_status gc_dcd_decode(const float *scales, const uint8_t *codes, uint64_t n, int bits,
                        uint32_t bucket, float *x_hat, hipStream_t stream);

/*
 * DCD-PSGD step 1 ([DCD] step 1): the weighted average of the replicas (the
 * node's own model among them) and a stochastic gradient step:
 *   S_i = +0, then S_i = fl32(S_i + fl32(weights[j] * replicas[j][i])) for
 *         j = 0..K-1 in array order;
 *   x_half_i = fl32(S_i - fl32(lr * grad_i)).
 *   replicas (host array of K device pointers, 1 <= K <= GC_MAX_REPLICAS),
 *   weights (host array of K: row i of the mixing matrix W), grad [n] in,
 *   x_half [n] out (must not alias grad or a replica).
 * Errors: GC_EINVAL (null, K out of range, aliasing), GC_ERANGE (n > 2^32 - 8192).
 */
#define GC_MAX_REPLICAS 16
gc_status gc_dcd_mix(const float *const *replicas, const float *weights, int K,
                     const float *grad, float lr, float *x_half, uint64_t n,
                     hipStream_t stream);

/*
 * ECD-PSGD sender ([DCD] ECD-PSGD, Eq. 3): the extrapolated value
 *   z_i = fl32(fl32(a * x_prev_i) + fl32(b * x_i)),  a = fl32(1 - t/2), b = fl32(t/2)
 * (coefficients formed in double), quantized exactly as gc_dcd_compress
 * quantizes z (same code layout and scales) with Philox step = t.
 *   x_prev = x_{t-1}, x = x_t [n] in; t >= 1; scales, codes out.
 * Errors: as gc_dcd_decode; GC_EINVAL also for t = 0.
 */
gc_status gc_ecd_compress(const float *x_prev, const float *x, uint64_t n, uint64_t t,
                          int bits, uint32_t bucket, uint64_t seed, float *scales,
                          uint8_t *codes, hipStream_t stream);

/*
 * ECD-PSGD receiver ([DCD] ECD-PSGD, Eq. 4): the estimate of a neighbour's
 * model, x_tilde_i <- fl32(fl32(c1 * x_tilde_i) + fl32(c2 * C_i)) with
 * c1 = fl32(1 - 2/t), c2 = fl32(2/t) (formed in double), C_i decoded as in
 * gc_dcd_decode.  t >= 1.
 * Errors: as gc_dcd_decode; GC_EINVAL also for t = 0.
 */
gc_status gc_ecd_update(const float *scales, const uint8_t *codes, uint64_t n, int bits,
                        uint32_t bucket, uint64_t t, float *x_tilde, hipStream_t stream);

/* ---------------------------------------------------------------- Slim-DP */
/*
 * Slim-DP's communication set ([SlimDP] §3: a core of significant parameters
 * chosen by the server, plus an explorer of random parameters from outside
 * the core chosen by each worker at every communication).
 *
 * Core:  S_i = fl32(|w_i| + fl32(c * |g_i|)), c > 0 (the page combines the
 *   magnitudes of the parameter and of its gradient as a weighted sum with a
 *   positive coefficient; its equation is not printed).  Per segment, the k_s
 *   entries first in the order (S descending, index ascending) form the core
 *   (k_s from `plan`, e.g. ceil(beta * n_s)).
 *     core      : ascending idx, val = S_i; exactly sum(k_s) entries.
 *     core_mask : gc_slimdp_mask_words(plan) u32 words out: per segment a run
 *                 of ceil(n_s/32) words, bit j%32 of word j/32 set iff entry j
 *                 of the segment is in the core.
 * Explorer: per segment, the m_s non-core entries first in the order (key
 *   descending, index ascending), key_j = r >> 1 | 1 with r = word j%4 of
 *   Philox4x32-10(counter (j/4, s, lo(step), hi(step)), key (lo(seed),
 *   hi(seed))) for entry j of segment s; core entries never qualify.  A
 *   uniformly random set of m_s non-core entries, resampled with `step`.
 *     plan      : the same segments as core_plan with k_s = m_s, and
 *                 m_s + (core k_s) <= n_s.
 *     out       : ascending idx, val = delta_i; exactly sum(m_s) entries.
 * Core values: the core's keys are cached on both sides ([SlimDP] key caching
 *   filter), so a push sends only values: values[j] = delta[core->idx[j]]
 *   for j < gc_plan_total_k(core_plan) (core as gc_slimdp_core wrote it;
 *   indices at or past n_total are clamped to the last element).
 * Workspaces: gc_plan_workspace_bytes(plan, GC_OP_DGC).
 * Errors: GC_EINVAL (null, c not positive and finite, plans that differ in
 *         segments, core + explorer above a segment), GC_ECAPACITY.
 */
uint64_t  gc_slimdp_mask_words(const gc_plan *plan);
gc_status gc_slimdp_core(const gc_plan *plan, const float *w, const float *g, float c,
                         gc_sparse *core, uint32_t *core_mask, void *ws, size_t ws_bytes,
                         hipStream_t stream);
gc_status gc_slimdp_explore(const gc_plan *plan, const gc_plan *core_plan, const float *delta,
                            const uint32_t *core_mask, uint64_t seed, uint64_t step,
                            gc_sparse *out, void *ws, size_t ws_bytes, hipStream_t stream);
gc_status gc_slimdp_core_values(const gc_plan *core_plan, const gc_sparse *core,
                                const float *delta, float *values, hipStream_t stream);

/* ----------------------------------------------------------- measurement */
/*
 * Kernel timing for measurement tools (off by default).  While enabled, each
 * launch of a selected kernel is bracketed by a pair of HIP events recorded
 * on the caller's stream; nothing else changes.
 *   kernels : comma-separated kernel names ("dgc_update,ada_apply"), "*" for
 *             all, NULL or "" to disable.  Names: dgc_norm, dgc_prep,
 *             dgc_sample, dgc_bound, dgc_ssample, dgc_squant, dgc_update,
 *             dgc_select, dgc_stage, dgc_refine, dgc_sbase, dgc_count,
 *             dgc_scan, dgc_emit, ada_max, ada_binsum, ada_scale, ada_offsets,
 *             ada_apply, ada_fold, ada_emit, ada_residual,
 *             pack_tiles, pack_count, pack_layout, pack_write, unpack_walk,
 *             unpack_count, unpack_scan, unpack_write, decode_index,
 *             decode, dcd, dcd_decode, dcd_mix, ecd_compress, ecd_update,
 *             slimdp_values, stream_probe (Slim-DP selection reuses the
 *             dgc_* names).
 * gc_timing_take waits for the recorded events of one kernel and returns the
 * summed duration in milliseconds and the number of launches, then forgets
 * them.  Host-thread safe; not for use while a stream is being captured.
 */
gc_status gc_timing_enable(const char *kernels);
gc_status gc_timing_take(const char *kernel, double *total_ms, uint64_t *launches);

/*
 * A streaming reference for measurement tools, not part of any method:
 * d[i] = a[i] + b[i] and e[i] = c[i] + d[i] (fp32) for i < n, that is three
 * reads and two writes per element, the HBM traffic of the DGC update, in
 * the same chunk tiling, lane layout and cache hints as the dense kernels
 * and with none of their other work.  Timed beside dgc_update it gives the
 * bandwidth that access pattern reaches on the device.
 *   a, b, c : device, n floats each, read.   d, e : device, n floats each,
 *             written; they must not overlap each other or the inputs.
 *   n       : below 2^32; 0 enqueues nothing.
 * All pointers 4-byte aligned.  Errors (GC_EINVAL null or misaligned
 * pointer, GC_ERANGE n) are detected before anything is enqueued.
 * Asynchronous on `stream`.
 */
gc_status gc_stream_probe(const float *a, const float *b, const float *c, float *d, float *e, uint64_t n,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GRADCOMP_H */
