/*
 * Oracle for libgradcomp — TEST INFRASTRUCTURE ONLY (see oracle.h).
 *
 * Plain loops in the order the pages describe the steps.  Library routines
 * used as steps: qsort (ordering for top-k), sqrt, copysignf, floorf.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------ pairwise sum */
/* Node [lo, lo+len) of the perfect binary tree over the zero-padded terms.
 * A node that lies wholly in the padding is a sum of +0.0 terms, i.e. +0.0. */
static double psum_node(const double *x, uint64_t m, uint64_t lo, uint64_t len)
{
    if (lo >= m) return 0.0;
    if (len == 1) return x[lo];
    uint64_t h = len / 2;
    double left = psum_node(x, m, lo, h);
    double right = psum_node(x, m, lo + h, h);
    return left + right;
}

double orc_psum64(const double *x, uint64_t m)
{
    if (m == 0) return 0.0;
    uint64_t M = 1;
    while (M < m) M <<= 1;
    return psum_node(x, m, 0, M);
}

/* ----------------------------------------------------------------- AdaComp */
/*
 * AdaComp (Chen et al.), "Proposed method":
 *  - the layer's residual plus the new gradient is split into fixed-size bins
 *    of L_T and each bin's max magnitude marks its important entries;
 *  - inside a bin, the max and its neighbours that pass an adaptive threshold
 *    (a scale factor, empirically 2x) are selected;
 *  - selected entries are quantized to sign times one layer-wide scale, the
 *    mean of the bins' |g_max|;
 *  - what is not sent stays in the residual (residual gradient compression,
 *    Abstract); layers are treated independently.
 */
/*
 * Two readings of the adaptive threshold (the pages do not fix which one is
 * meant; neither is pinned by them):
 *  rule 0 (the default): the scale factor s multiplies the accumulated
 *    residual G = R + dW; entry i is sent when g_max(bin) > 0 and
 *    fl(s |G_i|) >= g_max(bin);
 *  rule 1: the factor weighs the new gradient instead, H = R + s dW, formed
 *    from G as H_i = fl(G_i + fl((s - 1) dW_i)) (for s = 2, fl(G_i + dW_i));
 *    entry i is sent when g_max(bin) > 0 and |H_i| >= g_max(bin), and every
 *    entry with |G_i| = g_max(bin) is sent as well (the bin's max always is).
 * Everything else (bin maxima of |G|, the layer scale, sign times scale, the
 * residual G - q) is the same under both.
 */
static void adacomp_segment(const orc_seg *sg, const float *dW, float *R,
                            float s, int rule, uint32_t *idx, float *val,
                            uint32_t *count, float *scale_out, float *gmax_out)
{
    const uint64_t base = sg->offset;
    const uint32_t n = sg->length, L = sg->bin_len;
    const uint32_t nb = (n + L - 1) / L;
    float *G = (float *)malloc(sizeof(float) * (size_t)n);
    float *gmax = (float *)malloc(sizeof(float) * (size_t)nb);
    double *gm64 = (double *)malloc(sizeof(double) * (size_t)nb);

    /* residual + gradient */
    for (uint32_t i = 0; i < n; ++i) G[i] = R[base + i] + dW[base + i];

    /* bin maxima; bins restart at the segment start, the last may be short;
     * a NaN never compares greater, so it does not count toward a maximum */
    for (uint32_t b = 0; b < nb; ++b) {
        float mx = 0.0f;
        uint32_t lo = b * L, hi = lo + L < n ? lo + L : n;
        for (uint32_t i = lo; i < hi; ++i) {
            float a = fabsf(G[i]);
            if (a > mx) mx = a;
        }
        gmax[b] = mx;
        gm64[b] = (double)mx;
    }

    /* layer scale: mean of the bin maxima over the whole layer */
    double total = orc_psum64(gm64, nb);
    float scale = (float)(total / (double)nb);

    /* selection, quantization, new residual */
    uint32_t c = 0;
    const float s1 = s - 1.0f;
    for (uint32_t i = 0; i < n; ++i) {
        float g = G[i];
        float gm = gmax[i / L];
        int send;
        if (rule == 0) {
            float t = s * fabsf(g);
            send = gm > 0.0f && t >= gm;
        } else {
            float h = g + s1 * dW[base + i];
            send = gm > 0.0f && (fabsf(h) >= gm || fabsf(g) >= gm);
        }
        if (send) {
            float q = copysignf(scale, g);
            R[base + i] = g - q;
            idx[c] = (uint32_t)(base + i);
            val[c] = q;
            ++c;
        } else {
            R[base + i] = g;
        }
    }
    *count = c;
    *scale_out = scale;
    if (gmax_out) memcpy(gmax_out, gmax, sizeof(float) * (size_t)nb);
    free(G);
    free(gmax);
    free(gm64);
}

void orc_adacomp(const orc_seg *segs, int nseg, const float *dW, float *R,
                 float scale_factor, uint32_t *out_idx, float *out_val,
                 uint32_t *seg_off, float *seg_scale, float *gmax_out)
{
    orc_adacomp_rule(segs, nseg, dW, R, scale_factor, 0, out_idx, out_val, seg_off, seg_scale, gmax_out);
}

void orc_adacomp_rule(const orc_seg *segs, int nseg, const float *dW, float *R,
                      float scale_factor, int rule, uint32_t *out_idx, float *out_val,
                      uint32_t *seg_off, float *seg_scale, float *gmax_out)
{
    /* segment s may emit up to n_s entries; stage each at its own offset */
    uint64_t *stage_at = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)(nseg + 1));
    uint64_t *bin_at = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)(nseg + 1));
    stage_at[0] = 0;
    bin_at[0] = 0;
    for (int s = 0; s < nseg; ++s) {
        stage_at[s + 1] = stage_at[s] + segs[s].length;
        bin_at[s + 1] = bin_at[s] + (segs[s].length + segs[s].bin_len - 1) / segs[s].bin_len;
    }
    uint64_t ntot = stage_at[nseg];
    uint32_t *sidx = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(ntot ? ntot : 1));
    float *sval = (float *)malloc(sizeof(float) * (size_t)(ntot ? ntot : 1));
    uint32_t *cnt = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(nseg ? nseg : 1));

#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < nseg; ++s)
        adacomp_segment(&segs[s], dW, R, scale_factor, rule, sidx + stage_at[s],
                        sval + stage_at[s], &cnt[s], &seg_scale[s],
                        gmax_out ? gmax_out + bin_at[s] : NULL);

    uint32_t pos = 0;
    for (int s = 0; s < nseg; ++s) {
        seg_off[s] = pos;
        memcpy(out_idx + pos, sidx + stage_at[s], sizeof(uint32_t) * cnt[s]);
        memcpy(out_val + pos, sval + stage_at[s], sizeof(float) * cnt[s]);
        pos += cnt[s];
    }
    seg_off[nseg] = pos;
    free(stage_at);
    free(bin_at);
    free(sidx);
    free(sval);
    free(cnt);
}

/* --------------------------------------------------------------------- DGC */
typedef struct keyed {
    uint32_t key;
    uint32_t pos;
} keyed;

/* order: larger key first; equal keys by smaller position */
static int by_key_desc_pos_asc(const void *a, const void *b)
{
    const keyed *x = (const keyed *)a, *y = (const keyed *)b;
    if (x->key != y->key) return x->key > y->key ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

static int u32_asc(const void *a, const void *b)
{
    uint32_t x = *(const uint32_t *)a, y = *(const uint32_t *)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

static uint32_t abs_bits(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    return u & 0x7FFFFFFFu;
}

/*
 * Deep Gradient Compression (Lin et al.), per gradient tensor:
 *  - App. C: the current gradient is clipped by its L2 norm before it is
 *    added to the accumulation; the node's threshold is thr_G * N^-1/2;
 *  - §3.2 / App. B, D: momentum correction accumulates the momentum-adjusted
 *    gradient into V before sparsification.  Vanilla momentum (Alg. 3):
 *    U <- m U + G, V <- V + U.  Nesterov momentum (Alg. 4, App. B): the
 *    conventional Nesterov step direction is m U + G with U <- m U + G, and
 *    it is that direction which is accumulated: V <- V + (m U + G);
 *  - §3.1 / §5: only the largest entries of V (top 0.1%) are sent, the rest
 *    keep accumulating locally;
 *  - §5 / §6 (sampled selection): the threshold is estimated from a sample of
 *    the entries, and when the estimate passes far more entries than the
 *    target, the exact threshold is taken among those already selected
 *    (hierarchical selection);
 *  - §3.3: momentum factor masking clears U (and V) where entries were sent.
 */
static uint32_t sample_block_offset(uint32_t w, uint32_t P)
{
    uint32_t h = w * 2654435769u; /* Fibonacci hashing of the window index, mod 2^32 */
    return 32u * (h % P);
}

static void dgc_segment(const orc_seg *sg, const float *Gin, float *U, float *V,
                        const orc_dgc_opts *o, uint32_t *idx, float *val,
                        uint32_t *count, float *clip)
{
    const uint64_t base = sg->offset;
    const uint32_t n = sg->length, k = sg->k;
    const float m = o->momentum;

    float c = 1.0f;
    if (o->thr_G > 0.0f) {
        float thr = (float)((double)o->thr_G / sqrt((double)o->num_nodes));
        double *sq = (double *)malloc(sizeof(double) * (size_t)n);
        for (uint32_t i = 0; i < n; ++i) {
            double g = (double)Gin[base + i];
            sq[i] = g * g; /* exact: a 24-bit mantissa squared fits in 53 bits */
        }
        double norm = sqrt(orc_psum64(sq, n));
        free(sq);
        if (norm > (double)thr) c = (float)((double)thr / norm);
    }
    *clip = c;

    for (uint32_t i = 0; i < n; ++i) {
        float g = c * Gin[base + i];
        float u = m * U[base + i];
        u = u + g;
        U[base + i] = u;
        if (o->nesterov) {
            float d = m * u;
            d = d + g;
            V[base + i] = V[base + i] + d;
        } else {
            V[base + i] = V[base + i] + u;
        }
    }

    keyed *order = (keyed *)malloc(sizeof(keyed) * (size_t)n);
    for (uint32_t i = 0; i < n; ++i) {
        order[i].key = abs_bits(V[base + i]);
        order[i].pos = i;
    }
    qsort(order, n, sizeof(keyed), by_key_desc_pos_asc);

    /* how many of the ordered entries are sent */
    uint32_t nsend = k;
    if (o->sampled) {
        const uint32_t P = o->sample_period;
        const uint64_t win = 32ull * P;
        const uint64_t nwin = (n + win - 1) / win;
        uint32_t *skeys = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(nwin * 32));
        uint64_t S = 0;
        for (uint64_t w = 0; w < nwin; ++w) {
            uint64_t p0 = w * win + sample_block_offset((uint32_t)w, P);
            for (uint32_t l = 0; l < 32; ++l)
                if (p0 + l < n) skeys[S++] = abs_bits(V[base + p0 + l]);
        }
        /* the r-th largest sample key, r = ceil(S k / n): the sample's
         * estimate of the k-th largest key of the whole tensor */
        uint64_t r = (S * k + n - 1) / n;
        qsort(skeys, (size_t)S, sizeof(uint32_t), u32_asc);
        uint32_t thr = skeys[S - r];
        free(skeys);
        uint32_t passed = 0; /* entries at or above the estimate */
        while (passed < n && order[passed].key >= thr) ++passed;
        uint64_t budget = (uint64_t)o->over * k;
        if (budget > n) budget = n;
        nsend = passed <= budget ? passed : k; /* else: exact top-k among them */
    }

    uint32_t *chosen = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(nsend ? nsend : 1));
    for (uint32_t j = 0; j < nsend; ++j) chosen[j] = order[j].pos;
    qsort(chosen, nsend, sizeof(uint32_t), u32_asc);
    for (uint32_t j = 0; j < nsend; ++j) {
        uint64_t e = base + chosen[j];
        idx[j] = (uint32_t)e;
        val[j] = V[e];
        V[e] = 0.0f;
        U[e] = 0.0f;
    }
    *count = nsend;
    free(chosen);
    free(order);
}

void orc_dgc_ex(const orc_seg *segs, int nseg, const float *G, float *U, float *V,
                const orc_dgc_opts *opts, uint32_t *out_idx, float *out_val,
                uint32_t *seg_off, float *clip_out)
{
    /* segment s stages its entries at its own slot range, at most
     * min(n_s, over k_s) of them (k_s in exact mode) */
    uint64_t *slot = (uint64_t *)malloc(sizeof(uint64_t) * (size_t)(nseg + 1));
    slot[0] = 0;
    for (int s = 0; s < nseg; ++s) {
        uint64_t cap = segs[s].k;
        if (opts->sampled) {
            cap = (uint64_t)opts->over * segs[s].k;
            if (cap > segs[s].length) cap = segs[s].length;
        }
        slot[s + 1] = slot[s] + cap;
    }
    uint64_t tot = slot[nseg];
    uint32_t *sidx = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(tot ? tot : 1));
    float *sval = (float *)malloc(sizeof(float) * (size_t)(tot ? tot : 1));
    uint32_t *cnt = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(nseg ? nseg : 1));
    float *clip = (float *)malloc(sizeof(float) * (size_t)(nseg ? nseg : 1));
#pragma omp parallel for schedule(dynamic, 1)
    for (int s = 0; s < nseg; ++s)
        dgc_segment(&segs[s], G, U, V, opts, sidx + slot[s], sval + slot[s], &cnt[s], &clip[s]);
    uint32_t pos = 0;
    for (int s = 0; s < nseg; ++s) {
        seg_off[s] = pos;
        memcpy(out_idx + pos, sidx + slot[s], sizeof(uint32_t) * cnt[s]);
        memcpy(out_val + pos, sval + slot[s], sizeof(float) * cnt[s]);
        pos += cnt[s];
    }
    seg_off[nseg] = pos;
    if (clip_out) memcpy(clip_out, clip, sizeof(float) * (size_t)nseg);
    free(slot);
    free(sidx);
    free(sval);
    free(cnt);
    free(clip);
}

void orc_dgc(const orc_seg *segs, int nseg, const float *G, float *U, float *V,
             float momentum, float thr_G, int num_nodes, uint32_t *out_idx,
             float *out_val, uint32_t *seg_off, float *clip_out)
{
    orc_dgc_opts o;
    memset(&o, 0, sizeof o);
    o.momentum = momentum;
    o.thr_G = thr_G;
    o.num_nodes = num_nodes;
    orc_dgc_ex(segs, nseg, G, U, V, &o, out_idx, out_val, seg_off, clip_out);
}

/* -------------------------------------------------------------------- pack */
/*
 * DGC §3.1: the encoder stores 32-bit values and 16-bit zero-run lengths.
 * Layout (little-endian, 4-byte aligned blocks) as documented with gc_pack:
 * stream header, a table with each block's offset, codes and entries, then
 * the blocks in segment order, each with a checkpoint (entries and reader
 * position before the code) at every 4096th code.
 */
static void put_u32(uint8_t *p, uint32_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
    p[2] = (uint8_t)(v >> 16);
    p[3] = (uint8_t)(v >> 24);
}

static void put_u64(uint8_t *p, uint64_t v)
{
    put_u32(p, (uint32_t)v);
    put_u32(p + 4, (uint32_t)(v >> 32));
}

static void put_u16(uint8_t *p, uint16_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
}

static void put_f32(uint8_t *p, float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    put_u32(p, u);
}

#define ORC_MAGIC(a, b, c, d) \
    ((uint32_t)(a) | (uint32_t)(b) << 8 | (uint32_t)(c) << 16 | (uint32_t)(d) << 24)
#define ORC_CKPT 4096u /* codes between checkpoints */

/* Bytes of a block of E codes. */
static uint64_t block_size(int kind, uint64_t E)
{
    return 16 + 2 * E + 2 * (E % 2) + (kind == 1 ? 4 * E : 0) + 8 * ((E + ORC_CKPT - 1) / ORC_CKPT);
}

/* Codes (entries plus escapes) of segment s's entries. */
static uint64_t seg_codes(const orc_seg *sg, const uint32_t *idx, uint32_t j0, uint32_t j1, uint32_t MAX)
{
    uint64_t E = 0, p = 0;
    for (uint32_t j = j0; j < j1; ++j) {
        uint64_t rel = idx[j] - sg->offset;
        E += (rel - p) / MAX + 1;
        p = rel + 1;
    }
    return E;
}

uint64_t orc_pack(int kind, const orc_seg *segs, int nseg,
                  const uint32_t *idx, const float *val,
                  const uint32_t *seg_off, const float *seg_scale,
                  uint8_t *out, uint64_t cap)
{
    const uint32_t MAX = kind == 1 ? 65535u : 32767u;
    /* first pass: the stream length */
    uint64_t total = 16 + 16 * (uint64_t)nseg;
    for (int s = 0; s < nseg; ++s)
        total += block_size(kind, seg_codes(&segs[s], idx, seg_off[s], seg_off[s + 1], MAX));
    if (total > cap) return 0;

    put_u32(out, ORC_MAGIC('G', 'C', 'P', '2'));
    put_u32(out + 4, (uint32_t)kind);
    put_u32(out + 8, (uint32_t)nseg);
    put_u32(out + 12, 0);
    uint64_t at = 16 + 16 * (uint64_t)nseg;
    for (int s = 0; s < nseg; ++s) {
        const uint64_t E = seg_codes(&segs[s], idx, seg_off[s], seg_off[s + 1], MAX);
        const uint32_t cnt = seg_off[s + 1] - seg_off[s];
        uint8_t *tab = out + 16 + 16 * (uint64_t)s;
        put_u64(tab, at);
        put_u32(tab + 8, (uint32_t)E);
        put_u32(tab + 12, cnt);
        uint8_t *w = out + at;
        put_u32(w, kind == 1 ? ORC_MAGIC('D', 'G', 'C', '1') : ORC_MAGIC('A', 'D', 'C', '1'));
        put_u32(w + 4, segs[s].length);
        put_u32(w + 8, (uint32_t)E);
        if (kind == 1)
            put_u32(w + 12, cnt);
        else
            put_f32(w + 12, seg_scale[s]);
        uint8_t *runs = w + 16;
        uint8_t *vals = runs + 2 * E + 2 * (E % 2);
        uint8_t *ckpt = vals + (kind == 1 ? 4 * E : 0);
        /* e: codes written; pr: the reader's position before the next code;
           done: entries written */
        uint64_t e = 0, pr = 0;
        uint32_t done = 0;
        for (uint32_t j = seg_off[s]; j < seg_off[s + 1]; ++j) {
            uint64_t rel = idx[j] - segs[s].offset;
            uint64_t gap = rel - pr;
            while (gap >= MAX) { /* escape: skip MAX positions, carry nothing */
                if (e % ORC_CKPT == 0) {
                    put_u32(ckpt + 8 * (e / ORC_CKPT), done);
                    put_u32(ckpt + 8 * (e / ORC_CKPT) + 4, (uint32_t)pr);
                }
                put_u16(runs + 2 * e, (uint16_t)MAX);
                if (kind == 1) put_f32(vals + 4 * e, 0.0f);
                ++e;
                pr += MAX;
                gap -= MAX;
            }
            if (e % ORC_CKPT == 0) {
                put_u32(ckpt + 8 * (e / ORC_CKPT), done);
                put_u32(ckpt + 8 * (e / ORC_CKPT) + 4, (uint32_t)pr);
            }
            if (kind == 1) {
                put_u16(runs + 2 * e, (uint16_t)gap);
                put_f32(vals + 4 * e, val[j]);
            } else {
                uint16_t sign = signbit(val[j]) ? 0x8000u : 0u;
                put_u16(runs + 2 * e, (uint16_t)(sign | gap));
            }
            ++e;
            ++done;
            pr = rel + 1;
        }
        if (E % 2) put_u16(runs + 2 * E, 0);
        at += block_size(kind, E);
    }
    return at;
}

/* ------------------------------------------------------------------ unpack */
/*
 * The receiver's side of the DGC §3.1 encoder: the stream read back into a
 * message.  A segment's entries come in code order; a code's run counts the
 * unsent elements before its entry, an escape (DGC run 0xFFFF, AdaComp run
 * 0x7FFF) skips that many elements and carries no entry.  AdaComp entries take
 * +-scale by their sign bit.  Returns 0, or nonzero for a stream that does not
 * fit the plan: 1 bad stream header, or a table entry that is not where the
 * blocks lie; 2 bad block header or size, or trailing bytes; 3 an entry outside
 * its segment; 4 more entries than cap; 5 entries or positions that disagree
 * with the table, the DGC header count or a checkpoint.
 */
static uint32_t get_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | (uint32_t)p[1] << 8 | (uint32_t)p[2] << 16 | (uint32_t)p[3] << 24;
}

static uint64_t get_u64(const uint8_t *p)
{
    return (uint64_t)get_u32(p) | (uint64_t)get_u32(p + 4) << 32;
}

int orc_unpack(int kind, const orc_seg *segs, int nseg, const uint8_t *buf, uint64_t nbytes,
               uint32_t *idx, float *val, uint32_t *seg_off, float *seg_scale, uint64_t cap)
{
    const uint64_t head = 16 + 16 * (uint64_t)nseg;
    if (nbytes < head || get_u32(buf) != ORC_MAGIC('G', 'C', 'P', '2') || get_u32(buf + 4) != (uint32_t)kind ||
        get_u32(buf + 8) != (uint32_t)nseg || get_u32(buf + 12) != 0)
        return 1;
    const uint32_t MAX = kind == 1 ? 65535u : 32767u;
    const uint32_t bmagic = kind == 1 ? ORC_MAGIC('D', 'G', 'C', '1') : ORC_MAGIC('A', 'D', 'C', '1');
    uint64_t at = head, out = 0;
    for (int s = 0; s < nseg; ++s) {
        seg_off[s] = (uint32_t)out;
        const uint8_t *tab = buf + 16 + 16 * (uint64_t)s;
        if (get_u64(tab) != at) return 1;
        if (at + 16 > nbytes || get_u32(buf + at) != bmagic || get_u32(buf + at + 4) != segs[s].length)
            return 2;
        uint64_t E = get_u32(buf + at + 8);
        uint32_t w3 = get_u32(buf + at + 12);
        if (get_u32(tab + 8) != E) return 2;
        const uint32_t cnt = get_u32(tab + 12);
        uint64_t size = block_size(kind, E);
        if (at + size > nbytes) return 2;
        float scale;
        memcpy(&scale, &w3, sizeof scale);
        seg_scale[s] = kind == 1 ? 0.0f : scale;
        const uint8_t *runs = buf + at + 16;
        const uint8_t *vals = runs + 2 * E + 2 * (E % 2);
        const uint8_t *ckpt = vals + (kind == 1 ? 4 * E : 0);
        uint64_t p = 0, count = 0;
        for (uint64_t e = 0; e < E; ++e) {
            if (e % ORC_CKPT == 0 &&
                (get_u32(ckpt + 8 * (e / ORC_CKPT)) != count || get_u32(ckpt + 8 * (e / ORC_CKPT) + 4) != p))
                return 5;
            uint32_t code = (uint32_t)runs[2 * e] | (uint32_t)runs[2 * e + 1] << 8;
            uint32_t run = kind == 1 ? code : (code & 0x7FFFu);
            if (run == MAX) {
                p += MAX;
                continue;
            }
            uint64_t rel = p + run;
            if (rel >= segs[s].length) return 3;
            if (out >= cap) return 4;
            idx[out] = (uint32_t)(segs[s].offset + rel);
            if (kind == 1) {
                uint32_t u = get_u32(vals + 4 * e);
                memcpy(&val[out], &u, sizeof u);
            } else {
                val[out] = (code & 0x8000u) ? -scale : scale;
            }
            ++out;
            ++count;
            p = rel + 1;
        }
        if (count != cnt || (kind == 1 && count != w3)) return 5;
        at += size;
    }
    seg_off[nseg] = (uint32_t)out;
    return at == nbytes ? 0 : 2;
}

/* ------------------------------------------------------------------ decode */
/*
 * DGC App. A: the nodes' gradients are summed; AdaComp: the learners'
 * compressed gradients are averaged.  Messages are added in array order.
 */
void orc_decode(const orc_seg *segs, int nseg, int K,
                const uint32_t *const *idx, const float *const *val,
                const uint64_t *count, float *dense, int mode, int accumulate)
{
    uint64_t n = 0;
    for (int s = 0; s < nseg; ++s) {
        uint64_t end = segs[s].offset + segs[s].length;
        if (end > n) n = end;
    }
    float *S = (float *)calloc(n ? n : 1, sizeof(float)); /* all +0.0f */
    for (int k = 0; k < K; ++k)
        for (uint64_t j = 0; j < count[k]; ++j) S[idx[k][j]] = S[idx[k][j]] + val[k][j];
    for (int s = 0; s < nseg; ++s) {
        for (uint32_t i = 0; i < segs[s].length; ++i) {
            uint64_t e = segs[s].offset + i;
            float r = mode == 1 ? S[e] / (float)K : S[e];
            dense[e] = accumulate ? dense[e] + r : r;
        }
    }
    free(S);
}

/* -------------------------------------------------------------- Philox4x32 */
/*
 * Philox4x32-10, from Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
 * as easy as 1, 2, 3" (SC'11): ten rounds of two 32x32->64 multiplies with the
 * round key added (Weyl sequence) between rounds.
 */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* --------------------------------------------------------------------- DCD */
/*
 * Random quantization C(z) of a flat vector (the compression operator of
 * DCD-PSGD and ECD-PSGD; the page allows random quantization or random
 * sparsification; Slim-DP's Quant-DP setting uses buckets of 512) at 8 or 4
 * bits: unbiased stochastic rounding to a uniform grid whose top level is the
 * bucket's max magnitude.  C_out[i] receives C(z)_i.
 */
/* Random quantization of z[0..n), element i being element base + i of the
 * model (base a multiple of the bucket): buckets and the Philox counter
 * follow the model's indices. */
static void quantize(const float *z, uint64_t n, uint64_t base, int bits, uint32_t bucket,
                     uint64_t seed, uint64_t step, float *scales, uint8_t *codes, float *C_out)
{
    const uint32_t L = (1u << (bits - 1)) - 1u;
    const float Lf = (float)L;
    const uint64_t nb = (n + bucket - 1) / bucket;
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    if (bits == 4) memset(codes, 0, (size_t)((n + 1) / 2));

#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < (int64_t)nb; ++b) {
        uint64_t lo = (uint64_t)b * bucket;
        uint64_t hi = lo + bucket < n ? lo + bucket : n;
        float sb = 0.0f;
        for (uint64_t i = lo; i < hi; ++i) {
            float a = fabsf(z[i]);
            if (a > sb) sb = a; /* a NaN never counts toward the bucket max */
        }
        scales[b] = sb;
        float inv = sb > 0.0f ? Lf / sb : 0.0f;
        float stepq = sb > 0.0f ? sb / Lf : 0.0f;
        for (uint64_t i = lo; i < hi; ++i) {
            uint32_t level = 0;
            float y = sb > 0.0f ? fabsf(z[i]) * inv : 0.0f;
            if (y > Lf) y = Lf;
            /* a NaN difference, and every difference in a bucket whose max is
             * infinite (|z| * 0), quantizes to level 0 */
            if (sb > 0.0f && !isnan(y)) {
                float l0 = floorf(y);
                float f = y - l0;
                uint64_t q = (base + i) / 4;
                uint32_t ctr[4] = {(uint32_t)q, (uint32_t)(q >> 32), (uint32_t)step,
                                   (uint32_t)(step >> 32)};
                uint32_t r[4];
                orc_philox4x32_10(ctr, key, r);
                float u = (float)(r[(base + i) % 4] >> 8) * 0x1p-24f;
                level = (uint32_t)l0 + (u < f ? 1u : 0u);
            }
            float C = 0.0f;
            uint32_t code = 0;
            if (level > 0) {
                float mag = (float)level * stepq;
                C = signbit(z[i]) ? -mag : mag;
                code = (signbit(z[i]) ? 1u << (bits - 1) : 0u) | level;
            }
            C_out[i] = C;
            if (bits == 8) {
                codes[i] = (uint8_t)code;
            } else {
                /* buckets hold an even number of elements, so a byte never
                 * straddles two buckets (or two threads) */
                codes[i / 2] |= (uint8_t)(code << (4 * (i % 2)));
            }
        }
    }
}

/* C(z)_i from the transmitted codes and bucket scales: the inverse of
 * quantize's encoding (level, sign; value level * fl(s_b / L)). */
static float dequantize(const float *scales, const uint8_t *codes, uint64_t i, int bits,
                        uint32_t bucket)
{
    const uint32_t L = (1u << (bits - 1)) - 1u;
    uint32_t code = bits == 8 ? codes[i] : (uint32_t)(codes[i / 2] >> (4 * (i % 2))) & 0xFu;
    uint32_t level = code & L;
    if (level == 0) return 0.0f;
    float sb = scales[i / bucket];
    float stepq = sb / (float)L;
    float mag = (float)level * stepq;
    return (code >> (bits - 1)) ? -mag : mag;
}

/*
 * DCD-PSGD (Tang et al.) step 2: z = x_{t+1/2} - x_t, x_{t+1} = x_t + C(z).
 */
void orc_dcd_window(const float *x, const float *x_half, float *x_out, uint64_t m, uint64_t base,
                    int bits, uint32_t bucket, uint64_t seed, uint64_t step,
                    float *scales, uint8_t *codes)
{
    float *z = (float *)calloc(m ? m : 1, sizeof(float));
    float *C = (float *)calloc(m ? m : 1, sizeof(float));
    for (uint64_t i = 0; i < m; ++i) z[i] = x_half[i] - x[i];
    quantize(z, m, base, bits, bucket, seed, step, scales, codes, C);
    for (uint64_t i = 0; i < m; ++i) x_out[i] = x[i] + C[i];
    free(z);
    free(C);
}

void orc_dcd(const float *x, const float *x_half, float *x_out, uint64_t n,
             int bits, uint32_t bucket, uint64_t seed, uint64_t step,
             float *scales, uint8_t *codes)
{
    orc_dcd_window(x, x_half, x_out, n, 0, bits, bucket, seed, step, scales, codes);
}

/*
 * DCD-PSGD step 3: a neighbour's replica advances by the received C(z):
 * x_hat <- x_hat + C(z).
 */
void orc_dcd_decode(const float *scales, const uint8_t *codes, uint64_t n, int bits,
                    uint32_t bucket, float *x_hat)
{
    for (uint64_t i = 0; i < n; ++i) x_hat[i] = x_hat[i] + dequantize(scales, codes, i, bits, bucket);
}

/*
 * DCD-PSGD step 1: x_{t+1/2} = sum_j W_ij x_hat_j - gamma * grad, the weighted
 * terms added in the order given, from +0.
 */
void orc_dcd_mix(int K, const float *const *replicas, const float *weights, const float *grad,
                 float lr, float *x_half, uint64_t n)
{
    for (uint64_t i = 0; i < n; ++i) {
        float s = 0.0f;
        for (int j = 0; j < K; ++j) {
            float term = weights[j] * replicas[j][i];
            s = s + term;
        }
        float g = lr * grad[i];
        x_half[i] = s - g;
    }
}

/*
 * ECD-PSGD, Eq. (3): the sender extrapolates z_t = (1 - t/2) x_{t-1} + (t/2) x_t
 * and sends C(z_t).  The coefficients are formed in double and rounded to fp32;
 * t is also the random-number step.
 */
void orc_ecd_compress(const float *x_prev, const float *x, uint64_t n, uint64_t t, int bits,
                      uint32_t bucket, uint64_t seed, float *scales, uint8_t *codes)
{
    const float a = (float)(1.0 - 0.5 * (double)t), b = (float)(0.5 * (double)t);
    float *z = (float *)calloc(n ? n : 1, sizeof(float));
    float *C = (float *)calloc(n ? n : 1, sizeof(float));
    for (uint64_t i = 0; i < n; ++i) {
        float p = a * x_prev[i];
        float q = b * x[i];
        z[i] = p + q;
    }
    quantize(z, n, 0, bits, bucket, seed, t, scales, codes, C);
    free(z);
    free(C);
}

/*
 * ECD-PSGD, Eq. (4): the receiver's estimate of the sender's model,
 * x~_t = (1 - 2/t) x~_{t-1} + (2/t) C(z_t), coefficients in double rounded to fp32.
 */
void orc_ecd_update(const float *scales, const uint8_t *codes, uint64_t n, int bits,
                    uint32_t bucket, uint64_t t, float *x_tilde)
{
    const float c1 = (float)(1.0 - 2.0 / (double)t), c2 = (float)(2.0 / (double)t);
    for (uint64_t i = 0; i < n; ++i) {
        float p = c1 * x_tilde[i];
        float q = c2 * dequantize(scales, codes, i, bits, bucket);
        x_tilde[i] = p + q;
    }
}

/* ------------------------------------------------------------------ Slim-DP */
/*
 * Slim-DP (Sun et al.), §3: the communication set is a core of significant
 * parameters plus a random explorer.
 *  - Significance of parameter i combines the magnitude of the parameter and
 *    of its gradient as a weighted sum with a positive coefficient c (the
 *    equation itself is not on the page): S_i = |w_i| + c |g_i|;
 *  - the core is the top-ranked parameters by S (here per tensor, k_s of
 *    them, ties to the lower index); a bitmap marks it, one word-aligned run
 *    of ceil(n_s/32) words per tensor, bit j%32 of word j/32 for entry j;
 *  - the explorer is a uniformly random set of the parameters outside the
 *    core, resampled every communication: the m_s non-core entries with the
 *    largest Philox4x32-10 keys (key (seed lo, seed hi), counter (j/4, s,
 *    step lo, step hi), word j%4, as r >> 1 | 1; core entries rank below).
 */
static void topk_by_key(const uint32_t *key, uint32_t n, uint32_t k, uint32_t *chosen)
{
    keyed *order = (keyed *)malloc(sizeof(keyed) * (size_t)(n ? n : 1));
    for (uint32_t i = 0; i < n; ++i) {
        order[i].key = key[i];
        order[i].pos = i;
    }
    qsort(order, n, sizeof(keyed), by_key_desc_pos_asc);
    for (uint32_t j = 0; j < k; ++j) chosen[j] = order[j].pos;
    qsort(chosen, k, sizeof(uint32_t), u32_asc);
    free(order);
}

void orc_slimdp_core(const orc_seg *segs, int nseg, const float *w, const float *g, float c,
                     uint32_t *core_idx, float *core_val, uint32_t *seg_off, uint32_t *mask)
{
    uint32_t pos = 0;
    uint64_t mbase = 0;
    for (int s = 0; s < nseg; ++s) {
        const uint64_t base = segs[s].offset;
        const uint32_t n = segs[s].length, k = segs[s].k;
        float *S = (float *)malloc(sizeof(float) * (size_t)n);
        uint32_t *key = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)n);
        uint32_t *chosen = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)k);
        for (uint32_t i = 0; i < n; ++i) {
            float cg = c * fabsf(g[base + i]);
            S[i] = fabsf(w[base + i]) + cg;
            key[i] = abs_bits(S[i]);
        }
        topk_by_key(key, n, k, chosen);
        uint32_t words = (n + 31) / 32;
        memset(mask + mbase, 0, sizeof(uint32_t) * words);
        seg_off[s] = pos;
        for (uint32_t j = 0; j < k; ++j) {
            core_idx[pos + j] = (uint32_t)(base + chosen[j]);
            core_val[pos + j] = S[chosen[j]];
            mask[mbase + chosen[j] / 32] |= 1u << (chosen[j] % 32);
        }
        pos += k;
        mbase += words;
        free(S);
        free(key);
        free(chosen);
    }
    seg_off[nseg] = pos;
}

void orc_slimdp_explore(const orc_seg *segs, int nseg, const float *delta, const uint32_t *mask,
                        uint64_t seed, uint64_t step, uint32_t *idx, float *val, uint32_t *seg_off)
{
    const uint32_t pkey[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t pos = 0;
    uint64_t mbase = 0;
    for (int s = 0; s < nseg; ++s) {
        const uint64_t base = segs[s].offset;
        const uint32_t n = segs[s].length, m = segs[s].k;
        uint32_t *key = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)n);
        uint32_t *chosen = (uint32_t *)malloc(sizeof(uint32_t) * (size_t)(m ? m : 1));
        for (uint32_t j = 0; j < n; ++j) {
            uint32_t ctr[4] = {j / 4, (uint32_t)s, (uint32_t)step, (uint32_t)(step >> 32)};
            uint32_t r[4];
            orc_philox4x32_10(ctr, pkey, r);
            int in_core = (mask[mbase + j / 32] >> (j % 32)) & 1u;
            key[j] = in_core ? 0u : ((r[j % 4] >> 1) | 1u);
        }
        topk_by_key(key, n, m, chosen);
        seg_off[s] = pos;
        for (uint32_t j = 0; j < m; ++j) {
            idx[pos + j] = (uint32_t)(base + chosen[j]);
            val[pos + j] = delta[base + chosen[j]];
        }
        pos += m;
        mbase += (n + 31) / 32;
        free(key);
        free(chosen);
    }
    seg_off[nseg] = pos;
}
