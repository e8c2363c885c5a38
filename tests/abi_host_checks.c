/* Host-side checks of libgradcomp driven from C, for the sanitizer build:
 * plan creation over valid and malformed segment tables, every plan query,
 * message and workspace sizes, and the argument checks each entry point
 * makes before it enqueues anything.  Every device pointer passed here is
 * NULL or accompanies an argument the host rejects, so nothing reaches a
 * GPU.  Exit status 0 when every check holds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include "gradcomp.h"

static int failures = 0;
#define CHECK(c)                                                      \
    do {                                                              \
        if (!(c)) {                                                   \
            printf("FAIL line %d: %s (%s)\n", __LINE__, #c, gc_last_error()); \
            ++failures;                                               \
        }                                                             \
    } while (0)

static gc_status make(const gc_segment *s, int n, uint64_t total, gc_plan **p) {
    *p = NULL;
    return gc_plan_create(s, n, total, p);
}

static void malformed_tables(void) {
    gc_plan *p = NULL;
    gc_segment one = {0, 100, 10, 5, 0};
    CHECK(gc_plan_create(&one, 1, 100, NULL) == GC_EINVAL);
    CHECK(make(NULL, 1, 100, &p) == GC_EINVAL && p == NULL);
    CHECK(make(&one, 0, 100, &p) == GC_EINVAL && p == NULL);
    CHECK(make(&one, -3, 100, &p) == GC_EINVAL && p == NULL);
    CHECK(make(&one, 1, (uint64_t)1 << 32, &p) == GC_ERANGE && p == NULL);
    CHECK(make(&one, 1, 99, &p) == GC_EINVAL && p == NULL);
    {
        gc_segment s[6][1] = {{{0, 0, 10, 1, 0}},     /* empty segment */
                              {{0, 100, 0, 5, 0}},    /* bin_len 0 */
                              {{0, 100, 10, 0, 0}},   /* k 0 */
                              {{0, 100, 10, 101, 0}}, /* k > length */
                              {{0, 100, 10, 5, 7}},   /* reserved set */
                              {{UINT64_MAX, 2, 1, 1, 0}}};  /* offset + length wraps */
        for (int i = 0; i < 6; ++i) {
            CHECK(make(s[i], 1, 1000, &p) == GC_EINVAL && p == NULL);
            CHECK(strlen(gc_last_error()) > 0);
        }
    }
    {
        gc_segment big = {0, 100, GC_MAX_BIN_LEN + 1, 5, 0};
        CHECK(make(&big, 1, 100, &p) == GC_ENOTSUP && p == NULL);
    }
    {
        gc_segment ov[2] = {{0, 100, 10, 5, 0}, {50, 100, 10, 5, 0}};   /* overlap */
        CHECK(make(ov, 2, 1000, &p) == GC_EINVAL && p == NULL);
        gc_segment desc[2] = {{500, 100, 10, 5, 0}, {0, 100, 10, 5, 0}}; /* descending */
        CHECK(make(desc, 2, 1000, &p) == GC_EINVAL && p == NULL);
        gc_segment past[2] = {{0, 100, 10, 5, 0}, {900, 101, 10, 5, 0}}; /* one past the end */
        CHECK(make(past, 2, 1000, &p) == GC_EINVAL && p == NULL);
        gc_segment wrap[2] = {{0, 100, 10, 5, 0}, {UINT64_MAX - 1, 3, 1, 1, 0}};
        CHECK(make(wrap, 2, 1000, &p) == GC_EINVAL && p == NULL);
    }
}

static void queries(void) {
    /* a layer table with gaps, odd lengths and every bin length class */
    enum { NS = 9 };
    gc_segment s[NS];
    const uint32_t len[NS] = {1, 2, 63, 4095, 4096, 4097, 12289, 50000, 131149};
    const uint32_t bl[NS] = {1, 2, 7, 50, 64, 500, 4096, 50, 500};
    uint64_t off = 3, total_k = 0, bins = 0;
    for (int i = 0; i < NS; ++i) {
        s[i].offset = off;
        s[i].length = len[i];
        s[i].bin_len = bl[i];
        s[i].k = gc_topk_count(len[i]);
        s[i].reserved = 0;
        total_k += s[i].k;
        bins += (len[i] + bl[i] - 1) / bl[i];
        off += len[i] + (uint64_t)(i % 3);
    }
    gc_plan *p = NULL;
    CHECK(make(s, NS, off + 5, &p) == GC_OK && p != NULL);
    if (!p) return;
    CHECK(gc_plan_num_segments(p) == NS);
    CHECK(gc_plan_num_elements(p) == off + 5);
    CHECK(gc_plan_total_k(p) == total_k);
    CHECK(gc_plan_total_bins(p) == bins);
    for (int op = GC_OP_DGC; op <= GC_OP_UNPACK; ++op) CHECK(gc_plan_workspace_bytes(p, op) > 0);
    CHECK(gc_plan_workspace_bytes(p, 0) == 0 && gc_plan_workspace_bytes(p, 99) == 0);
    CHECK(gc_plan_workspace_bytes(NULL, GC_OP_DGC) == 0);
    CHECK(gc_adacomp_state_bytes(p) > 0 && gc_adacomp_state_bytes(NULL) == 0);
    CHECK(gc_adacomp_message_cap(p) >= total_k);
    CHECK(gc_pack_bound(p, GC_KIND_DGC) > 0 && gc_pack_bound(p, GC_KIND_ADACOMP) > 0);
    CHECK(gc_pack_bound(p, 0) == 0 && gc_pack_bound(NULL, GC_KIND_DGC) == 0);
    CHECK(gc_slimdp_mask_words(p) > 0 && gc_slimdp_mask_words(NULL) == 0);
    {
        gc_dgc_options o;
        memset(&o, 0, sizeof o);
        o.momentum = 0.9f;
        o.num_nodes = 1;
        CHECK(gc_dgc_message_cap(p, &o) == total_k);
        CHECK(gc_dgc_message_cap(p, NULL) == total_k && gc_dgc_message_cap(NULL, &o) == 0);
        /* warm-up densities: ceil(n * num / den) per segment, at least 1 */
        o.density_num = 1;
        o.density_den = 4;
        uint64_t want = 0;
        for (int i = 0; i < NS; ++i) want += (len[i] + 3u) / 4u;
        CHECK(gc_dgc_message_cap(p, &o) == want);
        o.density_den = 0;
        o.select = GC_SELECT_SAMPLED;
        o.sample_period = 100;
        o.over = 2;
        CHECK(gc_dgc_message_cap(p, &o) >= total_k);
    }
    CHECK(gc_topk_count(0) == 1 && gc_topk_count(1) == 1 && gc_topk_count(1000) == 1);
    CHECK(gc_topk_count(1001) == 2 && gc_topk_count(UINT32_MAX) == 4294968u);
    CHECK(gc_decompress_noalloc_max_chunks(1) > 0);
    CHECK(gc_decompress_noalloc_max_chunks(0) == 0 && gc_decompress_noalloc_max_chunks(-1) == 0);
    CHECK(gc_decompress_noalloc_max_chunks(GC_MAX_MESSAGES + 1) == 0);
    gc_plan_destroy(p);
}

/* every entry point with null buffers: rejected on the host, a reason kept */
static void host_rejections(void) {
    gc_segment one = {0, 5000, 50, 5, 0};
    gc_plan *p = NULL;
    CHECK(make(&one, 1, 5000, &p) == GC_OK);
    gc_sparse sp;
    memset(&sp, 0, sizeof sp);
    gc_dgc_options o;
    memset(&o, 0, sizeof o);
    o.momentum = 0.9f;
    o.num_nodes = 1;
    uint64_t nbytes = 0;
    uint32_t status = 0;
    double ms = 0;
    uint64_t launches = 0;
    const float *reps[2] = {NULL, NULL};
    const float wts[2] = {0.5f, 0.5f};
#define REJECT(call)                              \
    do {                                          \
        gc_status r_ = (call);                    \
        CHECK(r_ != GC_OK);                       \
        CHECK(strlen(gc_last_error()) > 0);       \
    } while (0)
    REJECT(gc_dgc_step(NULL, NULL, NULL, NULL, 0.9f, 1.0f, 1, &sp, NULL, 0, NULL));
    REJECT(gc_dgc_step(p, NULL, NULL, NULL, 0.9f, 1.0f, 1, &sp, NULL, 0, NULL));
    REJECT(gc_dgc_step(p, NULL, NULL, NULL, 1.5f, 1.0f, 1, NULL, NULL, 0, NULL));
    REJECT(gc_dgc_step_ex(p, NULL, NULL, NULL, &o, &sp, NULL, 0, NULL));
    REJECT(gc_dgc_step_ex(p, NULL, NULL, NULL, NULL, &sp, NULL, 0, NULL));
    REJECT(gc_adacomp_compress(p, NULL, NULL, NULL, 0, 2.0f, &sp, NULL, 0, NULL));
    REJECT(gc_adacomp_compress(NULL, NULL, NULL, NULL, 0, 2.0f, NULL, NULL, 0, NULL));
    REJECT(gc_adacomp_residual(p, NULL, NULL, 0, NULL, NULL));
    REJECT(gc_pack(p, GC_KIND_DGC, &sp, NULL, 0, &nbytes, NULL, 0, NULL));
    REJECT(gc_pack(p, 7, &sp, NULL, 0, &nbytes, NULL, 0, NULL));
    REJECT(gc_unpack(p, GC_KIND_ADACOMP, NULL, 0, &sp, &status, NULL, 0, NULL));
    REJECT(gc_decompress_accumulate(p, &sp, 0, NULL, GC_SUM, 0, NULL, 0, NULL));
    REJECT(gc_decompress_accumulate(p, &sp, GC_MAX_MESSAGES + 1, NULL, GC_AVG, 0, NULL, 0, NULL));
    REJECT(gc_decompress_accumulate_noalloc(p, &sp, 1, NULL, GC_SUM, 0, NULL));
    REJECT(gc_dcd_compress(NULL, NULL, NULL, 100, 4, 512, 1, 0, NULL, NULL, NULL));
    REJECT(gc_dcd_compress(NULL, NULL, NULL, 100, 3, 512, 1, 0, NULL, NULL, NULL));
    REJECT(gc_dcd_decode(NULL, NULL, 100, 4, 512, NULL, NULL));
    REJECT(gc_dcd_mix(reps, wts, 2, NULL, 0.1f, NULL, 100, NULL));
    REJECT(gc_dcd_mix(reps, wts, GC_MAX_REPLICAS + 1, NULL, 0.1f, NULL, 100, NULL));
    REJECT(gc_ecd_compress(NULL, NULL, 100, 1, 4, 512, 1, NULL, NULL, NULL));
    REJECT(gc_ecd_update(NULL, NULL, 100, 4, 512, 1, NULL, NULL));
    REJECT(gc_slimdp_core(p, NULL, NULL, 0.1f, &sp, NULL, NULL, 0, NULL));
    REJECT(gc_slimdp_explore(p, p, NULL, NULL, 1, 2, &sp, NULL, 0, NULL));
    REJECT(gc_slimdp_core_values(p, &sp, NULL, NULL, NULL));
    REJECT(gc_stream_probe(NULL, NULL, NULL, NULL, NULL, 100, NULL));
    REJECT(gc_timing_take(NULL, &ms, &launches));
    CHECK(gc_timing_enable(NULL) == GC_OK);
#undef REJECT
    gc_plan_destroy(p);
    gc_plan_destroy(NULL);
}

/* many small plans: creation and teardown leave nothing behind */
static void many_plans(void) {
    enum { NS = 17000 };
    gc_segment *s = (gc_segment *)calloc(NS, sizeof(gc_segment));
    if (!s) return;
    uint64_t off = 0;
    for (int i = 0; i < NS; ++i) {
        s[i].offset = off;
        s[i].length = 1 + (uint32_t)(i % 97) * 37u;
        s[i].bin_len = 1 + (uint32_t)(i % 13);
        s[i].k = 1 + s[i].length / 1000u;
        off += s[i].length + (uint64_t)(i & 1);
    }
    for (int r = 0; r < 3; ++r) {
        gc_plan *p = NULL;
        CHECK(make(s, NS, off, &p) == GC_OK);
        CHECK(gc_plan_num_segments(p) == NS);
        CHECK(gc_plan_workspace_bytes(p, GC_OP_DGC) > 0);
        gc_plan_destroy(p);
    }
    free(s);
}

int main(void) {
    CHECK(strstr(gc_version(), "libgradcomp") != NULL);
    malformed_tables();
    queries();
    host_rejections();
    many_plans();
    if (failures) {
        printf("%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
