"""The C ABI from C: a C99 program compiled by gcc against include/gradcomp.h
(plain C, no C++ or HIP compiler) links to libgradcomp.so and calls its
host-side entry points.  Nothing here touches a device: plan queries, the
host checks that reject bad arguments before anything is enqueued, and the
error strings."""
import os
import shutil
import subprocess

import pytest

from gradient_compression_dnn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "gradcomp.h"

#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); return 1; } } while (0)

int main(void) {
    /* two segments with a gap, k and bins as a layer table would give them */
    gc_segment segs[2] = {{0, 5000, 50, 5, 0}, {6000, 100, 7, 1, 0}};
    gc_plan *p = NULL;
    CHECK(strstr(gc_version(), "libgradcomp") != NULL);
    CHECK(gc_topk_count(1001) == 2);
    CHECK(gc_plan_create(segs, 2, 6100, &p) == GC_OK && p != NULL);
    CHECK(gc_plan_num_segments(p) == 2);
    CHECK(gc_plan_num_elements(p) == 6100);
    CHECK(gc_plan_total_k(p) == 6);
    CHECK(gc_plan_total_bins(p) == 100 + 15);
    CHECK(gc_plan_workspace_bytes(p, GC_OP_DGC) > 0);
    CHECK(gc_pack_bound(p, GC_KIND_DGC) > 0 && gc_pack_bound(p, 99) == 0);
    CHECK(gc_slimdp_mask_words(p) == 157 + 4);
    CHECK(gc_adacomp_message_cap(p) == 5100);
    {
        gc_dgc_options o;
        memset(&o, 0, sizeof o);
        o.momentum = 0.9f;
        o.num_nodes = 1;
        o.momentum_kind = GC_MOMENTUM_VANILLA;
        o.select = GC_SELECT_SAMPLED;
        o.sample_period = 100;
        o.over = 2;
        CHECK(gc_dgc_message_cap(p, &o) == 10 + 2);
    }
    /* host-side rejections: nothing is enqueued and the reason is kept */
    CHECK(gc_dgc_step(NULL, NULL, NULL, NULL, 0.9f, 0.0f, 1, NULL, NULL, 0, NULL) == GC_EINVAL);
    CHECK(strlen(gc_last_error()) > 0);
    CHECK(gc_decompress_accumulate(p, NULL, 0, NULL, GC_SUM, 0, NULL, 0, NULL) == GC_EINVAL);
    {
        gc_segment bad = {0, 10, 1, 11, 0};  /* k > length */
        gc_plan *q = NULL;
        CHECK(gc_plan_create(&bad, 1, 10, &q) == GC_EINVAL && q == NULL);
        CHECK(strstr(gc_last_error(), "k must be") != NULL);
    }
    gc_plan_destroy(p);
    printf("ok\n");
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs gcc and the ROCm headers")
def test_c_program_links_and_calls_the_host_entry_points(tmp_path):
    B.load()  # the library must be built
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(B.LIB_PATH)
    # a non-HIP compiler names the platform for hip_runtime_api.h
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", ROCM_INCLUDE, str(src), "-o", str(exe), "-L", libdir, "-lgradcomp", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


GPU_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include <hip/hip_runtime_api.h>
#include "gradcomp.h"

#define CHECK(c) do { if (!(c)) { printf("FAIL line %d: %s\n", __LINE__, #c); return 1; } } while (0)
#define HIP(c) CHECK((c) == hipSuccess)

/* Two segments with a gap; G_i = i + 1 inside them, so that the DGC step's
 * top-k (from a zero state, no clipping, momentum 0.5) is each segment's last
 * k elements, sent with V = G. */
int main(void) {
    enum { N = 3000, K0 = 4, K1 = 2 };
    gc_segment segs[2] = {{0, 1000, 50, K0, 0}, {1500, 1500, 50, K1, 0}};
    gc_plan *p = NULL;
    CHECK(gc_plan_create(segs, 2, N, &p) == GC_OK);
    static float host[N];
    for (int i = 0; i < N; ++i) host[i] = (float)(i + 1);
    float *G, *U, *V, *dense, *val;
    uint32_t *idx, *seg_off;
    uint8_t *ws, *packed;
    uint64_t *nbytes;
    size_t wsb = gc_plan_workspace_bytes(p, GC_OP_DGC);
    if (gc_plan_workspace_bytes(p, GC_OP_PACK) > wsb) wsb = gc_plan_workspace_bytes(p, GC_OP_PACK);
    if (gc_plan_workspace_bytes(p, GC_OP_DECODE) > wsb) wsb = gc_plan_workspace_bytes(p, GC_OP_DECODE);
    uint64_t bound = gc_pack_bound(p, GC_KIND_DGC);
    HIP(hipMalloc((void **)&G, N * 4));
    HIP(hipMalloc((void **)&U, N * 4));
    HIP(hipMalloc((void **)&V, N * 4));
    HIP(hipMalloc((void **)&dense, N * 4));
    HIP(hipMalloc((void **)&idx, 64));
    HIP(hipMalloc((void **)&val, 64));
    HIP(hipMalloc((void **)&seg_off, 16));
    HIP(hipMalloc((void **)&ws, wsb));
    HIP(hipMalloc((void **)&packed, bound));
    HIP(hipMalloc((void **)&nbytes, 8));
    HIP(hipMemcpy(G, host, N * 4, hipMemcpyHostToDevice));
    HIP(hipMemset(U, 0, N * 4));
    HIP(hipMemset(V, 0, N * 4));
    HIP(hipMemset(dense, 0, N * 4));  /* the decode writes segment elements only */
    gc_sparse msg = {idx, val, seg_off, NULL, K0 + K1};
    CHECK(gc_dgc_step(p, G, U, V, 0.5f, 0.0f, 1, &msg, ws, wsb, NULL) == GC_OK);
    CHECK(gc_pack(p, GC_KIND_DGC, &msg, packed, bound, nbytes, ws, wsb, NULL) == GC_OK);
    CHECK(gc_decompress_accumulate(p, &msg, 1, dense, GC_SUM, 0, ws, wsb, NULL) == GC_OK);
    HIP(hipDeviceSynchronize());
    uint32_t hidx[K0 + K1], hoff[3];
    float hval[K0 + K1], hV[N];
    uint64_t hn = 0;
    HIP(hipMemcpy(hidx, idx, sizeof hidx, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(hval, val, sizeof hval, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(hoff, seg_off, sizeof hoff, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(hV, V, sizeof hV, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(&hn, nbytes, 8, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(host, dense, N * 4, hipMemcpyDeviceToHost));
    CHECK(hoff[0] == 0 && hoff[1] == K0 && hoff[2] == K0 + K1);
    for (int j = 0; j < K0; ++j) CHECK(hidx[j] == 1000 - K0 + j && hval[j] == (float)(1000 - K0 + j + 1));
    for (int j = 0; j < K1; ++j) CHECK(hidx[K0 + j] == 3000 - K1 + j && hval[K0 + j] == (float)(3000 - K1 + j + 1));
    CHECK(hV[999] == 0.0f && hV[995] == 996.0f);  /* masked where sent, V = G elsewhere */
    /* stream header, block table, two blocks of K codes and one checkpoint each */
    CHECK(hn == 16 + 2 * 16 + (16 + 2 * K0 + 4 * K0 + 8) + (16 + 2 * K1 + 4 * K1 + 8));
    CHECK(host[999] == 1000.0f && host[998] == 999.0f && host[995] == 0.0f && host[1200] == 0.0f);
    gc_plan_destroy(p);
    printf("ok\n");
    return 0;
}
"""


@pytest.mark.gpu
def test_c_program_runs_the_path_on_the_gpu(tmp_path):
    """The same C ABI from a C program on the GPU: device buffers from
    hipMalloc, a DGC step, its packed stream and its decode, checked against
    values that follow by hand from the input pattern."""
    B.load()
    src = tmp_path / "path.c"
    src.write_text(GPU_PROGRAM)
    exe = tmp_path / "path"
    libdir = os.path.dirname(B.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", ROCM_INCLUDE, str(src), "-o", str(exe), "-L", libdir, "-lgradcomp", "-L", "/opt/rocm/lib",
           "-lamdhip64", f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
