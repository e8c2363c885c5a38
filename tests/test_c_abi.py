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
