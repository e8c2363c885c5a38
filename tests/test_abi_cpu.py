"""Host-only checks of the C ABI: the library loads here (no GPU), exports
every function the header declares, and validates plans on the host."""
import ctypes
import os
import re

import numpy as np
import pytest

from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "gradcomp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gc_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = B.load()
    declared = header_functions()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(B.exported_symbols()) == declared


def test_version_and_topk_count():
    assert "libgradcomp" in B.gc_version()
    assert B.gc_topk_count(1) == 1
    assert B.gc_topk_count(1000) == 1
    assert B.gc_topk_count(1001) == 2
    assert B.gc_topk_count(1 << 20) == 1049


def _create(rows, n_total):
    lib = B.load()
    arr = (B.gc_segment * max(len(rows), 1))()
    for i, r in enumerate(rows):
        arr[i] = B.gc_segment(*r)
    h = ctypes.c_void_p()
    st = lib.gc_plan_create(arr, len(rows), n_total, ctypes.byref(h))
    if st == 0:
        lib.gc_plan_destroy(h)
    return st


@pytest.mark.parametrize("rows,n_total,code", [
    ([], 10, B.GC_EINVAL),                                   # no segments
    ([(0, 0, 1, 1, 0)], 10, B.GC_EINVAL),                    # empty segment
    ([(0, 5, 1, 1, 0), (4, 5, 1, 1, 0)], 10, B.GC_EINVAL),   # overlap
    ([(5, 5, 1, 1, 0), (0, 5, 1, 1, 0)], 10, B.GC_EINVAL),   # not ascending
    ([(0, 11, 1, 1, 0)], 10, B.GC_EINVAL),                   # past n_total
    ([(0, 5, 0, 1, 0)], 10, B.GC_EINVAL),                    # bin_len 0
    ([(0, 5, 1, 0, 0)], 10, B.GC_EINVAL),                    # k 0
    ([(0, 5, 1, 6, 0)], 10, B.GC_EINVAL),                    # k > length
    ([(0, 5, 1, 1, 7)], 10, B.GC_EINVAL),                    # reserved != 0
    ([(0, 5, 4097, 1, 0)], 10, B.GC_ENOTSUP),                # bin_len too large
    ([(0, 5, 1, 1, 0)], 1 << 32, B.GC_ERANGE),               # indices are u32
    ([(0, B.GC_MAX_SEGMENT_LEN + 1, 1, 1, 0)], (1 << 32) - 1, B.GC_ENOTSUP),  # u32 code count
    ([(0, 0xFFFFFFFF, 64, 1, 0)], (1 << 32) - 1, B.GC_ENOTSUP),
    ([(0, 5, 1, 5, 0), (7, 3, 2, 1, 0)], 10, B.GC_OK),       # gap allowed
    # offsets near 2^64: offset + length wraps to a small value
    ([((1 << 64) - 1, 1, 1, 1, 0)], 10, B.GC_EINVAL),
    ([((1 << 64) - 1, 2, 1, 1, 0)], 10, B.GC_EINVAL),
    ([(0, 5, 1, 1, 0), ((1 << 64) - 2, 3, 1, 1, 0)], 10, B.GC_EINVAL),
    ([(10, 1, 1, 1, 0)], 10, B.GC_EINVAL),                   # starts at n_total
])
def test_plan_validation(rows, n_total, code):
    assert _create(rows, n_total) == code
    if code != B.GC_OK:
        assert B.gc_last_error() != ""


def test_plan_rejects_negative_offsets_from_the_binding():
    # an int64 table offset of -1 reaches the library as 2^64 - 1
    for off, n in ((-1, 1), (-1, 2), (-2, 3)):
        with pytest.raises(B.GCError) as e:
            B.Plan(np.array([[off, n, 1, 1]], dtype=np.int64), 10)
        assert e.value.status == B.GC_EINVAL


def test_noalloc_decode_capacity():
    # 8 MiB of u32 start entries: K * (chunks + 1) <= 2^21
    assert B.gc_decompress_noalloc_max_chunks(1) == (1 << 21) - 1
    assert B.gc_decompress_noalloc_max_chunks(8) == (1 << 18) - 1
    assert B.gc_decompress_noalloc_max_chunks(64) == (1 << 15) - 1
    assert B.gc_decompress_noalloc_max_chunks(0) == 0
    assert B.gc_decompress_noalloc_max_chunks(65) == 0
    # the DeepSpeech layout (29,760 chunks) fits 64 messages
    w = W.make_config("deepspeech")
    assert B.Plan(w.table, w.n_total).total_k > 0
    assert sum(-(-int(n) // 4096) for n in w.table[:, 1]) <= B.gc_decompress_noalloc_max_chunks(64)


def test_plan_queries_and_workspace_on_workloads():
    for name in ("fc1m", "resnet50", "deepspeech"):
        w = W.make_config(name)
        p = B.Plan(w.table, w.n_total)
        t = w.table
        assert p.total_k == int(t[:, 3].sum())
        assert p.total_bins == int(((t[:, 1] + t[:, 2] - 1) // t[:, 2]).sum())
        for op in (B.GC_OP_DGC, B.GC_OP_ADACOMP, B.GC_OP_PACK, B.GC_OP_DECODE, B.GC_OP_UNPACK):
            assert p.workspace_bytes(op) > 0
        # staging needs 8 bytes per element at most, plus small tables
        assert p.workspace_bytes(B.GC_OP_DGC) < 9 * w.n_total + (64 << 20)
        # deferred AdaComp state: one selection bit per element slot, plus the scales
        assert p.adacomp_state_bytes >= w.n_total // 8
        assert p.adacomp_state_bytes < w.n_total // 8 + (4 << 20)
        # the pack bound covers the format's closed form at k entries per segment
        E = t[:, 3]
        assert p.pack_bound(B.GC_KIND_DGC) >= 16 + int(np.sum(16 + 16 + 6 * E + 2 * (E % 2) + 8 * -(-E // 4096)))
        del p


def test_longest_segments_at_the_top_of_the_index_range():
    # the longest segment ends at the last u32 index; counts that round up
    # a length near 2^32 must not wrap
    L = B.GC_MAX_SEGMENT_LEN
    n_total = (1 << 32) - 1
    for bin_len in (1, 50, 4096):
        t = np.array([[7, 100, bin_len, 3], [n_total - L, L, bin_len, L]], dtype=np.int64)
        p = B.Plan(t, n_total)
        assert p.total_k == 3 + L
        assert p.total_bins == -(-100 // bin_len) + -(-L // bin_len)
        assert B.gc_slimdp_mask_words(p) == 4 + -(-L // 32)
        assert p.workspace_bytes(B.GC_OP_DGC) >= 8 * n_total
        # every DGC chunk has a few u32 counters in the workspace
        assert p.workspace_bytes(B.GC_OP_DECODE) >= 4 * -(-L // 4096)
        # an AdaComp message that sends every element: entries plus escapes
        codes = L + L // 32767 + 1
        assert codes < 1 << 32
        assert p.pack_bound(B.GC_KIND_ADACOMP) >= 16 + 2 * (16 + 16) + 2 * codes + 8 * -(-codes // 4096)
        del p


def test_hot_calls_reject_null_plan_without_touching_a_device():
    lib = B.load()
    assert lib.gc_plan_upload(None) == B.GC_EINVAL
    assert lib.gc_dgc_step(None, None, None, None, 0.9, 0.0, 1, None, None, 0, None) == B.GC_EINVAL
    assert lib.gc_adacomp_compress(None, None, None, None, 0, 2.0, None, None, 0, None) == B.GC_EINVAL
    assert lib.gc_adacomp_residual(None, None, None, 0, None, None) == B.GC_EINVAL
    assert lib.gc_adacomp_state_bytes(None) == 0
    assert lib.gc_pack(None, 1, None, None, 0, None, None, 0, None) == B.GC_EINVAL
    assert lib.gc_decompress_accumulate(None, None, 1, None, 1, 0, None, 0, None) == B.GC_EINVAL
    assert lib.gc_dcd_compress(None, None, None, 10, 4, 512, 0, 0, None, None, None) == B.GC_EINVAL


def test_dgc_ex_host_checks_and_message_cap():
    lib = B.load()
    assert lib.gc_dgc_step_ex(None, None, None, None, None, None, None, 0, None) == B.GC_EINVAL
    t = W.make_table([5000, 100, 7], [1, 1, 1], [5, 1, 3])
    p = B.Plan(t)
    exact = B.dgc_options(0.9)
    assert B.gc_dgc_message_cap(p, exact) == 9
    # sampled: sum of min(n_s, over * k_s)
    assert B.gc_dgc_message_cap(p, B.dgc_options(0.9, sampled=True, over=2)) == 10 + 2 + 6
    assert B.gc_dgc_message_cap(p, B.dgc_options(0.9, sampled=True, over=3)) == 15 + 3 + 7
    assert lib.gc_dgc_message_cap(None, None) == 0
    # a per-call density: ceil(n_s num / den), at least 1, at most n_s
    assert B.gc_dgc_message_cap(p, B.dgc_options(0.9, density=(1, 4))) == 1250 + 25 + 2
    assert B.gc_dgc_message_cap(p, B.dgc_options(0.9, density=(1, 256))) == 20 + 1 + 1
    assert B.gc_dgc_message_cap(p, B.dgc_options(0.9, density=(3, 3))) == 5000 + 100 + 7


def test_adacomp_message_cap_is_the_sum_of_the_segment_lengths():
    t = W.make_table([5000, 100, 7], [1, 1, 1], [5, 1, 3], [10, 2000, 3])
    p = B.Plan(t, W.table_extent(t) + 50)
    assert B.gc_adacomp_message_cap(p) == 5107
    assert B.load().gc_adacomp_message_cap(None) == 0
    # the host checks the capacity before anything touches a device (the
    # pointers are never dereferenced on these paths)
    lib, fake = B.load(), ctypes.c_void_p(256)

    def call(cap):
        msg = B.gc_sparse(fake, fake, fake, fake, cap)
        return lib.gc_adacomp_compress(p.handle, fake, fake, None, 0, 2.0, ctypes.byref(msg), None, 0, None)

    assert call(5106) == B.GC_ECAPACITY and "gc_adacomp_message_cap" in B.gc_last_error()
    assert call(5107) == B.GC_ECAPACITY and "workspace" in B.gc_last_error()  # next check: no workspace


def test_slimdp_mask_words():
    t = W.make_table([40, 5, 64], [1, 1, 1], [1, 1, 1])
    p = B.Plan(t)
    assert B.gc_slimdp_mask_words(p) == 2 + 1 + 2
    assert B.load().gc_slimdp_mask_words(None) == 0
    assert B.load().gc_slimdp_core(None, None, None, 1.0, None, None, None, 0, None) == B.GC_EINVAL


def test_dgc_ex_rejects_options_on_the_host():
    lib = B.load()
    p = B.Plan(W.make_table([5000], [1], [5]))
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    cases = [
        (B.dgc_options(0.9, sampled=True, sample_period=(1 << 26) + 1), "sample_period"),
        (B.dgc_options(0.9, sampled=True, sample_period=0), "sample_period"),
        (B.dgc_options(0.9, sampled=True, over=0), "over"),
        (B.dgc_options(1.0), "momentum"),
        (B.dgc_options(0.9, density=(0, 4)), "density_num"),
        (B.dgc_options(0.9, density=(5, 4)), "density_num"),
        (B.gc_dgc_options(0.9, 0.0, 1, 7, 0, 100, 2, 0), "momentum_kind"),
        (B.gc_dgc_options(0.9, 0.0, 1, 0, 5, 100, 2, 0), "select"),
        (B.gc_dgc_options(0.9, 0.0, 1, 0, 0, 100, 2, 1), "reserved"),
    ]
    for opt, word in cases:
        st = lib.gc_dgc_step_ex(p.handle, fake, fake, fake, ctypes.byref(opt), None, None, 0, None)
        assert st == B.GC_EINVAL and word in B.gc_last_error(), (word, B.gc_last_error())
    # a per-call density is for exact selection only
    opt = B.dgc_options(0.9, sampled=True, density=(1, 4))
    st = lib.gc_dgc_step_ex(p.handle, fake, fake, fake, ctypes.byref(opt), None, None, 0, None)
    assert st == B.GC_ENOTSUP and "density" in B.gc_last_error()


def test_last_error_is_per_thread():
    """Two host threads fail plan creation for different reasons at the same
    time: each reads back its own message (the error state is thread-local),
    and a success in one thread does not clear the other's."""
    import threading

    lib = B.load()
    barrier = threading.Barrier(3)
    seen = {}

    def worker(name, rows, n_total, code):
        arr = (B.gc_segment * len(rows))(*[B.gc_segment(*r) for r in rows])
        for _ in range(200):
            barrier.wait()
            h = ctypes.c_void_p()
            st = lib.gc_plan_create(arr, len(rows), n_total, ctypes.byref(h))
            if st == B.GC_OK:
                lib.gc_plan_destroy(h)
            barrier.wait()
            msg = lib.gc_last_error().decode()
            if st != code or (code != B.GC_OK and name not in msg) or (code == B.GC_OK and msg):
                seen.setdefault(name, []).append((st, msg))

    t1 = threading.Thread(target=worker, args=("k must be", [(0, 10, 1, 11, 0)], 10, B.GC_EINVAL))
    t2 = threading.Thread(target=worker, args=("n_total must be", [(0, 5, 1, 1, 0)], 1 << 32, B.GC_ERANGE))
    t3 = threading.Thread(target=worker, args=("ok", [(0, 5, 1, 1, 0)], 10, B.GC_OK))
    for t in (t1, t2, t3):
        t.start()
    for t in (t1, t2, t3):
        t.join()
    assert not seen, seen


def test_binding_checks_tensors_before_calling_the_library():
    """The binding passes only contiguous CUDA tensors of the right type and
    size: host tensors are refused before anything reaches the C ABI."""
    import torch

    p = B.Plan(W.make_table([5000, 100], [1, 1], [5, 1]))
    host = B.Sparse(torch.zeros(6, dtype=torch.int32), torch.zeros(6), torch.zeros(3, dtype=torch.int32),
                    torch.zeros(2), 6)
    with pytest.raises(ValueError, match="CUDA"):
        host.checked(p)
    x = torch.zeros(5100)
    with pytest.raises(ValueError, match="need a contiguous CUDA"):
        B.gc_dgc_step(p, x, x, x, 0.9, 0.0, 1, host, torch.zeros(16, dtype=torch.uint8))



def test_stream_probe_host_checks():
    """The streaming reference rejects bad arguments before enqueuing anything."""
    lib, fake = B.load(), ctypes.c_void_p(256)
    assert lib.gc_stream_probe(None, fake, fake, fake, fake, 1, None) == B.GC_EINVAL
    assert lib.gc_stream_probe(fake, fake, fake, fake, fake, 1 << 32, None) == B.GC_ERANGE
    assert lib.gc_stream_probe(fake, fake, ctypes.c_void_p(258), fake, fake, 8, None) == B.GC_EINVAL
    assert "aligned" in B.gc_last_error()
    assert lib.gc_stream_probe(fake, fake, fake, fake, fake, 0, None) == B.GC_OK  # nothing enqueued
