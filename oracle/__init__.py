"""Oracle for libgradcomp — TEST INFRASTRUCTURE ONLY.

A plain CPU definition of every result of the compression path, written in C
(``oracle.c``) and called through ctypes.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.  It
shares no code with the HIP path and never imports the product package.

Functions take and return NumPy arrays.  A "segment table" is an (nseg, 4)
integer array of (offset, length, bin_len, k) rows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
          "-fno-fast-math", "-fopenmp", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain IEEE arithmetic, no contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _DgcOpts(ctypes.Structure):
    _fields_ = [("momentum", ctypes.c_float), ("thr_G", ctypes.c_float),
                ("num_nodes", ctypes.c_int), ("nesterov", ctypes.c_int),
                ("sampled", ctypes.c_int), ("sample_period", ctypes.c_uint32),
                ("over", ctypes.c_uint32), ("pad", ctypes.c_uint32)]


class _Seg(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("length", ctypes.c_uint32),
                ("bin_len", ctypes.c_uint32), ("k", ctypes.c_uint32),
                ("pad", ctypes.c_uint32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")  # another build of oracle.c (the sanitizer check's)
        if not path:
            if not os.path.exists(_LIB):
                build(force=False)
            path = _LIB
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        L.orc_psum64.restype = ctypes.c_double
        L.orc_psum64.argtypes = [P, ctypes.c_uint64]
        L.orc_adacomp.argtypes = [P, ctypes.c_int, P, P, ctypes.c_float, P, P, P, P, P]
        L.orc_adacomp_rule.argtypes = [P, ctypes.c_int, P, P, ctypes.c_float, ctypes.c_int, P, P, P, P, P]
        L.orc_dgc.argtypes = [P, ctypes.c_int, P, P, P, ctypes.c_float, ctypes.c_float,
                              ctypes.c_int, P, P, P, P]
        L.orc_dgc_ex.argtypes = [P, ctypes.c_int, P, P, P, P, P, P, P, P]
        L.orc_pack.restype = ctypes.c_uint64
        L.orc_pack.argtypes = [ctypes.c_int, P, ctypes.c_int, P, P, P, P, P, ctypes.c_uint64]
        L.orc_unpack.restype = ctypes.c_int
        L.orc_unpack.argtypes = [ctypes.c_int, P, ctypes.c_int, P, ctypes.c_uint64, P, P, P, P,
                                 ctypes.c_uint64]
        L.orc_decode.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P, P,
                                 ctypes.c_int, ctypes.c_int]
        L.orc_philox4x32_10.argtypes = [P, P, P]
        L.orc_dcd.argtypes = [P, P, P, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32,
                              ctypes.c_uint64, ctypes.c_uint64, P, P]
        L.orc_dcd_window.argtypes = [P, P, P, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32,
                                     ctypes.c_uint64, ctypes.c_uint64, P, P]
        L.orc_dcd_decode.argtypes = [P, P, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32, P]
        L.orc_dcd_mix.argtypes = [ctypes.c_int, P, P, P, ctypes.c_float, P, ctypes.c_uint64]
        L.orc_ecd_compress.argtypes = [P, P, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                       ctypes.c_uint32, ctypes.c_uint64, P, P]
        L.orc_ecd_update.argtypes = [P, P, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32,
                                     ctypes.c_uint64, P]
        L.orc_slimdp_core.argtypes = [P, ctypes.c_int, P, P, ctypes.c_float, P, P, P, P]
        L.orc_slimdp_explore.argtypes = [P, ctypes.c_int, P, P, ctypes.c_uint64, ctypes.c_uint64,
                                         P, P, P]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_num_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _segs(table) -> ctypes.Array:
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    arr = (_Seg * max(len(t), 1))()
    for i, (o, n, lt, k) in enumerate(t):
        arr[i] = _Seg(int(o), int(n), int(lt), int(k), 0)
    return arr


def _f32(a, copy=False):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a.copy() if copy else a


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def psum64(x) -> float:
    """Pairwise fp64 sum over the zero-padded power-of-two tree."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    return lib().orc_psum64(_ptr(x), x.size)


# AdaComp threshold readings (oracle.c): the factor on the accumulated
# residual (the default), or on the new gradient with the bin max always sent
RULE_RESIDUAL = 0
RULE_GRADIENT = 1


def adacomp(table, dW, R, scale_factor=2.0, rule=RULE_RESIDUAL):
    """One AdaComp step.  Returns (R_new, idx, val, seg_off, seg_scale, gmax)."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    dW = _f32(dW)
    R = _f32(R, copy=True)
    n_entries_max = int(t[:, 1].sum()) if len(t) else 0
    nbins = int(((t[:, 1] + t[:, 2] - 1) // t[:, 2]).sum()) if len(t) else 0
    idx = np.zeros(max(n_entries_max, 1), np.uint32)
    val = np.zeros(max(n_entries_max, 1), np.float32)
    seg_off = np.zeros(len(t) + 1, np.uint32)
    seg_scale = np.zeros(max(len(t), 1), np.float32)
    gmax = np.zeros(max(nbins, 1), np.float32)
    lib().orc_adacomp_rule(_segs(t), len(t), _ptr(dW), _ptr(R), float(scale_factor), int(rule), _ptr(idx),
                           _ptr(val), _ptr(seg_off), _ptr(seg_scale), _ptr(gmax))
    m = int(seg_off[-1])
    return R, idx[:m].copy(), val[:m].copy(), seg_off, seg_scale[:len(t)], gmax[:nbins]


def dgc(table, G, U, V, momentum=0.9, thr_G=0.0, num_nodes=1):
    """One DGC step.  Returns (U_new, V_new, idx, val, seg_off, clip)."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    G = _f32(G)
    U = _f32(U, copy=True)
    V = _f32(V, copy=True)
    ktot = int(t[:, 3].sum()) if len(t) else 0
    idx = np.zeros(max(ktot, 1), np.uint32)
    val = np.zeros(max(ktot, 1), np.float32)
    seg_off = np.zeros(len(t) + 1, np.uint32)
    clip = np.zeros(max(len(t), 1), np.float32)
    lib().orc_dgc(_segs(t), len(t), _ptr(G), _ptr(U), _ptr(V), float(momentum), float(thr_G),
                  int(num_nodes), _ptr(idx), _ptr(val), _ptr(seg_off), _ptr(clip))
    return U, V, idx[:ktot].copy(), val[:ktot].copy(), seg_off, clip[:len(t)]


def dgc_ex(table, G, U, V, momentum=0.9, thr_G=0.0, num_nodes=1, nesterov=False,
           sampled=False, sample_period=100, over=2):
    """One DGC step with the momentum kind and selection mode chosen.
    Returns (U_new, V_new, idx, val, seg_off, clip); the message is compact."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    G = _f32(G)
    U = _f32(U, copy=True)
    V = _f32(V, copy=True)
    if sampled:
        cap = int(np.minimum(t[:, 1], int(over) * t[:, 3]).sum()) if len(t) else 0
    else:
        cap = int(t[:, 3].sum()) if len(t) else 0
    idx = np.zeros(max(cap, 1), np.uint32)
    val = np.zeros(max(cap, 1), np.float32)
    seg_off = np.zeros(len(t) + 1, np.uint32)
    clip = np.zeros(max(len(t), 1), np.float32)
    o = _DgcOpts(float(momentum), float(thr_G), int(num_nodes), int(bool(nesterov)),
                 int(bool(sampled)), int(sample_period), int(over), 0)
    lib().orc_dgc_ex(_segs(t), len(t), _ptr(G), _ptr(U), _ptr(V), ctypes.byref(o), _ptr(idx),
                     _ptr(val), _ptr(seg_off), _ptr(clip))
    m = int(seg_off[-1])
    return U, V, idx[:m].copy(), val[:m].copy(), seg_off, clip[:len(t)]


def pack(kind, table, idx, val, seg_off, seg_scale=None, cap=None) -> bytes:
    """Run-length pack a message; kind 1 = DGC, 2 = AdaComp."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    idx = np.ascontiguousarray(idx, dtype=np.uint32)
    val = _f32(val)
    seg_off = np.ascontiguousarray(seg_off, dtype=np.uint32)
    sc = _f32(seg_scale if seg_scale is not None else np.zeros(max(len(t), 1)))
    if cap is None:
        MAX = 65535 if kind == 1 else 32767
        per = 6 if kind == 1 else 2
        cap = 16
        for s in range(len(t)):
            codes = int(seg_off[s + 1] - seg_off[s]) + int(t[s, 1]) // MAX + 1  # at most
            cap += 16 + 16 + 2 + per * codes + 8 * ((codes + 4095) // 4096)
    out = np.zeros(int(cap), np.uint8)
    nbytes = lib().orc_pack(int(kind), _segs(t), len(t), _ptr(idx), _ptr(val), _ptr(seg_off),
                            _ptr(sc), _ptr(out), int(cap))
    if nbytes == 0:
        raise ValueError("capacity too small")
    return out[:nbytes].tobytes()


def unpack(kind, table, data: bytes, cap=None):
    """Read a packed stream back.  Returns (status, idx, val, seg_off, seg_scale);
    status 0 for a stream that fits the plan."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    buf = np.frombuffer(bytes(data), dtype=np.uint8).copy() if len(data) else np.zeros(1, np.uint8)
    if cap is None:
        cap = int(t[:, 1].sum()) if len(t) else 0
    idx = np.zeros(max(cap, 1), np.uint32)
    val = np.zeros(max(cap, 1), np.float32)
    seg_off = np.zeros(len(t) + 1, np.uint32)
    seg_scale = np.zeros(max(len(t), 1), np.float32)
    st = lib().orc_unpack(int(kind), _segs(t), len(t), _ptr(buf), len(data), _ptr(idx), _ptr(val),
                          _ptr(seg_off), _ptr(seg_scale), int(cap))
    m = int(seg_off[-1]) if st == 0 else 0
    return st, idx[:m].copy(), val[:m].copy(), seg_off, seg_scale[:len(t)]


def decode(table, n_total, messages, mode=1, dense=None):
    """Aggregate messages [(idx, val), ...] in order; mode 0 sum, 1 average.
    With ``dense`` given, the result is added into a copy of it."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    K = len(messages)
    idxs = [np.ascontiguousarray(m[0], dtype=np.uint32) for m in messages]
    vals = [_f32(m[1]) for m in messages]
    ip = (ctypes.c_void_p * max(K, 1))(*[i.ctypes.data for i in idxs])
    vp = (ctypes.c_void_p * max(K, 1))(*[v.ctypes.data for v in vals])
    cnt = np.array([i.size for i in idxs] or [0], dtype=np.uint64)
    acc = dense is not None
    out = _f32(dense, copy=True) if acc else np.zeros(int(n_total), np.float32)
    lib().orc_decode(_segs(t), len(t), K, ip, vp, _ptr(cnt), _ptr(out), int(mode), int(acc))
    return out


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def dcd(x, x_half, bits=4, bucket=512, seed=0, step=0):
    """Returns (x_out, scales, codes)."""
    x = _f32(x)
    xh = _f32(x_half)
    n = x.size
    xo = np.empty(n, np.float32)
    scales = np.zeros(max((n + bucket - 1) // bucket, 1), np.float32)
    codes = np.zeros(max((n * bits + 7) // 8, 1), np.uint8)
    lib().orc_dcd(_ptr(x), _ptr(xh), _ptr(xo), n, int(bits), int(bucket), int(seed) & (2**64 - 1),
                  int(step) & (2**64 - 1), _ptr(scales), _ptr(codes))
    return xo, scales[:(n + bucket - 1) // bucket], codes[:(n * bits + 7) // 8]


def dcd_window(x, x_half, base, bits=4, bucket=512, seed=0, step=0):
    """dcd() for elements [base, base + len(x)) of a longer model (base a
    multiple of bucket): buckets and Philox counters follow the model's
    indices.  Returns (x_out, scales, codes) of the window."""
    if base % bucket:
        raise ValueError("base must be a multiple of bucket")
    x = _f32(x)
    xh = _f32(x_half)
    m = x.size
    xo = np.empty(m, np.float32)
    scales = np.zeros(max((m + bucket - 1) // bucket, 1), np.float32)
    codes = np.zeros(max((m * bits + 7) // 8, 1), np.uint8)
    lib().orc_dcd_window(_ptr(x), _ptr(xh), _ptr(xo), m, int(base), int(bits), int(bucket),
                         int(seed) & (2**64 - 1), int(step) & (2**64 - 1), _ptr(scales), _ptr(codes))
    return xo, scales[:(m + bucket - 1) // bucket], codes[:(m * bits + 7) // 8]


def dcd_decode(scales, codes, x_hat, bits=4, bucket=512):
    """DCD-PSGD step 3 on a copy of x_hat: x_hat + C(z)."""
    xh = _f32(x_hat, copy=True)
    sc = _f32(scales)
    cd = np.ascontiguousarray(codes, dtype=np.uint8)
    lib().orc_dcd_decode(_ptr(sc), _ptr(cd), xh.size, int(bits), int(bucket), _ptr(xh))
    return xh


def dcd_mix(replicas, weights, grad, lr):
    """DCD-PSGD step 1: sum_j weights[j] * replicas[j] (in order) - lr * grad."""
    reps = [_f32(r) for r in replicas]
    K = len(reps)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    g = _f32(grad)
    out = np.empty(g.size, np.float32)
    rp = (ctypes.c_void_p * max(K, 1))(*[r.ctypes.data for r in reps])
    lib().orc_dcd_mix(K, rp, _ptr(w), _ptr(g), float(lr), _ptr(out), g.size)
    return out


def ecd_compress(x_prev, x, t, bits=4, bucket=512, seed=0):
    """ECD-PSGD Eq. (3): (scales, codes) of C((1 - t/2) x_prev + (t/2) x)."""
    xp = _f32(x_prev)
    xx = _f32(x)
    n = xx.size
    scales = np.zeros(max((n + bucket - 1) // bucket, 1), np.float32)
    codes = np.zeros(max((n * bits + 7) // 8, 1), np.uint8)
    lib().orc_ecd_compress(_ptr(xp), _ptr(xx), n, int(t), int(bits), int(bucket),
                           int(seed) & (2**64 - 1), _ptr(scales), _ptr(codes))
    return scales[:(n + bucket - 1) // bucket], codes[:(n * bits + 7) // 8]


def ecd_update(scales, codes, x_tilde, t, bits=4, bucket=512):
    """ECD-PSGD Eq. (4) on a copy of x_tilde."""
    xt = _f32(x_tilde, copy=True)
    sc = _f32(scales)
    cd = np.ascontiguousarray(codes, dtype=np.uint8)
    lib().orc_ecd_update(_ptr(sc), _ptr(cd), xt.size, int(bits), int(bucket), int(t), _ptr(xt))
    return xt


def mask_words(table) -> int:
    """Words of a Slim-DP core bitmap: ceil(n_s / 32) per segment."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    return int(((t[:, 1] + 31) // 32).sum())


def slimdp_core(table, w, g, c):
    """Returns (core_idx, core_val (= S), seg_off, mask)."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    w = _f32(w)
    g = _f32(g)
    K = int(t[:, 3].sum())
    idx = np.zeros(max(K, 1), np.uint32)
    val = np.zeros(max(K, 1), np.float32)
    off = np.zeros(len(t) + 1, np.uint32)
    mask = np.zeros(max(mask_words(t), 1), np.uint32)
    lib().orc_slimdp_core(_segs(t), len(t), _ptr(w), _ptr(g), float(c), _ptr(idx), _ptr(val),
                          _ptr(off), _ptr(mask))
    return idx[:K].copy(), val[:K].copy(), off, mask[:mask_words(t)].copy()


def slimdp_explore(table, delta, mask, seed, step):
    """Returns (idx, val (= delta at idx), seg_off)."""
    t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
    d = _f32(delta)
    mk = np.ascontiguousarray(mask, dtype=np.uint32)
    K = int(t[:, 3].sum())
    idx = np.zeros(max(K, 1), np.uint32)
    val = np.zeros(max(K, 1), np.float32)
    off = np.zeros(len(t) + 1, np.uint32)
    lib().orc_slimdp_explore(_segs(t), len(t), _ptr(d), _ptr(mk), int(seed) & (2**64 - 1),
                             int(step) & (2**64 - 1), _ptr(idx), _ptr(val), _ptr(off))
    return idx[:K].copy(), val[:K].copy(), off
