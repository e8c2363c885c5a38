"""ctypes binding of libgradcomp: the C-ABI calls under the same names.

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

GC_OK, GC_EINVAL, GC_ECAPACITY, GC_ERANGE, GC_EHIP, GC_ENOTSUP = 0, -1, -2, -3, -4, -5
GC_OP_DGC, GC_OP_ADACOMP, GC_OP_PACK, GC_OP_DECODE, GC_OP_UNPACK = 1, 2, 3, 4, 5
GC_KIND_DGC, GC_KIND_ADACOMP = 1, 2
GC_SUM, GC_AVG = 0, 1
GC_MOMENTUM_VANILLA, GC_MOMENTUM_NESTEROV = 0, 1
GC_SELECT_EXACT, GC_SELECT_SAMPLED = 0, 1
GC_ADACOMP_RULE_RESIDUAL, GC_ADACOMP_RULE_GRADIENT = 0, 1
GC_MAX_BIN_LEN = 4096
GC_MAX_MESSAGES = 64
GC_MAX_SEGMENT_LEN = 0xFFFC0000
GC_MAX_REPLICAS = 16

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgradcomp.so")


class GCError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libgradcomp status {status}: {msg}")
        self.status = status


class gc_segment(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("length", ctypes.c_uint32),
                ("bin_len", ctypes.c_uint32), ("k", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


class gc_sparse(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("val", ctypes.c_void_p),
                ("seg_off", ctypes.c_void_p), ("seg_scale", ctypes.c_void_p),
                ("cap", ctypes.c_uint64)]


class gc_dgc_options(ctypes.Structure):
    _fields_ = [("momentum", ctypes.c_float), ("thr_G", ctypes.c_float),
                ("num_nodes", ctypes.c_int), ("momentum_kind", ctypes.c_int),
                ("select", ctypes.c_int), ("sample_period", ctypes.c_uint32),
                ("over", ctypes.c_uint32), ("reserved", ctypes.c_uint32),
                ("density_num", ctypes.c_uint32), ("density_den", ctypes.c_uint32)]


class gc_adacomp_options(ctypes.Structure):
    _fields_ = [("scale_factor", ctypes.c_float), ("rule", ctypes.c_int),
                ("reserved", ctypes.c_uint32 * 2)]


_lib = None

# every symbol the header declares, with (restype, argtypes)
_P = ctypes.c_void_p
_SIGS = {
    "gc_last_error": (ctypes.c_char_p, []),
    "gc_version": (ctypes.c_char_p, []),
    "gc_plan_create": (ctypes.c_int, [_P, ctypes.c_int, ctypes.c_uint64, _P]),
    "gc_plan_destroy": (None, [_P]),
    "gc_plan_num_segments": (ctypes.c_int, [_P]),
    "gc_plan_num_elements": (ctypes.c_uint64, [_P]),
    "gc_plan_total_k": (ctypes.c_uint64, [_P]),
    "gc_plan_total_bins": (ctypes.c_uint64, [_P]),
    "gc_topk_count": (ctypes.c_uint32, [ctypes.c_uint32]),
    "gc_plan_workspace_bytes": (ctypes.c_size_t, [_P, ctypes.c_int]),
    "gc_adacomp_compress": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_size_t, ctypes.c_float, _P, _P,
                                           ctypes.c_size_t, _P]),
    "gc_dgc_pack_bound": (ctypes.c_uint64, [_P, _P]),
    "gc_adacomp_compress_ex": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_size_t, _P, _P, _P,
                                              ctypes.c_size_t, _P]),
    "gc_adacomp_state_bytes": (ctypes.c_size_t, [_P]),
    "gc_adacomp_message_cap": (ctypes.c_uint64, [_P]),
    "gc_plan_upload": (ctypes.c_int, [_P]),
    "gc_adacomp_residual": (ctypes.c_int, [_P, _P, _P, ctypes.c_size_t, _P, _P]),
    "gc_dgc_step": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                                   _P, _P, ctypes.c_size_t, _P]),
    "gc_dgc_message_cap": (ctypes.c_uint64, [_P, _P]),
    "gc_dgc_step_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "gc_pack_bound": (ctypes.c_uint64, [_P, ctypes.c_int]),
    "gc_pack": (ctypes.c_int, [_P, ctypes.c_int, _P, _P, ctypes.c_uint64, _P, _P, ctypes.c_size_t, _P]),
    "gc_unpack": (ctypes.c_int, [_P, ctypes.c_int, _P, ctypes.c_uint64, _P, _P, _P, ctypes.c_size_t, _P]),
    "gc_decompress_accumulate": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int,
                                                _P, ctypes.c_size_t, _P]),
    "gc_decompress_noalloc_max_chunks": (ctypes.c_uint64, [ctypes.c_int]),
    "gc_decompress_accumulate_noalloc": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, ctypes.c_int, ctypes.c_int,
                                                        _P]),
    "gc_dcd_compress": (ctypes.c_int, [_P, _P, _P, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32,
                                       ctypes.c_uint64, ctypes.c_uint64, _P, _P, _P]),
    "gc_dcd_decode": (ctypes.c_int, [_P, _P, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32, _P, _P]),
    "gc_dcd_mix": (ctypes.c_int, [_P, _P, ctypes.c_int, _P, ctypes.c_float, _P, ctypes.c_uint64, _P]),
    "gc_ecd_compress": (ctypes.c_int, [_P, _P, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int,
                                       ctypes.c_uint32, ctypes.c_uint64, _P, _P, _P]),
    "gc_ecd_update": (ctypes.c_int, [_P, _P, ctypes.c_uint64, ctypes.c_int, ctypes.c_uint32,
                                     ctypes.c_uint64, _P, _P]),
    "gc_slimdp_mask_words": (ctypes.c_uint64, [_P]),
    "gc_slimdp_core": (ctypes.c_int, [_P, _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_size_t, _P]),
    "gc_slimdp_explore": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_uint64, ctypes.c_uint64, _P, _P,
                                         ctypes.c_size_t, _P]),
    "gc_slimdp_core_values": (ctypes.c_int, [_P, _P, _P, _P, _P]),
    "gc_timing_enable": (ctypes.c_int, [ctypes.c_char_p]),
    "gc_timing_take": (ctypes.c_int, [ctypes.c_char_p, _P, _P]),
    "gc_stream_probe": (ctypes.c_int, [_P, _P, _P, _P, _P, ctypes.c_uint64, _P]),
}

KERNELS = ("dgc_norm", "dgc_prep", "dgc_prepare", "dgc_sample", "dgc_bound", "dgc_ssample", "dgc_squant", "dgc_update", "dgc_collect",
           "dgc_select", "dgc_stage", "dgc_refine", "dgc_sbase", "dgc_count", "dgc_scan", "dgc_emit", "ada_max", "ada_binsum", "ada_scale", "ada_offsets", "ada_apply",
           "ada_fold", "ada_emit", "ada_residual",
           "pack_plan", "pack_write", "pack_relayout", "pack_rewrite", "pack_main", "pack_fix", "unpack_layout",
           "unpack_write", "decode_index", "decode", "dcd",
           "dcd_decode", "dcd_mix", "ecd_compress", "ecd_update", "slimdp_values", "stream_probe")


def gc_timing_enable(kernels) -> None:
    """Bracket launches of the named kernels with HIP events ("*" = all,
    None or "" = off)."""
    if kernels is None:
        arg = None
    elif isinstance(kernels, str):
        arg = kernels.encode()
    else:
        arg = ",".join(kernels).encode()
    _check(load().gc_timing_enable(arg))


def gc_stream_probe(a, b, c, d, e) -> None:
    """The streaming reference: d = a + b, e = c + d over a.numel() fp32
    elements (three reads, two writes per element)."""
    n = a.numel()
    _check(load().gc_stream_probe(_f32(a, n, "a"), _f32(b, n, "b"), _f32(c, n, "c"), _f32(d, n, "d"),
                                  _f32(e, n, "e"), n, _stream(d)))


def gc_timing_take(kernel: str):
    """(total milliseconds, launches) recorded for a kernel since the last take."""
    ms = ctypes.c_double()
    n = ctypes.c_uint64()
    _check(load().gc_timing_take(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def load():
    """Load libgradcomp.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(status: int):
    if status != GC_OK:
        raise GCError(status, load().gc_last_error().decode())


def gc_version() -> str:
    return load().gc_version().decode()


def gc_last_error() -> str:
    return load().gc_last_error().decode()


def gc_topk_count(n: int) -> int:
    return int(load().gc_topk_count(int(n)))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# The C ABI trusts the sizes it is given; these checks make every pointer the
# binding passes down a contiguous CUDA tensor of the right type holding at
# least the elements the call may touch.
def _dev(t, dtype, n: int, name: str):
    if not torch.is_tensor(t) or t.dtype != dtype or not t.is_cuda or not t.is_contiguous() or t.numel() < n:
        raise ValueError(f"{name}: need a contiguous CUDA {str(dtype).replace('torch.', '')} tensor "
                         f"of >= {n} elements")
    return _ptr(t)


def _f32(t: torch.Tensor, n: int, name: str):
    return _dev(t, torch.float32, n, name)


def _ws(ws: torch.Tensor, name: str = "ws"):
    """A workspace: uint8, so that its element count is its byte count."""
    return _dev(ws, torch.uint8, 1, name), ws.numel()


def _state(state):
    return ctypes.c_void_p(0) if state is None else _dev(state, torch.uint8, 1, "state")


# ---------------------------------------------------------------- plans
class Plan:
    """A validated segment table (gc_plan)."""

    def __init__(self, table, n_total: int | None = None):
        t = np.asarray(table, dtype=np.int64).reshape(-1, 4)
        self.table = t
        self.n_total = int(n_total if n_total is not None else (t[-1, 0] + t[-1, 1] if len(t) else 0))
        arr = (gc_segment * max(len(t), 1))()
        for i, (o, n, lt, k) in enumerate(t):
            arr[i] = gc_segment(int(o), int(n), int(lt), int(k), 0)
        h = ctypes.c_void_p()
        _check(load().gc_plan_create(arr, len(t), self.n_total, ctypes.byref(h)))
        self.handle = h
        self.nseg = len(t)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.gc_plan_destroy(h)
            self.handle = None

    @property
    def total_k(self) -> int:
        return int(load().gc_plan_total_k(self.handle))

    @property
    def total_bins(self) -> int:
        return int(load().gc_plan_total_bins(self.handle))

    def upload(self) -> None:
        """Put the plan's tables on the current device (gc_plan_upload)."""
        _check(load().gc_plan_upload(self.handle))

    def workspace_bytes(self, op: int) -> int:
        return int(load().gc_plan_workspace_bytes(self.handle, op))

    def workspace(self, op: int, device="cuda") -> torch.Tensor:
        return torch.empty(max(self.workspace_bytes(op), 1), dtype=torch.uint8, device=device)

    def pack_bound(self, kind: int) -> int:
        return int(load().gc_pack_bound(self.handle, kind))

    @property
    def adacomp_state_bytes(self) -> int:
        return int(load().gc_adacomp_state_bytes(self.handle))

    def adacomp_state(self, device="cuda") -> torch.Tensor:
        """A zero-filled deferred-residual state for one learner (torch
        allocations are 256-byte aligned)."""
        return torch.zeros(max(self.adacomp_state_bytes, 1), dtype=torch.uint8, device=device)


def gc_plan_create(table, n_total=None) -> Plan:
    return Plan(table, n_total)


def gc_plan_workspace_bytes(plan: Plan, op: int) -> int:
    return plan.workspace_bytes(op)


def gc_pack_bound(plan: Plan, kind: int) -> int:
    return plan.pack_bound(kind)


@dataclass
class Sparse:
    """A message: device tensors idx (int32 holding u32), val, seg_off, seg_scale."""
    idx: torch.Tensor
    val: torch.Tensor
    seg_off: torch.Tensor
    seg_scale: torch.Tensor
    cap: int

    @staticmethod
    def empty(plan: Plan, cap: int, device="cuda") -> "Sparse":
        return Sparse(torch.zeros(max(cap, 1), dtype=torch.int32, device=device),
                      torch.zeros(max(cap, 1), dtype=torch.float32, device=device),
                      torch.zeros(plan.nseg + 1, dtype=torch.int32, device=device),
                      torch.zeros(max(plan.nseg, 1), dtype=torch.float32, device=device), cap)

    def struct(self) -> gc_sparse:
        return gc_sparse(self.idx.data_ptr(), self.val.data_ptr(), self.seg_off.data_ptr(),
                         self.seg_scale.data_ptr(), self.cap)

    def checked(self, plan: "Plan", name: str = "message") -> gc_sparse:
        """The struct, after checking that the tensors hold cap entries and
        the plan's per-segment arrays."""
        _dev(self.idx, torch.int32, self.cap, f"{name}.idx")
        _dev(self.val, torch.float32, self.cap, f"{name}.val")
        _dev(self.seg_off, torch.int32, plan.nseg + 1, f"{name}.seg_off")
        _dev(self.seg_scale, torch.float32, max(plan.nseg, 1), f"{name}.seg_scale")
        return self.struct()

    def count(self) -> int:
        return int(self.seg_off[-1].item())

    def host(self):
        """(idx u32, val f32, seg_off u32, seg_scale f32) as NumPy arrays."""
        n = self.count()
        return (self.idx[:n].cpu().numpy().view(np.uint32), self.val[:n].cpu().numpy(),
                self.seg_off.cpu().numpy().view(np.uint32), self.seg_scale.cpu().numpy())


# -------------------------------------------------------------- hot calls
def gc_adacomp_compress(plan: Plan, dW, R, scale_factor: float, out: Sparse, ws: torch.Tensor,
                        state: torch.Tensor | None = None, rule: int | None = None):
    """state None: R is the exact residual.  state (Plan.adacomp_state()):
    deferred mode, the residual is (R, state).  rule None:
    gc_adacomp_compress (the default reading); else gc_adacomp_compress_ex
    with that GC_ADACOMP_RULE_*."""
    n = plan.n_total
    msg = out.checked(plan, "out")
    args = (plan.handle, _f32(dW, n, "dW"), _f32(R, n, "R"), _state(state),
            state.numel() if state is not None else 0)
    if rule is None:
        _check(load().gc_adacomp_compress(*args, float(scale_factor), ctypes.byref(msg), *_ws(ws), _stream(R)))
    else:
        opt = gc_adacomp_options(float(scale_factor), int(rule))
        _check(load().gc_adacomp_compress_ex(*args, ctypes.byref(opt), ctypes.byref(msg), *_ws(ws), _stream(R)))


def gc_adacomp_message_cap(plan: Plan) -> int:
    """Slots an AdaComp message needs: the sum of the segment lengths."""
    return int(load().gc_adacomp_message_cap(plan.handle))


def gc_adacomp_state_bytes(plan: Plan) -> int:
    return plan.adacomp_state_bytes


def gc_adacomp_residual(plan: Plan, R, state: torch.Tensor | None, R_out):
    n = plan.n_total
    _check(load().gc_adacomp_residual(plan.handle, _f32(R, n, "R"), _state(state),
                                      state.numel() if state is not None else 0,
                                      _f32(R_out, n, "R_out"), _stream(R_out)))


def gc_dgc_step(plan: Plan, G, U, V, momentum: float, thr_G: float, num_nodes: int, out: Sparse,
                ws: torch.Tensor):
    n = plan.n_total
    msg = out.checked(plan, "out")
    _check(load().gc_dgc_step(plan.handle, _f32(G, n, "G"), _f32(U, n, "U"), _f32(V, n, "V"),
                              float(momentum), float(thr_G), int(num_nodes), ctypes.byref(msg),
                              *_ws(ws), _stream(V)))


def dgc_options(momentum: float, thr_G: float = 0.0, num_nodes: int = 1, nesterov: bool = False,
                sampled: bool = False, sample_period: int = 100, over: int = 2,
                density: tuple[int, int] | None = None) -> gc_dgc_options:
    """density=(num, den): this call keeps ceil(n_s num / den) entries per
    segment instead of the plan's k (warm-up)."""
    num, den = density if density is not None else (0, 0)
    return gc_dgc_options(float(momentum), float(thr_G), int(num_nodes),
                          GC_MOMENTUM_NESTEROV if nesterov else GC_MOMENTUM_VANILLA,
                          GC_SELECT_SAMPLED if sampled else GC_SELECT_EXACT,
                          int(sample_period), int(over), 0, int(num), int(den))


def gc_dgc_message_cap(plan: Plan, opt: gc_dgc_options) -> int:
    return int(load().gc_dgc_message_cap(plan.handle, ctypes.byref(opt)))


def gc_dgc_pack_bound(plan: Plan, opt: gc_dgc_options | None) -> int:
    return int(load().gc_dgc_pack_bound(plan.handle, ctypes.byref(opt) if opt is not None else None))


def gc_dgc_step_ex(plan: Plan, G, U, V, opt: gc_dgc_options, out: Sparse, ws: torch.Tensor):
    n = plan.n_total
    msg = out.checked(plan, "out")
    _check(load().gc_dgc_step_ex(plan.handle, _f32(G, n, "G"), _f32(U, n, "U"), _f32(V, n, "V"),
                                 ctypes.byref(opt), ctypes.byref(msg), *_ws(ws), _stream(V)))


def gc_pack(plan: Plan, kind: int, msg: Sparse, out: torch.Tensor, out_bytes: torch.Tensor,
            ws: torch.Tensor):
    if out.dtype != torch.uint8 or out_bytes.dtype != torch.int64:
        raise ValueError("gc_pack: out must be uint8 and out_bytes int64 (holding u64)")
    m = msg.checked(plan, "msg")
    _check(load().gc_pack(plan.handle, int(kind), ctypes.byref(m), _dev(out, torch.uint8, 1, "out"), out.numel(),
                          _dev(out_bytes, torch.int64, 1, "out_bytes"), *_ws(ws), _stream(out)))


def gc_unpack(plan: Plan, kind: int, data: torch.Tensor, nbytes: int, out: Sparse, status: torch.Tensor,
              ws: torch.Tensor):
    """data: uint8 device tensor holding the stream's nbytes bytes; status:
    an int32 device tensor (holding u32) that receives the stream's status."""
    if data.dtype != torch.uint8 or data.numel() < nbytes or status.dtype != torch.int32:
        raise ValueError("gc_unpack: data must be uint8 with nbytes bytes, status int32")
    m = out.checked(plan, "out")
    _check(load().gc_unpack(plan.handle, int(kind), _dev(data, torch.uint8, nbytes, "data"), int(nbytes), ctypes.byref(m), _dev(status, torch.int32, 1, "status"),
                            *_ws(ws), _stream(data)))


def gc_decompress_accumulate(plan: Plan, msgs, dense, mode: int, accumulate: bool,
                             ws: torch.Tensor):
    K = len(msgs)
    arr = (gc_sparse * max(K, 1))(*[m.checked(plan, f"msgs[{i}]") for i, m in enumerate(msgs)])
    _check(load().gc_decompress_accumulate(plan.handle, arr, K, _f32(dense, plan.n_total, "dense"),
                                           int(mode), int(bool(accumulate)), *_ws(ws),
                                           _stream(dense)))


def gc_decompress_noalloc_max_chunks(K: int) -> int:
    return int(load().gc_decompress_noalloc_max_chunks(int(K)))


def gc_decompress_accumulate_noalloc(plan: Plan, msgs, dense, mode: int, accumulate: bool):
    """gc_decompress_accumulate with the library's fixed device scratch in
    place of a workspace; the plan must have been uploaded (Plan.upload)."""
    K = len(msgs)
    arr = (gc_sparse * max(K, 1))(*[m.checked(plan, f"msgs[{i}]") for i, m in enumerate(msgs)])
    _check(load().gc_decompress_accumulate_noalloc(plan.handle, arr, K, _f32(dense, plan.n_total, "dense"),
                                                   int(mode), int(bool(accumulate)), _stream(dense)))


def gc_dcd_compress(x, x_half, x_out, bits: int, bucket: int, seed: int, step: int,
                    scales: torch.Tensor, codes: torch.Tensor):
    n = x.numel()
    nb = (n + bucket - 1) // bucket
    if scales.numel() < nb or codes.numel() < (n * bits + 7) // 8 or codes.dtype != torch.uint8:
        raise ValueError("gc_dcd_compress: scales or codes too small")
    _check(load().gc_dcd_compress(_f32(x, n, "x"), _f32(x_half, n, "x_half"), _f32(x_out, n, "x_out"),
                                  n, int(bits), int(bucket), int(seed) & (2 ** 64 - 1),
                                  int(step) & (2 ** 64 - 1), _f32(scales, nb, "scales"), _dev(codes, torch.uint8, (n * bits + 7) // 8, "codes"),
                                  _stream(x_out)))


def _codes_check(n: int, bits: int, bucket: int, scales: torch.Tensor, codes: torch.Tensor, fn: str):
    nb = (n + bucket - 1) // bucket
    if scales.numel() < nb or codes.numel() < (n * bits + 7) // 8 or codes.dtype != torch.uint8:
        raise ValueError(f"{fn}: scales or codes too small")
    return nb


def gc_dcd_decode(scales: torch.Tensor, codes: torch.Tensor, x_hat, bits: int, bucket: int):
    n = x_hat.numel()
    nb = _codes_check(n, bits, bucket, scales, codes, "gc_dcd_decode")
    _check(load().gc_dcd_decode(_f32(scales, nb, "scales"), _dev(codes, torch.uint8, (n * bits + 7) // 8, "codes"), n, int(bits), int(bucket),
                                _f32(x_hat, n, "x_hat"), _stream(x_hat)))


def gc_dcd_mix(replicas, weights, grad, lr: float, x_half):
    n = x_half.numel()
    K = len(replicas)
    reps = (ctypes.c_void_p * max(K, 1))(*[_f32(r, n, "replica").value for r in replicas])
    w = (ctypes.c_float * max(K, 1))(*[float(v) for v in weights])
    _check(load().gc_dcd_mix(reps, w, K, _f32(grad, n, "grad"), float(lr), _f32(x_half, n, "x_half"), n,
                             _stream(x_half)))


def gc_ecd_compress(x_prev, x, t: int, bits: int, bucket: int, seed: int, scales: torch.Tensor,
                    codes: torch.Tensor):
    n = x.numel()
    nb = _codes_check(n, bits, bucket, scales, codes, "gc_ecd_compress")
    _check(load().gc_ecd_compress(_f32(x_prev, n, "x_prev"), _f32(x, n, "x"), n, int(t), int(bits),
                                  int(bucket), int(seed) & (2 ** 64 - 1), _f32(scales, nb, "scales"),
                                  _dev(codes, torch.uint8, (n * bits + 7) // 8, "codes"), _stream(x)))


def gc_ecd_update(scales: torch.Tensor, codes: torch.Tensor, x_tilde, t: int, bits: int, bucket: int):
    n = x_tilde.numel()
    nb = _codes_check(n, bits, bucket, scales, codes, "gc_ecd_update")
    _check(load().gc_ecd_update(_f32(scales, nb, "scales"), _dev(codes, torch.uint8, (n * bits + 7) // 8, "codes"), n, int(bits), int(bucket), int(t),
                                _f32(x_tilde, n, "x_tilde"), _stream(x_tilde)))


def gc_slimdp_mask_words(plan: Plan) -> int:
    return int(load().gc_slimdp_mask_words(plan.handle))


def gc_slimdp_core(plan: Plan, w, g, c: float, core: Sparse, core_mask: torch.Tensor, ws: torch.Tensor):
    n = plan.n_total
    if core_mask.dtype != torch.int32 or core_mask.numel() < gc_slimdp_mask_words(plan):
        raise ValueError("gc_slimdp_core: core_mask must be int32 (holding u32) of gc_slimdp_mask_words words")
    msg = core.checked(plan, "core")
    _check(load().gc_slimdp_core(plan.handle, _f32(w, n, "w"), _f32(g, n, "g"), float(c), ctypes.byref(msg),
                                 _dev(core_mask, torch.int32, gc_slimdp_mask_words(plan), "core_mask"), *_ws(ws), _stream(core_mask)))


def gc_slimdp_explore(plan: Plan, core_plan: Plan, delta, core_mask: torch.Tensor, seed: int, step: int,
                      out: Sparse, ws: torch.Tensor):
    n = plan.n_total
    msg = out.checked(plan, "out")
    _check(load().gc_slimdp_explore(plan.handle, core_plan.handle, _f32(delta, n, "delta"), _dev(core_mask, torch.int32, gc_slimdp_mask_words(plan), "core_mask"),
                                    int(seed) & (2 ** 64 - 1), int(step) & (2 ** 64 - 1), ctypes.byref(msg),
                                    *_ws(ws), _stream(delta)))


def gc_slimdp_core_values(core_plan: Plan, core: Sparse, delta, values):
    msg = core.checked(core_plan, "core")
    _check(load().gc_slimdp_core_values(core_plan.handle, ctypes.byref(msg), _f32(delta, core_plan.n_total, "delta"),
                                        _f32(values, core_plan.total_k, "values"), _stream(values)))
