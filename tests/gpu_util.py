"""Helpers for GPU parity tests: run the HIP path through the C ABI and
return NumPy results comparable with the oracle's."""
import sys

import numpy as np
import torch

from gradient_compression_dnn_amd import binding as B


def say(msg: str):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev(), dtype=dtype)


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def same_bits(a, b) -> bool:
    return np.array_equal(bits(a), bits(b))


def ulp_report(a, b) -> str:
    a, b = np.asarray(a, np.float32), np.asarray(b, np.float32)
    bad = np.nonzero(bits(a) != bits(b))[0]
    if bad.size == 0:
        return "identical"
    i = bad[0]
    return f"{bad.size} differ; first at {i}: {a[i]!r} vs {b[i]!r}"


class HipPath:
    """One plan with its workspaces and message buffers on cuda:0."""

    def __init__(self, table, n_total=None):
        self.plan = B.Plan(table, n_total)
        self.n = self.plan.n_total
        self.ws = {}

    def workspace(self, op):
        if op not in self.ws:
            self.ws[op] = self.plan.workspace(op, dev())
        return self.ws[op]

    def dgc(self, G, U, V, momentum=0.9, thr_G=0.0, num_nodes=1, tensors=False):
        Gd, Ud, Vd = (x if torch.is_tensor(x) else to_dev(x) for x in (G, U, V))
        out = B.Sparse.empty(self.plan, self.plan.total_k, dev())
        B.gc_dgc_step(self.plan, Gd, Ud, Vd, momentum, thr_G, num_nodes, out,
                      self.workspace(B.GC_OP_DGC))
        torch.cuda.synchronize()
        if tensors:
            return Ud, Vd, out
        idx, val, off, _ = out.host()
        return Ud.cpu().numpy(), Vd.cpu().numpy(), idx, val, off

    def dgc_ex(self, G, U, V, opt, tensors=False):
        """gc_dgc_step_ex with a gc_dgc_options struct (binding.dgc_options)."""
        Gd, Ud, Vd = (x if torch.is_tensor(x) else to_dev(x) for x in (G, U, V))
        out = B.Sparse.empty(self.plan, B.gc_dgc_message_cap(self.plan, opt), dev())
        B.gc_dgc_step_ex(self.plan, Gd, Ud, Vd, opt, out, self.workspace(B.GC_OP_DGC))
        torch.cuda.synchronize()
        if tensors:
            return Ud, Vd, out
        idx, val, off, _ = out.host()
        return Ud.cpu().numpy(), Vd.cpu().numpy(), idx, val, off

    def adacomp(self, dW, R, scale_factor=2.0, tensors=False, state=None, rule=None):
        """One AdaComp call; with `state` (a deferred-residual state tensor) the
        returned R is the exact residual, materialized by gc_adacomp_residual,
        while the device R keeps the deferred form.  rule: a GC_ADACOMP_RULE_*
        for gc_adacomp_compress_ex, None for gc_adacomp_compress."""
        dWd = dW if torch.is_tensor(dW) else to_dev(dW)
        Rd = R if torch.is_tensor(R) else to_dev(R)
        out = B.Sparse.empty(self.plan, self.n, dev())
        B.gc_adacomp_compress(self.plan, dWd, Rd, scale_factor, out, self.workspace(B.GC_OP_ADACOMP),
                              state=state, rule=rule)
        torch.cuda.synchronize()
        if state is not None and not tensors:
            exact = torch.empty_like(Rd)
            B.gc_adacomp_residual(self.plan, Rd, state, exact)
            torch.cuda.synchronize()
            idx, val, off, scale = out.host()
            return exact.cpu().numpy(), idx, val, off, scale[:self.plan.nseg]
        if tensors:
            return Rd, out
        idx, val, off, scale = out.host()
        return Rd.cpu().numpy(), idx, val, off, scale[:self.plan.nseg]

    def pack(self, kind, msg: "B.Sparse"):
        cap = self.plan.pack_bound(kind)
        out = torch.zeros(cap, dtype=torch.uint8, device=dev())
        nbytes = torch.zeros(1, dtype=torch.int64, device=dev())
        B.gc_pack(self.plan, kind, msg, out, nbytes, self.workspace(B.GC_OP_PACK))
        torch.cuda.synchronize()
        nb = int(nbytes.item())
        return out[:nb].cpu().numpy().tobytes()

    def decode(self, msgs, mode=B.GC_AVG, dense=None):
        acc = dense is not None
        d = to_dev(dense) if acc else torch.zeros(self.n, dtype=torch.float32, device=dev())
        B.gc_decompress_accumulate(self.plan, msgs, d, mode, acc, self.workspace(B.GC_OP_DECODE))
        torch.cuda.synchronize()
        return d.cpu().numpy()


def sparse_from_host(plan: "B.Plan", idx, val, seg_off, seg_scale=None) -> "B.Sparse":
    cap = max(len(idx), 1)
    s = B.Sparse.empty(plan, cap, dev())
    if len(idx):
        s.idx[:len(idx)] = torch.from_numpy(np.asarray(idx, np.uint32).view(np.int32)).to(dev())
        s.val[:len(idx)] = torch.from_numpy(np.asarray(val, np.float32)).to(dev())
    s.seg_off[:] = torch.from_numpy(np.asarray(seg_off, np.uint32).view(np.int32)).to(dev())
    if seg_scale is not None and len(seg_scale):
        s.seg_scale[:len(seg_scale)] = torch.from_numpy(np.asarray(seg_scale, np.float32)).to(dev())
    return s


def dcd(x, xh, bits_, bucket, seed, step, offset=0, inplace=False):
    """Run gc_dcd_compress; offset > 0 shifts every buffer to test unaligned
    pointers."""
    n = len(x)
    xb = torch.zeros(n + offset, dtype=torch.float32, device=dev())
    hb = torch.zeros(n + offset, dtype=torch.float32, device=dev())
    xb[offset:] = to_dev(x)
    hb[offset:] = to_dev(xh)
    xv, hv = xb[offset:], hb[offset:]
    ov = xv if inplace else torch.zeros(n + offset, dtype=torch.float32, device=dev())[offset:]
    nb = (n + bucket - 1) // bucket
    scales = torch.zeros(max(nb, 1), dtype=torch.float32, device=dev())
    codes = torch.zeros(max((n * bits_ + 7) // 8, 1) + 8, dtype=torch.uint8, device=dev())
    B.gc_dcd_compress(xv, hv, ov, bits_, bucket, seed, step, scales, codes)
    torch.cuda.synchronize()
    return (ov.cpu().numpy(), scales[:nb].cpu().numpy(),
            codes.cpu().numpy()[:(n * bits_ + 7) // 8], codes.cpu().numpy()[(n * bits_ + 7) // 8:])
