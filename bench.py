#!/usr/bin/env python3
"""Throughput of the gradient-compression hot path on one MI355X.

A step is one pass of the whole path over one DeepSpeech-scale fp32 gradient
(121,893,373 elements in 68 tensors, inputs resident in HBM):
  DGC step (clip at 1.0, momentum 0.9, exact top 0.1%, masking) + pack,
  AdaComp step (L_T = 500, factor 2) + pack,
  decompress-average of each message,
  DCD 4-bit random quantization of the model difference (buckets of 512).
value = fp32 gradient bytes compressed per second (two compressions of
4 * n bytes per step).  One JSON line is printed.

  python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure

# Algorithmic bytes of each kernel in one step, summed over its launches in
# the step: what the method itself must move (reads + writes of dense data,
# plus message bytes where the kernel's job is the message).  Returns
# {kernel: (bytes per step, launches per step)}.
def algorithmic_bytes(n: int, nbins: int, k_total: int, ada_entries: int, bucket: int = 512):
    return {
        "dgc_update": (20 * n, 1),                 # read G, U, V; write U, V
        "dgc_norm": (4 * n, 1),                    # read G
        "ada_fold": (12 * n, 1),                   # read R, dW; write R (deferred residual: one pass)
        "ada_emit": (8 * ada_entries, 1),          # message
        "dcd": (12 * n + n // 2 + 4 * ((n + bucket - 1) // bucket), 1),  # x, x_half, x_out, codes, scales
        # two launches: each writes the dense update and reads its message
        "decode": (8 * n + 8 * (k_total + ada_entries), 2),
        "dgc_emit": (8 * k_total + 8 * k_total, 1),  # message out + masking writes
    }


def source_digest() -> str:
    """Hash of the HIP sources, to tie stored counter readings to a build."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gradient_compression_dnn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def stored_step_traffic(digest: str):
    """HBM bytes of the whole step from committed counter runs, or None."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic_deepspeech.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    return d.get("step_hbm_bytes") if d.get("source_digest") == digest else None


def stored_traffic(kernel: str, digest: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None if
    the counters were taken on other sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic_deepspeech.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != digest:
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def stored_call_traffic(prefixes, digest: str):
    """HBM bytes per step of the kernels whose names start with one of
    `prefixes`, from committed rocprofv3 counter runs, or None if the counters
    were taken on other sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic_deepspeech.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_digest") != digest or not d.get("steps_in_run"):
        return None
    tot = sum(k["hbm_bytes_per_launch"] * k["launches"] for name, k in d.get("kernels", {}).items()
              if name.startswith(prefixes))
    return round(tot / d["steps_in_run"])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, grad_host, x0, steps_min_s: float = 10.0, max_steps: int = 24):
    """The oracle, as it stands, over a bounded sample of the same workload;
    then one step on a single thread over a smaller sample, and the library
    on the first sample (same inputs and steps) compared bit for bit with
    the oracle's last step.  grad_host(t, lo, hi) is elements [lo, hi) of
    step t's gradient on the host (the same bits the library is given)."""
    import numpy as np

    import oracle
    from gradient_compression_dnn_amd import workloads as W

    threads = len(os.sched_getaffinity(0))
    oracle.set_num_threads(threads)
    names = [nm for nm, _ in W.deepspeech_shapes()]

    def sample(layers):
        sel = [i for i, nm in enumerate(names) if nm.split(".")[0] in layers]
        sub = w.table[sel].copy()
        lo, hi = int(sub[0, 0]), int(sub[-1, 0] + sub[-1, 1])
        sub[:, 0] -= lo
        return sub, lo, hi

    def one_step(sub, lo, hi, t, U, V, R):
        n = hi - lo
        g = grad_host(t, lo, hi)
        x = x0[lo:hi]
        xh = W.dcd_half_step(x, g)
        t0 = time.perf_counter()
        U, V, idx, val, off, _ = oracle.dgc(sub, g, U, V, 0.9, 1.0, 1)
        dbytes = oracle.pack(1, sub, idx, val, off)
        R, ai, av, ao, asc, _ = oracle.adacomp(sub, g, R, 2.0)
        abytes = oracle.pack(2, sub, ai, av, ao, asc)
        dd = oracle.decode(sub, n, [(idx, val)], mode=1)
        ad = oracle.decode(sub, n, [(ai, av)], mode=1)
        xo, sc, cd = oracle.dcd(x, xh, 4, 512, 0x5EED, t)
        dt = time.perf_counter() - t0
        out = dict(U=U, V=V, R=R, dgc=(idx, val, off), dbytes=dbytes, ada=(ai, av, ao, asc), abytes=abytes,
                   dd=dd, ad=ad, dcd=(xo, sc, cd))
        return dt, out

    sub, lo, hi = sample(("gru1", "gru2", "gru3", "gru4"))
    n = hi - lo
    U = np.zeros(n, np.float32)
    V = np.zeros(n, np.float32)
    R = np.zeros(n, np.float32)
    done, t_total, last = 0, 0.0, None
    while done < max_steps and (t_total < steps_min_s or done == 0):
        dt, last = one_step(sub, lo, hi, done, U, V, R)
        U, V, R = last["U"], last["V"], last["R"]
        t_total += dt
        done += 1
    gbs = 2 * 4 * n * done / t_total / 1e9

    # one thread, one step over one GRU layer
    sub1, lo1, hi1 = sample(("gru2",))
    n1 = hi1 - lo1
    oracle.set_num_threads(1)
    z = np.zeros(n1, np.float32)
    dt1, _ = one_step(sub1, lo1, hi1, 0, z, z.copy(), z.copy())
    oracle.set_num_threads(threads)

    return {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"{done} full step(s) (DGC+pack, AdaComp+pack, 2 decodes, DCD) over the "
                      f"32 GRU tensors of layers 1-4 ({n:,} of {w.n_total:,} elements), "
                      f"{t_total:.1f} s on {threads} host threads",
            "cpu_model": cpu_model(),
            "single_thread": {"value": round(2 * 4 * n1 / dt1 / 1e9, 4), "unit": "GB/s",
                              "sample": f"1 step over the 8 tensors of GRU layer 2 ({n1:,} elements), "
                                        f"{dt1:.1f} s"},
            "parity": library_parity(sub, lo, hi, grad_host, x0, done, last)}


def library_parity(sub, lo, hi, grad_host, x0, steps, want):
    """The library over the oracle baseline's sample, with the same inputs and
    steps; the last step's outputs compared bit for bit with the oracle's."""
    import numpy as np
    import torch

    from gradient_compression_dnn_amd import binding as B
    from gradient_compression_dnn_amd import workloads as W

    dev = torch.device("cuda:0")
    n = hi - lo

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    def same(t, a):
        h = t.cpu().numpy() if torch.is_tensor(t) else t
        return bool(np.array_equal(np.asarray(h).view(np.uint32), np.ascontiguousarray(a, np.float32).view(np.uint32)))

    plan = B.Plan(sub, n)
    ws = {op: plan.workspace(op, dev) for op in (B.GC_OP_DGC, B.GC_OP_ADACOMP, B.GC_OP_PACK, B.GC_OP_DECODE)}
    U, V, R = (torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(3))
    state = plan.adacomp_state(dev)
    dmsg = B.Sparse.empty(plan, plan.total_k, dev)
    amsg = B.Sparse.empty(plan, n, dev)
    dbuf = torch.zeros(plan.pack_bound(B.GC_KIND_DGC), dtype=torch.uint8, device=dev)
    abuf = torch.zeros(plan.pack_bound(B.GC_KIND_ADACOMP), dtype=torch.uint8, device=dev)
    dn = torch.zeros(1, dtype=torch.int64, device=dev)
    an = torch.zeros(1, dtype=torch.int64, device=dev)
    dd, ad, xo = (torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(3))
    sc = torch.zeros((n + 511) // 512, dtype=torch.float32, device=dev)
    cd = torch.zeros((n + 1) // 2, dtype=torch.uint8, device=dev)
    x = x0[lo:hi]
    X = f32(x)
    for t in range(steps):
        gh = grad_host(t, lo, hi)
        g, xh = f32(gh), f32(W.dcd_half_step(x, gh))
        B.gc_dgc_step(plan, g, U, V, 0.9, 1.0, 1, dmsg, ws[B.GC_OP_DGC])
        B.gc_pack(plan, B.GC_KIND_DGC, dmsg, dbuf, dn, ws[B.GC_OP_PACK])
        B.gc_adacomp_compress(plan, g, R, 2.0, amsg, ws[B.GC_OP_ADACOMP], state=state)
        B.gc_pack(plan, B.GC_KIND_ADACOMP, amsg, abuf, an, ws[B.GC_OP_PACK])
        B.gc_decompress_accumulate(plan, [dmsg], dd, B.GC_AVG, False, ws[B.GC_OP_DECODE])
        B.gc_decompress_accumulate(plan, [amsg], ad, B.GC_AVG, False, ws[B.GC_OP_DECODE])
        B.gc_dcd_compress(X, xh, xo, 4, 512, 0x5EED, t, sc, cd)
    R_exact = torch.empty_like(R)
    B.gc_adacomp_residual(plan, R, state, R_exact)
    torch.cuda.synchronize()
    di, dv, doff, _ = dmsg.host()
    ai, av, aoff, asc = amsg.host()
    wi, wv, woff = want["dgc"]
    xi, xv, xoff, xsc = want["ada"]
    wo, wsc, wcd = want["dcd"]
    checks = {
        "dgc_U_V": same(U, want["U"]) and same(V, want["V"]),
        "dgc_message": (np.array_equal(di, wi) and same(dv, wv) and np.array_equal(doff, woff)),
        "dgc_packed_bytes": dbuf[:int(dn.item())].cpu().numpy().tobytes() == want["dbytes"],
        "adacomp_residual": same(R_exact, want["R"]),
        "adacomp_message": (np.array_equal(ai, xi) and same(av, xv) and np.array_equal(aoff, xoff)
                            and same(asc[:len(sub)], xsc)),
        "adacomp_packed_bytes": abuf[:int(an.item())].cpu().numpy().tobytes() == want["abytes"],
        "decoded": same(dd, want["dd"]) and same(ad, want["ad"]),
        "dcd": same(xo, wo) and same(sc, wsc) and bool(np.array_equal(cd.cpu().numpy(), wcd)),
    }
    return {"bitwise_equal": all(checks.values()), "checks": checks, "steps": steps, "elements": n,
            "what": "the library run on the oracle baseline's sample (same inputs and steps); "
                    "the last step's states, messages, packed bytes, decoded updates and DCD outputs "
                    "compared bit for bit"}


def measure_variants(B, plan, w, G, X, XH, XO, scales, codes, ws, bucket, dev, log, dmsg, amsg, dbuf, abuf,
                     dn, an, reps: int = 5):
    """Time the other calls of the path on the same workload, each alone
    (after the step timing, outside `value`): DGC with Nesterov momentum and
    with sampled selection, the replica side of DCD-PSGD and ECD-PSGD, the
    unpacking of the step's two streams, and Slim-DP's core, explorer and
    values-only push.  Per call: ms, the method's algorithmic bytes and their
    fraction of HBM peak, and the per-kernel split of one more call."""
    import torch

    n = plan.n_total
    nb = (n + bucket - 1) // bucket
    code_bytes = n // 2 + 4 * nb  # 4-bit codes and scales
    U2 = torch.zeros(n, dtype=torch.float32, device=dev)
    V2 = torch.zeros_like(U2)
    L = X + 1e-4  # two neighbours' replicas, near the node's model
    R_ = X - 1e-4
    XHAT = X.clone()
    XT = X.clone()
    out = {}

    def timed(name, fn, alg_bytes, extra=None):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            fn(1 + r)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        B.gc_timing_enable("*")
        fn(1 + reps)
        torch.cuda.synchronize()
        kern = {}
        for kname in B.KERNELS:
            kms, cnt = B.gc_timing_take(kname)
            if cnt:
                kern[kname] = round(kms * 1000.0, 2)
        B.gc_timing_enable(None)
        rec = {"ms": round(ms, 4), "alg_bytes": alg_bytes,
               "alg_hbm_frac": round(alg_bytes / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
               "kernel_us": kern}
        if extra:
            rec.update(extra())
        out[name] = rec
        log(f"variant {name}: {ms:.3f} ms, {rec['alg_hbm_frac']:.3f} of HBM peak")

    for label, opt in (("dgc_nesterov_exact", B.dgc_options(0.9, 1.0, 1, nesterov=True)),
                       ("dgc_sampled_p100_over2", B.dgc_options(0.9, 1.0, 1, sampled=True, sample_period=100, over=2)),
                       ("dgc_sampled_p1000_over2", B.dgc_options(0.9, 1.0, 1, sampled=True, sample_period=1000,
                                                                 over=2))):
        msg = B.Sparse.empty(plan, B.gc_dgc_message_cap(plan, opt), dev)
        U2.zero_()
        V2.zero_()

        def run(t, opt=opt, msg=msg):
            B.gc_dgc_step_ex(plan, G[t % len(G)], U2, V2, opt, msg, ws[B.GC_OP_DGC])

        timed(label, run, 20 * n, lambda msg=msg: {"entries": msg.count(), "k_total": plan.total_k})
    # the warm-up densities of the DGC page (sparsity 75%, 93.75%, 98.4375%,
    # 99.6%), each call's k set per call; the message and the masking writes
    # (16 B per entry) count with the update's 20 B per element
    for num, den in ((1, 4), (1, 16), (1, 64), (1, 256)):
        opt = B.dgc_options(0.9, 1.0, 1, density=(num, den))
        cap = B.gc_dgc_message_cap(plan, opt)
        msg = B.Sparse.empty(plan, cap, dev)
        U2.zero_()
        V2.zero_()

        def run(t, opt=opt, msg=msg):
            B.gc_dgc_step_ex(plan, G[t % len(G)], U2, V2, opt, msg, ws[B.GC_OP_DGC])

        timed(f"dgc_warmup_density_{num}_{den}", run, 20 * n + 16 * cap,
              lambda msg=msg: {"entries": msg.count()})
    timed("dcd_decode_4bit", lambda t: B.gc_dcd_decode(scales, codes, XHAT, 4, bucket), 8 * n + code_bytes)
    timed("dcd_mix_ring3", lambda t: B.gc_dcd_mix([X, L, R_], [0.5, 0.25, 0.25], G[t % len(G)], 0.1, XO),
          20 * n)  # three replicas and the gradient read, x_half written
    timed("ecd_compress_4bit", lambda t: B.gc_ecd_compress(X, XH[t % len(XH)], 2 + t, 4, bucket, 0x5EED,
                                                           scales, codes), 8 * n + code_bytes)
    timed("ecd_update_4bit", lambda t: B.gc_ecd_update(scales, codes, XT, 2 + t, 4, bucket), 8 * n + code_bytes)

    # the receiver's side of the exchange: the step's packed streams read back
    # into messages (the streams and messages come from the last timed step)
    ustat = torch.zeros(1, dtype=torch.int32, device=dev)
    wsu = plan.workspace(B.GC_OP_UNPACK, dev)
    for label, kind, buf, nbytes_dev, src in (("unpack_dgc_stream", B.GC_KIND_DGC, dbuf, dn, dmsg),
                                              ("unpack_adacomp_stream", B.GC_KIND_ADACOMP, abuf, an, amsg)):
        nbytes = int(nbytes_dev.item())
        entries = src.count()
        um = B.Sparse.empty(plan, max(entries, 1), dev)
        timed(label, lambda t, kind=kind, buf=buf, nbytes=nbytes, um=um:
              B.gc_unpack(plan, kind, buf, nbytes, um, ustat, wsu), nbytes + 8 * entries)
        assert int(ustat.item()) == 0, "the step's own stream must unpack cleanly"

    # Slim-DP at the page's VGG-16 setting (alpha 0.2, beta 0.1): a 10% core
    # by significance and a 10% explorer, per tensor
    import numpy as np
    tc = np.array(plan.table, np.int64)
    tc[:, 3] = np.ceil(tc[:, 1] * 0.1).astype(np.int64)
    core_plan = B.Plan(tc, n)
    exp_plan = B.Plan(tc, n)
    mask = torch.zeros(B.gc_slimdp_mask_words(core_plan), dtype=torch.int32, device=dev)
    core = B.Sparse.empty(core_plan, core_plan.total_k, dev)
    expl = B.Sparse.empty(exp_plan, exp_plan.total_k, dev)
    cvals = torch.zeros(core_plan.total_k, dtype=torch.float32, device=dev)
    kc = core_plan.total_k
    timed("slimdp_core_beta0.1", lambda t: B.gc_slimdp_core(core_plan, X, G[t % len(G)], 50.0, core, mask,
                                                            ws[B.GC_OP_DGC]),
          8 * n + n // 8 + 8 * kc)  # read w, g; write the bitmap and the core message
    timed("slimdp_explore_0.1", lambda t: B.gc_slimdp_explore(exp_plan, core_plan, G[t % len(G)], mask, 0x5EED, t,
                                                              expl, ws[B.GC_OP_DGC]),
          n // 8 + 12 * exp_plan.total_k)  # read the bitmap and delta at the entries; write the message
    timed("slimdp_core_values", lambda t: B.gc_slimdp_core_values(core_plan, core, G[t % len(G)], cvals), 12 * kc)
    return out


def adacomp_rule_messages(B, W, dev, log, steps: int = 10):
    """Both readings of AdaComp's adaptive threshold (the factor on the
    accumulated residual, the default; or on the new gradient, with the bin
    max always sent) on the DeepSpeech and LSTM LM workloads: `steps` steps
    from a zero residual with a fresh seeded gradient each (deferred
    residual), then the last step's message packed.  Reports the fraction of
    the n elements sent and the compression ratio 4 n / packed bytes.  Run
    outside the timed region."""
    import torch

    res = {"steps": steps,
           "page_context": "the AdaComp page reports ~200x end to end for fully connected and recurrent "
                           "layers and ~40x for convolutional layers (trained models, not these "
                           "synthetic gradients)"}
    for name in ("deepspeech", "lstm_lm"):
        w = W.make_config(name)
        n = w.n_total
        plan = B.Plan(w.table, n)
        wsa, wsp = plan.workspace(B.GC_OP_ADACOMP, dev), plan.workspace(B.GC_OP_PACK, dev)
        msg = B.Sparse.empty(plan, n, dev)
        buf = torch.zeros(plan.pack_bound(B.GC_KIND_ADACOMP), dtype=torch.uint8, device=dev)
        nbytes = torch.zeros(1, dtype=torch.int64, device=dev)
        per = {}
        for label, rule in (("residual", B.GC_ADACOMP_RULE_RESIDUAL), ("gradient", B.GC_ADACOMP_RULE_GRADIENT)):
            R = torch.zeros(n, dtype=torch.float32, device=dev)
            st = plan.adacomp_state(dev)
            for t in range(steps):
                g = W.gradient_device(w, t, dev)
                B.gc_adacomp_compress(plan, g, R, 2.0, msg, wsa, state=st, rule=rule)
            B.gc_pack(plan, B.GC_KIND_ADACOMP, msg, buf, nbytes, wsp)
            torch.cuda.synchronize()
            sent, nb = msg.count(), int(nbytes.item())
            per[label] = {"entries": sent, "entries_frac": round(sent / n, 5), "packed_bytes": nb,
                          "compression_ratio": round(4 * n / nb, 1)}
            log(f"adacomp {name} rule {label}: {100.0 * sent / n:.2f}% sent, {4 * n / nb:.1f}x")
        res[name] = per
        del R, st, msg, buf
    return res


def measure_configs(B, W, dev, log, reps: int = 10):
    """The other workloads of the configuration list, each timed alone after
    the step timing (not part of `value`): ms per step and dense fp32 GB/s.
      fc1m        one AdaComp step (L_T = 50) and one DGC step (top 0.1%, no clip);
                  the DGC step also cold (Infinity Cache evicted before each call)
      resnet50    DGC steps (momentum 0.9, clip 1.0, top 0.1% per tensor), warm and cold
      lstm_lm     AdaComp steps (L_T 500 / 50, residual carried)
      resnet50x8  8 learners' DGC steps (N = 8) and the 8-message average; the
                  8 learners' DGC steps as one call over a 1,288-tensor plan"""
    import torch

    out = {}

    def timed(name, fn, dense_bytes, alg_bytes):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            fn(1 + r)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "dense_GBs": round(dense_bytes / (ms / 1000.0) / 1e9, 1),
                     "alg_hbm_frac": round(alg_bytes / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"config {name}: {ms:.3f} ms")

    scratch = torch.empty(256 << 20, dtype=torch.float32, device=dev)  # 1 GiB

    def timed_cold(name, fn, dense_bytes, alg_bytes):
        """Each call after writing 1 GiB of scratch, which evicts the 256 MB
        Infinity Cache; only the call itself is inside the events."""
        fn(0)
        ms = 0.0
        for r in range(reps):
            scratch.fill_(float(r))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn(1 + r)
            e1.record()
            torch.cuda.synchronize()
            ms += e0.elapsed_time(e1) / reps
        out[name] = {"ms": round(ms, 4), "dense_GBs": round(dense_bytes / (ms / 1000.0) / 1e9, 1),
                     "alg_hbm_frac": round(alg_bytes / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"config {name}: {ms:.3f} ms")

    def dev_grads(w, count=2):
        return [torch.from_numpy(W.gradient(w, t)).to(dev) for t in range(count)]

    # fc1m
    w = W.make_config("fc1m")
    n = w.n_total
    plan = B.Plan(w.table, n)
    g = dev_grads(w)
    U, V, R = (torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(3))
    st = plan.adacomp_state(dev)
    dm = B.Sparse.empty(plan, plan.total_k, dev)
    am = B.Sparse.empty(plan, n, dev)
    wsd, wsa = plan.workspace(B.GC_OP_DGC, dev), plan.workspace(B.GC_OP_ADACOMP, dev)
    timed("fc1m_adacomp", lambda t: B.gc_adacomp_compress(plan, g[t % 2], R, 2.0, am, wsa, state=st), 4 * n, 12 * n)
    timed("fc1m_dgc", lambda t: B.gc_dgc_step(plan, g[t % 2], U, V, 0.9, 0.0, 1, dm, wsd), 4 * n, 20 * n)
    timed_cold("fc1m_dgc_cold", lambda t: B.gc_dgc_step(plan, g[t % 2], U, V, 0.9, 0.0, 1, dm, wsd), 4 * n, 20 * n)
    # the same two calls captured once in a HIP graph and replayed (the plan
    # is already on the device, and the hot calls allocate nothing)
    Gslot = g[0].clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.gc_adacomp_compress(plan, Gslot, R, 2.0, am, wsa, state=st)
        B.gc_dgc_step(plan, Gslot, U, V, 0.9, 0.0, 1, dm, wsd)
    torch.cuda.synchronize()
    timed("fc1m_adacomp_and_dgc_graph", lambda t: graph.replay(), 8 * n, 32 * n)
    # resnet50
    w = W.make_config("resnet50")
    n = w.n_total
    plan = B.Plan(w.table, n)
    g = dev_grads(w)
    U, V = (torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(2))
    dm = B.Sparse.empty(plan, plan.total_k, dev)
    wsd = plan.workspace(B.GC_OP_DGC, dev)
    timed("resnet50_dgc", lambda t: B.gc_dgc_step(plan, g[t % 2], U, V, 0.9, 1.0, 1, dm, wsd), 4 * n, 20 * n)
    timed_cold("resnet50_dgc_cold", lambda t: B.gc_dgc_step(plan, g[t % 2], U, V, 0.9, 1.0, 1, dm, wsd), 4 * n,
               20 * n)
    del g, U, V, wsd, scratch
    # lstm_lm
    w = W.make_config("lstm_lm")
    n = w.n_total
    plan = B.Plan(w.table, n)
    g = dev_grads(w)
    R = torch.zeros(n, dtype=torch.float32, device=dev)
    st = plan.adacomp_state(dev)
    am = B.Sparse.empty(plan, n, dev)
    wsa = plan.workspace(B.GC_OP_ADACOMP, dev)
    timed("lstm_lm_adacomp", lambda t: B.gc_adacomp_compress(plan, g[t % 2], R, 2.0, am, wsa, state=st), 4 * n, 12 * n)
    del g, R, am, wsa
    # resnet50x8: one plan per learner over its own 25.6M-element buffer
    w = W.make_config("resnet50x8")
    per = w.params["learner_len"]
    single = W.make_config("resnet50")
    plan = B.Plan(single.table, per)
    gall = torch.from_numpy(W.gradient(w, 0)).to(dev)
    G8 = [gall[j * per:(j + 1) * per] for j in range(8)]
    U8 = torch.zeros(8 * per, dtype=torch.float32, device=dev)
    V8 = torch.zeros_like(U8)
    msgs = [B.Sparse.empty(plan, plan.total_k, dev) for _ in range(8)]
    wsd, wsdec = plan.workspace(B.GC_OP_DGC, dev), plan.workspace(B.GC_OP_DECODE, dev)
    avg = torch.zeros(per, dtype=torch.float32, device=dev)

    def learners(t):
        for j in range(8):
            B.gc_dgc_step(plan, G8[j], U8[j * per:(j + 1) * per], V8[j * per:(j + 1) * per], 0.9, 1.0, 8, msgs[j], wsd)
        B.gc_decompress_accumulate(plan, msgs, avg, B.GC_AVG, False, wsdec)

    timed("resnet50x8_dgc_and_average", learners, 8 * 4 * per, 8 * 20 * per + 4 * per)
    # the same eight learners' DGC steps as one call: one plan over the eight
    # buffers (1,288 tensors), so the selection's launches serve all of them
    plan8 = B.Plan(w.table, w.n_total)
    msg8 = B.Sparse.empty(plan8, plan8.total_k, dev)
    wsd8 = plan8.workspace(B.GC_OP_DGC, dev)
    U8.zero_()
    V8.zero_()
    timed("resnet50x8_dgc_one_call", lambda t: B.gc_dgc_step(plan8, gall, U8, V8, 0.9, 1.0, 8, msg8, wsd8),
          8 * 4 * per, 8 * 20 * per)
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--max-grads", type=int, default=64,
                    help="most distinct seeded gradients held on the device (each step of the run "
                         "draws its own while the run has at most this many steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the DGC Nesterov / sampled and DCD replica / ECD calls")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU: the compression step is per learner and needs no "
              f"collective here; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from gradient_compression_dnn_amd import binding as B
    from gradient_compression_dnn_amd import workloads as W

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    w = W.make_config("deepspeech")
    n = w.n_total
    plan = B.Plan(w.table, n)
    # every step of the run (warm-up, instrumented, timed, breakdown, per-call)
    # gets its own gradient, seed 5000 + t, drawn on the device before any
    # step; past --max-grads steps the pool is cycled
    call_reps = max(3, min(args.steps, 10))  # back-to-back repeats of each call timed alone
    run_steps = args.warmup + args.steps + 2 + call_reps
    ng = max(1, min(run_steps, args.max_grads))
    log(f"workload deepspeech: {w.nseg} tensors, {n:,} elements; drawing {ng} gradients on the device")
    x0 = W.dcd_model(w)
    G = [W.gradient_device(w, t, dev) for t in range(ng)]
    X = torch.from_numpy(x0).to(dev)
    XH = [X - 0.1 * g for g in G]  # synthetic x_{t+1/2}, prepared outside the timed region
    torch.cuda.synchronize()

    def grad_host(t, lo, hi):
        return G[t % ng][lo:hi].cpu().numpy()
    U = torch.zeros(n, dtype=torch.float32, device=dev)
    V = torch.zeros_like(U)
    R = torch.zeros_like(U)
    astate = plan.adacomp_state(dev)  # deferred residual: (R, astate) is the learner's residual
    XO = torch.zeros_like(U)
    dmsg = B.Sparse.empty(plan, plan.total_k, dev)
    amsg = B.Sparse.empty(plan, n, dev)
    dbuf = torch.zeros(plan.pack_bound(B.GC_KIND_DGC), dtype=torch.uint8, device=dev)
    abuf = torch.zeros(plan.pack_bound(B.GC_KIND_ADACOMP), dtype=torch.uint8, device=dev)
    dn = torch.zeros(1, dtype=torch.int64, device=dev)
    an = torch.zeros(1, dtype=torch.int64, device=dev)
    ddense = torch.zeros_like(U)
    adense = torch.zeros_like(U)
    bucket = 512
    scales = torch.zeros((n + bucket - 1) // bucket, dtype=torch.float32, device=dev)
    codes = torch.zeros((n + 1) // 2, dtype=torch.uint8, device=dev)
    ws = {op: plan.workspace(op, dev) for op in (B.GC_OP_DGC, B.GC_OP_ADACOMP, B.GC_OP_PACK,
                                                 B.GC_OP_DECODE)}

    CALLS = ("dgc", "dgc_pack", "adacomp", "adacomp_pack", "dgc_decode", "adacomp_decode", "dcd")

    def step_calls(t):
        """The step's calls, in order, for step t."""
        g = G[t % len(G)]
        return (lambda: B.gc_dgc_step(plan, g, U, V, 0.9, 1.0, 1, dmsg, ws[B.GC_OP_DGC]),
                lambda: B.gc_pack(plan, B.GC_KIND_DGC, dmsg, dbuf, dn, ws[B.GC_OP_PACK]),
                lambda: B.gc_adacomp_compress(plan, g, R, 2.0, amsg, ws[B.GC_OP_ADACOMP], state=astate),
                lambda: B.gc_pack(plan, B.GC_KIND_ADACOMP, amsg, abuf, an, ws[B.GC_OP_PACK]),
                lambda: B.gc_decompress_accumulate(plan, [dmsg], ddense, B.GC_AVG, False, ws[B.GC_OP_DECODE]),
                lambda: B.gc_decompress_accumulate(plan, [amsg], adense, B.GC_AVG, False, ws[B.GC_OP_DECODE]),
                lambda: B.gc_dcd_compress(X, XH[t % len(XH)], XO, 4, bucket, 0x5EED, t, scales, codes))

    def step(t, marks=None):
        """One step; with `marks` (len(CALLS) + 1 events) each call is bracketed."""
        for i, call in enumerate(step_calls(t)):
            if marks:
                marks[i].record()
            call()
        if marks:
            marks[-1].record()

    # warm-up, then one instrumented step to find the dominant kernel
    log(f"warmup {args.warmup} step(s)")
    for t in range(args.warmup):
        step(t)
    B.gc_timing_enable("*")
    step(args.warmup)
    torch.cuda.synchronize()
    per_kernel = {}
    for kname in B.KERNELS:
        ms, cnt = B.gc_timing_take(kname)
        if cnt:
            per_kernel[kname] = (ms, cnt)
    dominant = max(per_kernel, key=lambda k: per_kernel[k][0])
    log("kernel times (ms/step): " + ", ".join(
        f"{k} {v[0]:.3f}" for k, v in sorted(per_kernel.items(), key=lambda kv: -kv[1][0])))

    # timed region: only the dominant kernel is bracketed by events
    B.gc_timing_enable(dominant)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} step(s)")
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps - 1)]
    t_start.record()
    for t in range(args.steps):
        step(args.warmup + 1 + t)
        if t + 1 < args.steps:
            marks[t].record()
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    bounds = [t_start] + marks + [t_end]
    step_ms = sorted(bounds[i].elapsed_time(bounds[i + 1]) for i in range(args.steps))
    dom_ms, dom_cnt = B.gc_timing_take(dominant)
    B.gc_timing_enable(None)
    ms_per_step = total_ms / args.steps

    # a per-kernel breakdown from one more instrumented step (not the timed one)
    B.gc_timing_enable("*")
    step(args.warmup + 1 + args.steps)
    torch.cuda.synchronize()
    breakdown = {}
    for kname in B.KERNELS:
        ms, cnt = B.gc_timing_take(kname)
        if cnt:
            breakdown[kname] = round(ms * 1000.0, 2)  # microseconds in one step
    B.gc_timing_enable(None)

    # the DCD step's signal-to-noise measure (alpha of the DCD page):
    # ||Z - C(Z)|| / ||Z|| with Z = x_half - x and C(Z) = x_out - x, taken
    # here, while XO still holds the breakdown step's output for its XH
    t_last = args.warmup + 1 + args.steps
    z = (XH[t_last % len(XH)].double() - X.double())
    cz = XO.double() - X.double()
    dcd_alpha = float(torch.linalg.vector_norm(z - cz) / torch.linalg.vector_norm(z))
    del z, cz

    # each call of the step alone (outside the timed region): the call
    # repeated back to back over the steps that follow, with events only
    # around the batch, so that no event marker (several microseconds each)
    # falls between two calls; the compressions take a fresh gradient (and
    # DCD a fresh step) each time, packs and decodes the last message
    call_ms = {}
    t_calls = args.warmup + 2 + args.steps
    reps = call_reps
    for i, c in enumerate(CALLS):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            step_calls(t_calls + r)[i]()
        e1.record()
        torch.cuda.synchronize()
        call_ms[c] = e0.elapsed_time(e1) / reps

    # the measured streaming ceiling: a plain 1 GiB device-to-device copy, best
    # of 5 (also the reference that scales rocprofv3's byte counters)
    ca = torch.zeros(256 << 20, dtype=torch.float32, device=dev)
    cb = torch.empty_like(ca)
    cb.copy_(ca)
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cb.copy_(ca)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    copy_gbs = 2 * ca.numel() * 4 / (best / 1000.0) / 1e9
    del ca, cb

    # the update's own access pattern with none of its selection work (three
    # reads, two writes per element, the dense kernels' layout and hints) on
    # the workload's size, best of 5: the streaming ceiling for dgc_update
    # (inputs: a gradient and the DCD model pair; outputs: the decode buffers,
    # rewritten by every step anyway)
    B.gc_stream_probe(G[0], X, XH[0], ddense, adense)
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.gc_stream_probe(G[0], X, XH[0], ddense, adense)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    stream_gbs = 20 * n / (best / 1000.0) / 1e9

    ada_entries = amsg.count()
    nbins = plan.total_bins
    alg = algorithmic_bytes(n, nbins, plan.total_k, ada_entries, bucket)
    dom_avg_s = dom_ms / dom_cnt / 1000.0
    digest = source_digest()
    roof = None
    if dominant in alg:
        # launches per step from the instrumented step
        per_launch = alg[dominant][0] // per_kernel[dominant][1]
        ach = per_launch / dom_avg_s / 1e9
        traffic = stored_traffic(dominant, digest)
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dominant, "avg_us": round(dom_avg_s * 1e6, 2), "launches": dom_cnt,
                "algorithmic_bytes_per_launch": per_launch}
    # each kernel's bytes over all its launches in the step, over its time in
    # the step (breakdown sums the launches too)
    kernel_frac = {}
    for k, us in breakdown.items():
        if k in alg and us > 0:
            kernel_frac[k] = round(alg[k][0] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)

    # per method: the call's own time, the method's algorithmic bytes and the
    # counters' bytes of its kernels (pack and decode: both calls together)
    def method(ms, alg_bytes, prefixes):
        ctr = stored_call_traffic(prefixes, digest)
        frac = lambda b: None if b is None else round(b / (ms / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)
        return {"ms": round(ms, 4), "alg_bytes": alg_bytes, "alg_hbm_frac": frac(alg_bytes),
                "counter_bytes": ctr, "counter_hbm_frac": frac(ctr)}

    methods = {
        "dgc": method(call_ms["dgc"], alg["dgc_update"][0] + alg["dgc_emit"][0], ("dgc_",)),
        "adacomp": method(call_ms["adacomp"], alg["ada_fold"][0] + alg["ada_emit"][0], ("ada_",)),
        "pack_both": method(call_ms["dgc_pack"] + call_ms["adacomp_pack"],
                            8 * (plan.total_k + ada_entries) + int(dn.item()) + int(an.item()), ("pack_",)),
        "decode_both": method(call_ms["dgc_decode"] + call_ms["adacomp_decode"], alg["decode"][0], ("decode",)),
        "dcd": method(call_ms["dcd"], alg["dcd"][0], ("dcd",)),
    }

    value = 2 * 4 * n / (ms_per_step / 1000.0) / 1e9
    # the method's own bytes for the whole step: DGC 20 B/elt, AdaComp 12, DCD 12.5 + scales,
    # two dense decodes 4 each, plus the messages read and written
    step_bytes = (alg["dgc_update"][0] + 12 * n + alg["dcd"][0] + alg["decode"][0]
                  + alg["dgc_emit"][0] + 8 * ada_entries + int(dn.item()) + int(an.item()))
    result = {
        "metric": "GB/s of fp32 gradient compressed per step (+% HBM peak), DGC & AdaComp",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "step_ms_median": round(step_ms[len(step_ms) // 2], 4), "step_ms_min": round(step_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "deepspeech: 121,893,373 fp32 gradient elements in 68 tensors "
                               "(5 conv + 7 bidirectional GRU, hidden 800 + FC), log-normal "
                               "per-tensor scales",
                   "step": "DGC(m=0.9, clip 1.0, top 0.1%, masking)+pack, AdaComp(L_T=500, x2)+pack, "
                           "2x decompress-average (K=1), DCD 4-bit bucket 512",
                   "gradients": (f"a fresh seeded gradient per step (seed 5000 + t), {ng} drawn on the device "
                                 f"before the run" + ("" if ng >= run_steps else
                                                     f", cycled past {ng} of the run's {run_steps} steps")),
                   "parallelism": "single GPU (one learner)"},
        "step_alg_bytes": step_bytes,
        "step_alg_hbm_frac": round(step_bytes / (ms_per_step / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
        # the counters' bytes for the whole step (committed rocprofv3 runs of these sources), over this step time
        "step_counter_hbm_bytes": stored_step_traffic(digest),
        "step_counter_hbm_frac": (None if stored_step_traffic(digest) is None else
                                  round(stored_step_traffic(digest) / (ms_per_step / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)),
        "roofline": roof,
        "methods": methods,
        "copy_ceiling": {"achieved": round(copy_gbs, 1), "unit": "GB/s", "frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                         "what": "device-to-device copy of 1 GiB (1 GiB read + 1 GiB written), best of 5"},
        "stream_ceiling": {"achieved": round(stream_gbs, 1), "unit": "GB/s", "frac": round(stream_gbs / HBM_PEAK_GBS, 4),
                           "dominant_share": (None if roof is None or roof["kernel"] != "dgc_update"
                                              else round(roof["achieved"] / stream_gbs, 4)),
                           "what": "gc_stream_probe: 3 fp32 reads + 2 writes per element over the workload's n "
                                   "in the dense kernels' layout and cache hints (dgc_update's traffic, no "
                                   "selection work), best of 5"},
        "kernel_us_per_step": breakdown,
        "kernel_alg_hbm_frac": kernel_frac,
        "messages": {"dgc_entries": plan.total_k, "adacomp_entries": ada_entries,
                     "dgc_packed_bytes": int(dn.item()), "adacomp_packed_bytes": int(an.item()),
                     "dgc_compression_ratio": round(4 * n / int(dn.item()), 1),
                     "adacomp_compression_ratio": round(4 * n / int(an.item()), 1),
                     "dcd_codes_and_scales_bytes": (n + 1) // 2 + 4 * ((n + bucket - 1) // bucket),
                     "dcd_alpha_emp": round(dcd_alpha, 5)},
        "source_digest": digest,
    }
    if not args.no_variants:
        log("variants")
        result["variants"] = measure_variants(B, plan, w, G, X, XH, XO, scales, codes, ws, bucket, dev, log,
                                              dmsg, amsg, dbuf, abuf, dn, an)
        result["configs"] = measure_configs(B, W, dev, log)
        result["messages"]["adacomp_rules"] = adacomp_rule_messages(B, W, dev, log)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(w, grad_host, x0)
        result["parity"] = result["cpu_baseline"].pop("parity")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
