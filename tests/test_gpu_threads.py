"""Host threads calling the library at once: four threads share one plan
(its first use on the device happens concurrently), each with its own
stream, state, workspaces and messages, running DGC and AdaComp steps, packs
and decodes while the others do.  Every thread's results equal the oracle's
bit for bit (the calls release the interpreter lock, so the host side really
runs in parallel)."""
import threading

import numpy as np
import pytest
import torch

import oracle
from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W
from tests.gpu_util import say, same_bits

pytestmark = pytest.mark.gpu


def test_threads_share_a_plan():
    t = W.make_table([70_000, 4097, 65, 150_001, 3], [50, 500, 7, 64, 1],
                     [70, 5, 1, 151, 1], [0, 3, 1, 2, 0])
    n = W.table_extent(t)
    plan = B.Plan(t, n)  # not yet on the device
    nthreads, steps = 4, 3
    inputs = []
    for i in range(nthreads):
        rng = np.random.default_rng(950 + i)
        inputs.append([W.random_values(rng, n, "laplace") for _ in range(steps)])
    results, errors = {}, []
    barrier = threading.Barrier(nthreads)

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                U = torch.zeros(n, device="cuda")
                V = torch.zeros(n, device="cuda")
                R = torch.zeros(n, device="cuda")
                state = plan.adacomp_state("cuda")
                ws = {op: plan.workspace(op, "cuda") for op in (B.GC_OP_DGC, B.GC_OP_ADACOMP, B.GC_OP_PACK,
                                                                B.GC_OP_DECODE)}
                dm = B.Sparse.empty(plan, plan.total_k, "cuda")
                am = B.Sparse.empty(plan, B.gc_adacomp_message_cap(plan), "cuda")
                buf = torch.zeros(plan.pack_bound(B.GC_KIND_ADACOMP), dtype=torch.uint8, device="cuda")
                nb = torch.zeros(1, dtype=torch.int64, device="cuda")
                dense = torch.zeros(n, device="cuda")
                gs = [torch.from_numpy(g).cuda() for g in inputs[i]]
                stream.synchronize()
                barrier.wait()
                for g in gs:
                    B.gc_dgc_step(plan, g, U, V, 0.9, 1e-3, 2, dm, ws[B.GC_OP_DGC])
                    B.gc_adacomp_compress(plan, g, R, 2.0, am, ws[B.GC_OP_ADACOMP], state=state)
                B.gc_pack(plan, B.GC_KIND_ADACOMP, am, buf, nb, ws[B.GC_OP_PACK])
                B.gc_decompress_accumulate(plan, [dm, am], dense, B.GC_SUM, False, ws[B.GC_OP_DECODE])
                Rx = torch.empty_like(R)
                B.gc_adacomp_residual(plan, R, state, Rx)
                stream.synchronize()
                results[i] = dict(U=U.cpu().numpy(), V=V.cpu().numpy(), R=Rx.cpu().numpy(), dm=dm.host(),
                                  am=am.host(), packed=buf[:int(nb.item())].cpu().numpy().tobytes(),
                                  dense=dense.cpu().numpy())
        except Exception as e:  # reported below, on the main thread
            errors.append((i, repr(e)))

    say(f"{nthreads} host threads on one plan")
    threads = [threading.Thread(target=worker, args=(i,)) for i in range(nthreads)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    z = np.zeros(n, np.float32)
    for i in range(nthreads):
        U, V, R = z, z, z
        for g in inputs[i]:
            U, V, didx, dval, doff, _ = oracle.dgc(t, g, U, V, 0.9, 1e-3, 2)
            R, aidx, aval, aoff, asc, _ = oracle.adacomp(t, g, R, 2.0)
        got = results[i]
        assert same_bits(got["U"], U) and same_bits(got["V"], V) and same_bits(got["R"], R), i
        gi, gv, go, _ = got["dm"]
        assert np.array_equal(gi, didx) and same_bits(gv, dval) and np.array_equal(go, doff), i
        gi, gv, go, gsc = got["am"]
        assert np.array_equal(gi, aidx) and same_bits(gv, aval) and np.array_equal(go, aoff), i
        assert got["packed"] == oracle.pack(2, t, aidx, aval, aoff, asc), i
        want = oracle.decode(t, n, [(didx, dval), (aidx, aval)], mode=0)
        assert same_bits(got["dense"], want), i
