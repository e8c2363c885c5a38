"""Calls on different streams are independent when they use different
workspaces and outputs: a DGC step and an AdaComp step of two learners run
concurrently on two streams (default priority) and must equal the same
calls run one after the other, bit for bit."""
import numpy as np
import pytest
import torch

from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def test_two_streams_match_sequential():
    w = W.make_config("resnet50")
    n = w.n_total
    plan = B.Plan(w.table, n)
    dev = torch.device("cuda:0")
    g = [torch.from_numpy(W.gradient(w, t)).to(dev) for t in range(2)]

    def learner():
        return dict(U=torch.zeros(n, device=dev), V=torch.zeros(n, device=dev), R=torch.zeros(n, device=dev),
                    st=plan.adacomp_state(dev), dm=B.Sparse.empty(plan, plan.total_k, dev),
                    am=B.Sparse.empty(plan, n, dev), wsd=plan.workspace(B.GC_OP_DGC, dev),
                    wsa=plan.workspace(B.GC_OP_ADACOMP, dev))

    def step(L, grad):
        B.gc_dgc_step(plan, grad, L["U"], L["V"], 0.9, 1.0, 2, L["dm"], L["wsd"])
        B.gc_adacomp_compress(plan, grad, L["R"], 2.0, L["am"], L["wsa"], state=L["st"])

    conc = [learner(), learner()]
    seq = [learner(), learner()]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for t in range(3):
        say(f"two streams step {t}")
        torch.cuda.synchronize()
        for j in range(2):
            with torch.cuda.stream(streams[j]):
                step(conc[j], g[(t + j) % 2])
        torch.cuda.synchronize()
        for j in range(2):
            step(seq[j], g[(t + j) % 2])
        torch.cuda.synchronize()
        for a, b in zip(conc, seq):
            for key in ("U", "V", "R"):
                assert np.array_equal(_bits(a[key]), _bits(b[key])), key
            assert torch.equal(a["st"], b["st"])
            for m in ("dm", "am"):
                ai, av, ao, _ = a[m].host()
                bi, bv, bo, _ = b[m].host()
                assert np.array_equal(ai, bi) and np.array_equal(ao, bo)
                assert np.array_equal(av.view(np.uint32), bv.view(np.uint32))
