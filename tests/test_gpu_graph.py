"""The hot calls under HIP graph capture: a DGC step (and an AdaComp step
with its deferred residual) on the 1M-element FC layer, and on a plan of
17,000 random tensors, is captured once and replayed several times, with
eager work and synchronizations between the replays; every replay's message
and state must equal an eager run of the same call on copies, bit for bit.
The plan is uploaded by a warm-up call before capture (the one allocation the
library makes)."""
import numpy as np
import pytest
import torch

from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.detach().cpu().numpy().view(np.uint32)


def _workload(name):
    """(table, n, four host gradients): the FC layer, or 17,000 random tensors
    (more than 16,384 chunks: the DGC candidate kernels take four per wave)."""
    if name == "fc1m":
        w = W.make_config("fc1m")
        return w.table, w.n_total, [W.gradient(w, t) for t in range(4)]
    rng = np.random.default_rng(77)
    t = W.random_table(rng, 17000, max_len=300, gaps=True)
    n = W.table_extent(t)
    return t, n, [W.random_values(rng, n, "laplace") for _ in range(4)]


@pytest.mark.parametrize("name", ["fc1m", "wide"])
def test_dgc_and_adacomp_steps_replay_like_eager(name):
    table, n, host_grads = _workload(name)
    plan = B.Plan(table, n)
    dev = torch.device("cuda:0")
    grads = [torch.from_numpy(g).to(dev) for g in host_grads]
    G = torch.empty(n, dtype=torch.float32, device=dev)  # the graph's input slot
    U, V, R = (torch.zeros(n, dtype=torch.float32, device=dev) for _ in range(3))
    st = plan.adacomp_state(dev)
    dm = B.Sparse.empty(plan, plan.total_k, dev)
    am = B.Sparse.empty(plan, n, dev)
    wsd, wsa = plan.workspace(B.GC_OP_DGC, dev), plan.workspace(B.GC_OP_ADACOMP, dev)
    # eager twins of every state and output
    Ue, Ve, Re = U.clone(), V.clone(), R.clone()
    ste = st.clone()
    dme = B.Sparse.empty(plan, plan.total_k, dev)
    ame = B.Sparse.empty(plan, n, dev)
    wsde, wsae = plan.workspace(B.GC_OP_DGC, dev), plan.workspace(B.GC_OP_ADACOMP, dev)

    def step(g, U_, V_, R_, st_, dm_, am_, wsd_, wsa_):
        B.gc_dgc_step(plan, g, U_, V_, 0.9, 1e-3, 2, dm_, wsd_)
        B.gc_adacomp_compress(plan, g, R_, 2.0, am_, wsa_, state=st_)

    # warm-up on the eager twins uploads the plan to the device
    G.copy_(grads[0])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(G, U.clone(), V.clone(), R.clone(), st.clone(), dm, am, wsd, wsa)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph capture")
    with torch.cuda.graph(graph):
        step(G, U, V, R, st, dm, am, wsd, wsa)
    torch.cuda.synchronize()
    for t in range(4):
        say(f"graph replay {t}")
        G.copy_(grads[t])
        graph.replay()
        torch.cuda.synchronize()
        step(grads[t], Ue, Ve, Re, ste, dme, ame, wsde, wsae)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(U), _bits(Ue)) and np.array_equal(_bits(V), _bits(Ve))
        assert np.array_equal(_bits(R), _bits(Re)) and torch.equal(st, ste)
        for a, b in ((dm, dme), (am, ame)):
            ai, av, ao, asc = a.host()
            bi, bv, bo, bsc = b.host()
            assert np.array_equal(ai, bi) and np.array_equal(ao, bo)
            assert np.array_equal(av.view(np.uint32), bv.view(np.uint32))
            assert np.array_equal(asc.view(np.uint32), bsc.view(np.uint32))
        # unrelated eager work between replays
        torch.cuda.synchronize()
        _ = (grads[t] * 2).sum().item()


def test_first_calls_of_an_uploaded_plan_capture():
    """gc_plan_upload puts the tables on the device, so even a plan's first
    DGC step can be captured (no allocation happens inside the capture); the
    replays equal eager steps on a second plan of the same layout."""
    w = W.make_config("fc1m")
    n = w.n_total
    dev = torch.device("cuda:0")
    plan, twin = B.Plan(w.table, n), B.Plan(w.table, n)
    plan.upload()
    plan.upload()  # idempotent
    grads = [torch.from_numpy(W.gradient(w, t)).to(dev) for t in range(3)]
    G = torch.empty(n, dtype=torch.float32, device=dev)
    U, V = torch.zeros(n, device=dev), torch.zeros(n, device=dev)
    Ue, Ve = U.clone(), V.clone()
    dm, dme = B.Sparse.empty(plan, plan.total_k, dev), B.Sparse.empty(twin, twin.total_k, dev)
    ws, wse = plan.workspace(B.GC_OP_DGC, dev), twin.workspace(B.GC_OP_DGC, dev)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    say("graph capture of an uploaded plan's first call")
    with torch.cuda.graph(graph):
        B.gc_dgc_step(plan, G, U, V, 0.9, 1e-3, 2, dm, ws)
    torch.cuda.synchronize()
    for t in range(3):
        G.copy_(grads[t])
        graph.replay()
        torch.cuda.synchronize()
        B.gc_dgc_step(twin, grads[t], Ue, Ve, 0.9, 1e-3, 2, dme, wse)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(U), _bits(Ue)) and np.array_equal(_bits(V), _bits(Ve))
        ai, av, ao, _ = dm.host()
        bi, bv, bo, _ = dme.host()
        assert np.array_equal(ai, bi) and np.array_equal(ao, bo) and np.array_equal(av.view(np.uint32), bv.view(np.uint32))

