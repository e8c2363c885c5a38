"""GPU parity on plans with hundreds of segments (more than one 256-wide
round in every per-segment scan: segment bases of sampled DGC, AdaComp
offsets, pack tiles and layout, decode's segment walk), for every call that
takes a plan, against the oracle bit for bit.  The 17,000-segment layout has
more than 16,384 chunks, where the selection's candidate kernels give each
wave four chunks, here mostly of different segments."""
import numpy as np
import pytest
import torch

import oracle
from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W
from tests.gpu_util import HipPath, same_bits, say, sparse_from_host, to_dev, ulp_report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=[(700, 3000), (17000, 300)], ids=["700seg", "17000seg"])
def layout(request):
    nseg, max_len = request.param
    rng = np.random.default_rng(900)
    t = W.random_table(rng, nseg, max_len=max_len, gaps=True)
    return t, W.table_extent(t), rng


def test_dgc_exact_sampled_nesterov(layout):
    t, n, rng = layout
    hp = HipPath(t, n)
    U = W.random_values(rng, n, "laplace")
    V = W.random_values(rng, n, "laplace")
    for sampled, nest, period in ((False, False, 0), (True, True, 7), (True, False, 1)):
        G = W.random_values(rng, n, "laplace")
        tag = f"manyseg dgc sampled={sampled} nesterov={nest} P={period}"
        say(tag)
        Uo, Vo, idx, val, off, _ = oracle.dgc_ex(t, G, U, V, 0.9, 1e-3, 3, nesterov=nest, sampled=sampled,
                                                 sample_period=max(period, 1), over=2)
        opt = B.dgc_options(0.9, 1e-3, 3, nesterov=nest, sampled=sampled, sample_period=max(period, 1), over=2)
        Ug, Vg, gidx, gval, goff = hp.dgc_ex(G, U, V, opt)
        assert np.array_equal(goff, off) and np.array_equal(gidx, idx), tag
        assert same_bits(gval, val) and same_bits(Ug, Uo) and same_bits(Vg, Vo), tag
        U, V = Uo, Vo


def test_adacomp_pack_decode(layout):
    t, n, rng = layout
    hp = HipPath(t, n)
    R = W.random_values(rng, n, "normal")
    msgs_h, msgs_d = [], []
    for step in range(3):
        dW = W.random_values(rng, n, "laplace")
        say(f"manyseg adacomp step {step}")
        Ro, idx, val, off, scale, _ = oracle.adacomp(t, dW, R, 2.0)
        Rd, am = hp.adacomp(dW, R, 2.0, tensors=True)
        gidx, gval, goff, gscale = am.host()
        assert np.array_equal(goff, off) and np.array_equal(gidx, idx)
        assert same_bits(gval, val) and same_bits(gscale[:len(t)], scale)
        assert same_bits(Rd.cpu().numpy(), Ro), ulp_report(Rd.cpu().numpy(), Ro)
        say(f"manyseg adacomp pack step {step}")
        assert hp.pack(B.GC_KIND_ADACOMP, am) == oracle.pack(2, t, idx, val, off, scale)
        R = Ro
        msgs_h.append((idx, val))
        msgs_d.append(am)
    say("manyseg decode")
    want = oracle.decode(t, n, msgs_h, mode=1)
    got = hp.decode(msgs_d, B.GC_AVG)
    assert same_bits(got, want), ulp_report(got, want)
    # a DGC message through the packer on the same plan
    G = W.random_values(rng, n, "normal")
    z = np.zeros(n, np.float32)
    _, _, didx, dval, doff, _ = oracle.dgc(t, G, z, z, 0.9)
    _, _, dm = hp.dgc(G, z.copy(), z.copy(), 0.9, tensors=True)
    say("manyseg dgc pack")
    assert hp.pack(B.GC_KIND_DGC, dm) == oracle.pack(1, t, didx, dval, doff, np.zeros(len(t), np.float32))


def test_slimdp(layout):
    t, n, rng = layout
    t = t[t[:, 1] >= 2]
    n = W.table_extent(t)
    tc = t.copy()
    tc[:, 3] = np.maximum(1, t[:, 1] // 10)
    te = tc.copy()
    cp, ep = B.Plan(tc), B.Plan(te, W.table_extent(tc))
    ws = cp.workspace(B.GC_OP_DGC, "cuda")
    mask = torch.zeros(B.gc_slimdp_mask_words(cp), dtype=torch.int32, device="cuda")
    w_, g_, d_ = (W.random_values(rng, n) for _ in range(3))
    say("manyseg slimdp")
    cidx, cval, coff, cmask = oracle.slimdp_core(tc, w_, g_, 2.0)
    core = B.Sparse.empty(cp, cp.total_k, "cuda")
    B.gc_slimdp_core(cp, to_dev(w_), to_dev(g_), 2.0, core, mask, ws)
    torch.cuda.synchronize()
    gi, gv, go, _ = core.host()
    assert np.array_equal(gi, cidx) and same_bits(gv, cval) and np.array_equal(go, coff)
    assert np.array_equal(mask.cpu().numpy().view(np.uint32), cmask)
    eidx, evals, eoff = oracle.slimdp_explore(te, d_, cmask, 5, 9)
    out = B.Sparse.empty(ep, ep.total_k, "cuda")
    B.gc_slimdp_explore(ep, cp, to_dev(d_), mask, 5, 9, out, ws)
    torch.cuda.synchronize()
    xi, xv, xo, _ = out.host()
    assert np.array_equal(xi, eidx) and same_bits(xv, evals) and np.array_equal(xo, eoff)


def test_more_segments_than_the_lds_tables_hold():
    """5000 segments: past the 4096 segment-table entries that pack and unpack
    keep in LDS, so their tile searches read the tables from global memory.
    DGC and AdaComp messages, both packs and unpacks, and their decode."""
    rng = np.random.default_rng(905)
    t = W.random_table(rng, 5000, max_len=200, gaps=True)
    n = W.table_extent(t)
    hp = HipPath(t, n)
    G = W.random_values(rng, n, "laplace")
    z = np.zeros(n, np.float32)
    say(f"5000 segments, n={n}: dgc")
    _, _, dm = hp.dgc(G, z.copy(), z.copy(), 0.9, 1e-3, 2, tensors=True)
    _, _, didx, dval, doff, _ = oracle.dgc(t, G, z, z, 0.9, 1e-3, 2)
    gi, gv, go, _ = dm.host()
    assert np.array_equal(go, doff) and np.array_equal(gi, didx) and same_bits(gv, dval)
    say("5000 segments: adacomp")
    _, am = hp.adacomp(G, z.copy(), 2.0, tensors=True)
    _, aidx, aval, aoff, asc, _ = oracle.adacomp(t, G, z, 2.0)
    gi, gv, go, _ = am.host()
    assert np.array_equal(go, aoff) and np.array_equal(gi, aidx) and same_bits(gv, aval)
    for kind, msg, want in ((1, dm, oracle.pack(1, t, didx, dval, doff)),
                            (2, am, oracle.pack(2, t, aidx, aval, aoff, asc))):
        say(f"5000 segments: pack and unpack kind={kind}")
        data = hp.pack(kind, msg)
        assert data == want
        buf = torch.zeros(len(data) + 4, dtype=torch.uint8, device="cuda")
        buf[:len(data)] = torch.from_numpy(np.frombuffer(data, np.uint8).copy()).cuda()
        out = B.Sparse.empty(hp.plan, msg.count(), "cuda")
        st = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        B.gc_unpack(hp.plan, kind, buf, len(data), out, st, hp.workspace(B.GC_OP_UNPACK))
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        ui, uv, uo, _ = out.host()
        mi, mv, mo, _ = msg.host()
        assert np.array_equal(ui, mi) and np.array_equal(uo, mo) and same_bits(uv, mv)
    say("5000 segments: decode")
    got = hp.decode([dm, am], B.GC_AVG)
    want = oracle.decode(t, n, [(didx, dval), (aidx, aval)], mode=1)
    assert same_bits(got, want), ulp_report(got, want)
