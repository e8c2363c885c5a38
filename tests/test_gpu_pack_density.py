"""Packing DGC messages that hold more than the plan's k per segment (the
warm-up densities, the sampled selection's budget): the stream bytes equal
the oracle's, the receiver reads them back to the same message, and a
stream larger than out_cap writes nothing and reports the size it needs."""
import numpy as np
import pytest
import torch

import oracle
from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W
from tests.gpu_util import HipPath, dev, same_bits, say

pytestmark = pytest.mark.gpu


def dgc_message(hp, t, opt, rng):
    n = hp.n
    G = W.random_values(rng, n, "laplace")
    U = W.random_values(rng, n, "normal")
    V = W.random_values(rng, n, "normal")
    return hp.dgc_ex(G, U, V, opt, tensors=True)[2]


def pack_into(hp, msg, cap, room=0):
    """gc_pack into the first `cap` bytes of a buffer of cap + room sentinel bytes."""
    buf = torch.full((cap + room,), 0xA5, dtype=torch.uint8, device=dev())
    nbytes = torch.zeros(1, dtype=torch.int64, device=dev())
    B.gc_pack(hp.plan, B.GC_KIND_DGC, msg, buf[:cap], nbytes, hp.workspace(B.GC_OP_PACK))
    torch.cuda.synchronize()
    return buf.cpu().numpy(), int(nbytes.item())


@pytest.mark.parametrize("density", [(1, 4), (1, 16), (1, 256)])
def test_warmup_density_message_packs_like_the_oracle(density):
    rng = np.random.default_rng(9300 + density[1])
    t = W.make_table([300_000, 4097, 50_000, 1, 70_001], [50] * 5, None, [0, 2, 1, 0, 3])
    hp = HipPath(t)
    opt = B.dgc_options(0.9, 0.0, 1, density=density)
    msg = dgc_message(hp, t, opt, rng)
    idx, val, off, _ = msg.host()
    assert np.any(np.diff(off) > t[:, 3]), "the message holds more than the plan's k somewhere"
    cap = B.gc_dgc_pack_bound(hp.plan, opt)
    assert cap > hp.plan.pack_bound(B.GC_KIND_DGC)
    say(f"pack density {density}: {len(idx)} entries, bound {cap}")
    data, nb = pack_into(hp, msg, cap)
    want = oracle.pack(1, t, idx, val, off)
    assert nb == len(want) and data[:nb].tobytes() == want
    # the receiver reads it back
    out = B.Sparse.empty(hp.plan, int(t[:, 1].sum()), dev())
    st = torch.zeros(1, dtype=torch.int32, device=dev())
    dbuf = torch.from_numpy(data[:nb].copy()).to(dev())
    B.gc_unpack(hp.plan, B.GC_KIND_DGC, dbuf, nb, out, st, hp.workspace(B.GC_OP_UNPACK))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    gi, gv, go, _ = out.host()
    assert np.array_equal(go, off) and np.array_equal(gi, idx) and same_bits(gv, val)


def test_sampled_message_over_k_packs_like_the_oracle():
    rng = np.random.default_rng(9310)
    t = W.make_table([200_000, 9000, 65_537], [50] * 3)
    hp = HipPath(t)
    opt = B.dgc_options(0.9, 0.0, 1, sampled=True, sample_period=7, over=3)
    msg = dgc_message(hp, t, opt, rng)
    idx, val, off, _ = msg.host()
    cap = B.gc_dgc_pack_bound(hp.plan, opt)
    data, nb = pack_into(hp, msg, cap)
    want = oracle.pack(1, t, idx, val, off)
    assert nb == len(want) and data[:nb].tobytes() == want


def test_a_stream_past_out_cap_writes_nothing_and_reports_its_size():
    rng = np.random.default_rng(9320)
    t = W.make_table([100_000, 30_000], [50] * 2)
    hp = HipPath(t)
    opt = B.dgc_options(0.9, 0.0, 1, density=(1, 8))
    msg = dgc_message(hp, t, opt, rng)
    idx, val, off, _ = msg.host()
    want = oracle.pack(1, t, idx, val, off)
    cap = hp.plan.pack_bound(B.GC_KIND_DGC)  # sized for the plan's k: too small here
    assert len(want) > cap
    data, nb = pack_into(hp, msg, cap, room=4096)
    assert nb == len(want)
    assert np.all(data == 0xA5), "nothing written, inside or past out_cap"
    # the same workspace then packs a message that fits
    opt0 = B.dgc_options(0.9, 0.0, 1)
    msg0 = dgc_message(hp, t, opt0, rng)
    i0, v0, o0, _ = msg0.host()
    data0, nb0 = pack_into(hp, msg0, cap)
    assert data0[:nb0].tobytes() == oracle.pack(1, t, i0, v0, o0)
