"""GPU parity of gc_adacomp_compress_ex under both readings of AdaComp's
adaptive threshold, against the oracle, bit for bit (indices, values,
segment offsets and scales, the residual), in both residual modes over
several steps with the residual carried: random layer tables with every bin
length class, value kinds with ties, zeros and denormals, scale factors
1 (the gradient reading then sends exactly the bin maxima) to 3.5; and the
LSTM language model's table at full size."""
import numpy as np
import pytest
import torch

import oracle
from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W
from tests.gpu_util import HipPath, dev, same_bits, say, to_dev, ulp_report

pytestmark = pytest.mark.gpu

RULES = [(B.GC_ADACOMP_RULE_GRADIENT, oracle.RULE_GRADIENT), (B.GC_ADACOMP_RULE_RESIDUAL, oracle.RULE_RESIDUAL)]


def run_steps(t, steps, sf, rule, deferred, rng, kind):
    hp = HipPath(t)
    n = hp.n
    R = W.random_values(rng, n, kind)
    Rd = to_dev(R)
    state = hp.plan.adacomp_state(dev()) if deferred else None
    for step in range(steps):
        dW = W.random_values(rng, n, kind)
        R, idx, val, off, scale, _ = oracle.adacomp(t, dW, R, sf, rule=rule[1])
        gR, gi, gv, go, gs = hp.adacomp(to_dev(dW), Rd, sf, state=state, rule=rule[0])
        assert np.array_equal(go, off), f"offsets, step {step}"
        assert np.array_equal(gi, idx), f"indices, step {step}"
        assert same_bits(gv, val), ulp_report(gv, val)
        assert same_bits(gs, scale), ulp_report(gs, scale)
        assert same_bits(gR, R), ulp_report(gR, R)


@pytest.mark.parametrize("deferred", [False, True], ids=["exact", "deferred"])
@pytest.mark.parametrize("kind", ["normal", "laplace", "ties", "zeros", "denormal"])
@pytest.mark.parametrize("sf", [1.0, 2.0, 3.5])
def test_gradient_rule_random_tables(sf, kind, deferred):
    rng = np.random.default_rng(9100 + int(sf * 10) + 7 * ["normal", "laplace", "ties", "zeros", "denormal"].index(kind))
    t = W.random_table(rng, int(rng.integers(1, 9)), max_len=70_000, gaps=True)
    say(f"adacomp gradient rule sf={sf} kind={kind} deferred={deferred} nseg={len(t)}")
    run_steps(t, 3, sf, RULES[0], deferred, rng, kind)


@pytest.mark.parametrize("deferred", [False, True], ids=["exact", "deferred"])
def test_every_bin_length_class(deferred):
    rng = np.random.default_rng(9200)
    lens = [1, 2, 63, 4095, 4096, 4097, 12289, 50000]
    bls = [1, 7, 50, 64, 500, 4096, 3, 2048]
    t = W.make_table(lens, bls, None, [0, 3, 1, 0, 5, 2, 0, 1])
    for rule in RULES:
        say(f"adacomp bin length classes rule={rule[0]} deferred={deferred}")
        run_steps(t, 2, 2.0, rule, deferred, rng, "normal")


def test_lstm_full_size_both_modes():
    w = W.make_config("lstm_lm")
    n = w.n_total
    hp = HipPath(w.table, n)
    R = np.zeros(n, np.float32)
    Re = torch.zeros(n, dtype=torch.float32, device=dev())
    Rd = torch.zeros_like(Re)
    state = hp.plan.adacomp_state(dev())
    ws = hp.workspace(B.GC_OP_ADACOMP)
    oe = B.Sparse.empty(hp.plan, n, dev())
    od = B.Sparse.empty(hp.plan, n, dev())
    rule = B.GC_ADACOMP_RULE_GRADIENT
    for step in range(4):
        g = W.gradient_device(w, step, dev())
        say(f"lstm adacomp gradient rule step {step}: hip")
        B.gc_adacomp_compress(hp.plan, g, Re, 2.0, oe, ws, rule=rule)
        B.gc_adacomp_compress(hp.plan, g, Rd, 2.0, od, ws, state=state, rule=rule)
        torch.cuda.synchronize()
        say(f"lstm adacomp gradient rule step {step}: oracle")
        R, idx, val, off, scale, _ = oracle.adacomp(w.table, g.cpu().numpy(), R, 2.0, rule=oracle.RULE_GRADIENT)
        for label, o in (("exact", oe), ("deferred", od)):
            gi, gv, go, gs = o.host()
            assert np.array_equal(go, off) and np.array_equal(gi, idx), f"{label} step {step}"
            assert same_bits(gv, val), ulp_report(gv, val)
            assert same_bits(gs[:len(w.table)], scale), ulp_report(gs[:len(w.table)], scale)
    assert same_bits(Re.cpu().numpy(), R), ulp_report(Re.cpu().numpy(), R)
    exact = torch.empty_like(Rd)
    B.gc_adacomp_residual(hp.plan, Rd, state, exact)
    torch.cuda.synchronize()
    assert same_bits(exact.cpu().numpy(), R), ulp_report(exact.cpu().numpy(), R)


def test_ex_rejects_bad_options():
    t = W.make_table([5000], [50], [5])
    hp = HipPath(t)
    out = B.Sparse.empty(hp.plan, hp.n, dev())
    z = torch.zeros(hp.n, device=dev())
    for sf, rule in ((2.0, 7), (0.5, B.GC_ADACOMP_RULE_GRADIENT), (float("inf"), B.GC_ADACOMP_RULE_GRADIENT)):
        with pytest.raises(B.GCError):
            B.gc_adacomp_compress(hp.plan, z, z.clone(), sf, out, hp.workspace(B.GC_OP_ADACOMP), rule=rule)
