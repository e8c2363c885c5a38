"""GPU parity of Slim-DP's core and explorer selection (Slim-DP §3) through
the C ABI against the oracle, bit for bit: core indices, significances,
bitmap words, explorer indices and values, the values-only core push; on
random layouts (ragged tails, odd offsets, gaps, ties, zeros), the hand
examples, and the DeepSpeech layout at the page's VGG-16 setting
(alpha = 0.2, beta = 0.1)."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W
from tests.gpu_util import same_bits, say, to_dev
from tests.test_gpu_parity import _dgc_sample_positions, mixed_table
from tests.test_oracle_slimdp import _arr

pytestmark = pytest.mark.gpu


def with_k(t, frac):
    t = np.array(t, np.int64)
    t[:, 3] = np.clip(np.ceil(t[:, 1] * frac).astype(np.int64), 1, None)
    return t


class SlimDP:
    def __init__(self, table_core, table_explore):
        self.core_plan = B.Plan(table_core)
        self.exp_plan = B.Plan(table_explore, self.core_plan.n_total)
        self.n = self.core_plan.n_total
        self.ws = self.core_plan.workspace(B.GC_OP_DGC, "cuda")
        self.mask = torch.zeros(max(B.gc_slimdp_mask_words(self.core_plan), 1), dtype=torch.int32, device="cuda")

    def core(self, w, g, c):
        core = B.Sparse.empty(self.core_plan, self.core_plan.total_k, "cuda")
        B.gc_slimdp_core(self.core_plan, to_dev(w), to_dev(g), c, core, self.mask, self.ws)
        torch.cuda.synchronize()
        return core

    def explore(self, delta, seed, step):
        out = B.Sparse.empty(self.exp_plan, self.exp_plan.total_k, "cuda")
        B.gc_slimdp_explore(self.exp_plan, self.core_plan, to_dev(delta), self.mask, seed, step, out, self.ws)
        torch.cuda.synchronize()
        return out

    def mask_host(self):
        return self.mask.cpu().numpy().view(np.uint32)[:B.gc_slimdp_mask_words(self.core_plan)]


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("kind", ["normal", "laplace", "ties", "zeros"])
@pytest.mark.parametrize("beta,extra", [(0.1, 0.1), (0.15, 0.15), (0.5, 0.3)])
def test_core_and_explorer_parity(seed, kind, beta, extra):
    rng = np.random.default_rng(700 + seed)
    t = mixed_table(rng, int(rng.integers(1, 10)))
    t = t[t[:, 1] >= 2]  # a core and an explorer per segment
    tc = with_k(t, beta)
    te = with_k(t, extra)
    te[:, 3] = np.minimum(te[:, 3], t[:, 1] - tc[:, 3])
    n = W.table_extent(t)
    sd = SlimDP(tc, te)
    w = W.random_values(rng, n, kind)
    g = W.random_values(rng, n, kind)
    c = float(rng.choice([0.25, 1.0, 37.5]))
    say(f"slimdp core seed={seed} kind={kind} beta={beta} n={n} c={c}")
    cidx, cval, coff, cmask = oracle.slimdp_core(tc, w, g, c)
    core = sd.core(w, g, c)
    gi, gv, go, _ = core.host()
    assert np.array_equal(go, coff) and np.array_equal(gi, cidx)
    assert same_bits(gv, cval)
    assert np.array_equal(sd.mask_host(), cmask)
    d = W.random_values(rng, n, "normal")
    for step in range(2):
        say(f"slimdp explore seed={seed} kind={kind} step={step}")
        eidx, evals, eoff = oracle.slimdp_explore(te, d, cmask, 99 + seed, step)
        out = sd.explore(d, 99 + seed, step)
        xi, xv, xo, _ = out.host()
        assert np.array_equal(xo, eoff) and np.array_equal(xi, eidx)
        assert same_bits(xv, evals)
    vals = torch.zeros(max(len(cidx), 1), dtype=torch.float32, device="cuda")
    B.gc_slimdp_core_values(sd.core_plan, core, to_dev(d), vals)
    torch.cuda.synchronize()
    assert same_bits(vals.cpu().numpy()[:len(cidx)], d[cidx])


def test_hand_examples_on_gpu(golden_dir):
    with open(os.path.join(golden_dir, "slimdp_hand.json")) as f:
        cases = json.load(f)["core"]
    for c in cases:
        t = np.array(c["segments"], np.int64)
        n = int(t[-1, 0] + t[-1, 1])
        te = t.copy()
        te[:, 3] = 1
        sd = SlimDP(t, te)
        say(f"slimdp hand {c['name']}")
        core = sd.core(_arr(c["w"], n), _arr(c["g"], n), c["c"])
        gi, gv, _, _ = core.host()
        assert gi.tolist() == c["expect_idx"] and gv.tolist() == c["expect_val"]
        assert sd.mask_host().tolist() == c["expect_mask"]


def test_explorer_rejects_mismatched_plans():
    t = W.make_table([5000, 300], [1, 1], [100, 10])
    sd = SlimDP(t, W.make_table([5000, 300], [1, 1], [4901, 1]))  # 100 + 4901 > 5000
    with pytest.raises(B.GCError):
        sd.explore(np.zeros(sd.n, np.float32), 1, 0)
    other = B.Plan(W.make_table([5000, 301], [1, 1], [1, 1]))
    out = B.Sparse.empty(other, other.total_k, "cuda")
    with pytest.raises(B.GCError):
        B.gc_slimdp_explore(other, sd.core_plan, to_dev(np.zeros(other.n_total, np.float32)), sd.mask, 1, 0,
                            out, sd.ws)


def test_deepspeech_vgg_setting():
    """alpha = 0.2, beta = 0.1 (the page's VGG-16 setting) on the DeepSpeech
    layout: a core of 10% per tensor and an explorer of another 10%."""
    wl = W.make_config("deepspeech")
    tc = with_k(wl.table, 0.1)
    te = with_k(wl.table, 0.1)
    sd = SlimDP(tc, te)
    n = wl.n_total
    w = W.dcd_model(wl)
    g = W.gradient(wl, 0)
    say("deepspeech slimdp core: oracle")
    cidx, cval, coff, cmask = oracle.slimdp_core(tc, w, g, 50.0)
    say("deepspeech slimdp core: hip")
    core = sd.core(w, g, 50.0)
    gi, gv, go, _ = core.host()
    assert np.array_equal(gi, cidx) and same_bits(gv, cval) and np.array_equal(sd.mask_host(), cmask)
    d = W.gradient(wl, 1)
    say("deepspeech slimdp explore")
    eidx, evals, eoff = oracle.slimdp_explore(te, d, cmask, 7, 3)
    xi, xv, xo, _ = sd.explore(d, 7, 3).host()
    assert np.array_equal(xi, eidx) and same_bits(xv, evals)
    assert abs(len(xi) + len(gi) - 0.2 * n) < 0.001 * n


@pytest.mark.parametrize("wide", [False, True], ids=["3seg", "wide"])
def test_core_sample_bound_fallback(wide):
    """Adversarial significances for the sampled staging bound of the core
    selection: the sampled elements of one tensor carry its largest |w|,
    spread over many octaves, so the bound lies far above the true k-th
    largest significance and the tensor is re-staged from w and g with the
    significance recomputed.  Bit-exact against the oracle.  The wide plan
    adds 16,400 one-chunk tensors, past the 16,384 chunks from which the
    candidate kernels give each wave four chunks."""
    rng = np.random.default_rng(93)
    extra = 16400 if wide else 0
    lens = [3000, 4096 * 16 + 123, 50000] + [64] * extra
    t = W.make_table(lens, [50] * len(lens), [max(1, math.ceil(0.1 * x)) for x in lens])
    n = W.table_extent(t)
    w_ = (rng.standard_normal(n) * 1e-20).astype(np.float32)
    g_ = (rng.standard_normal(n) * 1e-20).astype(np.float32)
    pos = _dgc_sample_positions(t)
    o1, l1 = int(t[1][0]), int(t[1][1])
    inseg = pos[(pos >= o1) & (pos < o1 + l1)]
    mags = (np.float32(2.0) ** (-(np.arange(inseg.size) / 4.0))).astype(np.float32)
    w_[inseg] = (mags * np.where(rng.random(inseg.size) < 0.5, -1, 1)).astype(np.float32)
    sd = SlimDP(t, t)
    say(f"slimdp core sample fallback wide={wide}")
    cidx, cval, coff, cmask = oracle.slimdp_core(t, w_, g_, 1.0)
    gi, gv, go, _ = sd.core(w_, g_, 1.0).host()
    assert np.array_equal(go, coff) and np.array_equal(gi, cidx) and same_bits(gv, cval)
    assert np.array_equal(sd.mask_host(), cmask)
