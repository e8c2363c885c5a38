"""Pins of the oracle's replica-side DCD-PSGD steps (replica decode, mixing)
and of ECD-PSGD's extrapolation (Eq. 3) and estimate update (Eq. 4), against
hand-derived values and properties fixed by the pages and the mathematics."""
import json
import os

import numpy as np
import pytest

import oracle


def load(golden_dir):
    with open(os.path.join(golden_dir, "dcd_replica_hand.json")) as f:
        return json.load(f)


def test_decode_hand(golden_dir):
    for c in load(golden_dir)["decode"]:
        got = oracle.dcd_decode(c["scales"], np.array(c["codes"], np.uint8), c["x_hat"],
                                c["bits"], c["bucket"])
        assert got.tolist() == c["expect"], c["name"]


def test_mix_hand(golden_dir):
    for c in load(golden_dir)["mix"]:
        got = oracle.dcd_mix(c["replicas"], c["weights"], c["grad"], c["lr"])
        assert got.tolist() == c["expect"], c["name"]


def test_ecd_hand(golden_dir):
    for c in load(golden_dir)["ecd"]:
        sc, codes = oracle.ecd_compress(c["x_prev"], c["x"], c["t"], c["bits"], c["bucket"], seed=5)
        assert sc.tolist() == c["expect_scales"], c["name"]
        assert codes.tolist() == c["expect_codes"], c["name"]
        xt = oracle.ecd_update(sc, codes, c["x_prev"], c["t"], c["bits"], c["bucket"])
        assert xt.tolist() == c["expect_x_tilde"], c["name"]


@pytest.mark.parametrize("bits,bucket,n", [(4, 512, 100_003), (8, 512, 4097), (4, 4, 9), (8, 4096, 1)])
def test_replica_tracks_the_sender(bits, bucket, n):
    """DCD-PSGD keeps every neighbour's replica equal to the sender's model:
    decoding the transmitted codes onto x_t reproduces x_{t+1} = x_t + C(z)
    bit for bit, step after step."""
    rng = np.random.default_rng(n + bits)
    x = rng.normal(0, 0.05, n).astype(np.float32)
    rep = x.copy()
    for step in range(3):
        xh = (x - np.float32(0.1) * rng.normal(0, 1e-2, n).astype(np.float32)).astype(np.float32)
        x_next, sc, codes = oracle.dcd(x, xh, bits, bucket, seed=11, step=step)
        rep = oracle.dcd_decode(sc, codes, rep, bits, bucket)
        assert np.array_equal(rep.view(np.uint32), x_next.view(np.uint32))
        x = x_next


def test_mix_identity_and_linearity():
    rng = np.random.default_rng(3)
    n = 5000
    x = (rng.integers(-2 ** 20, 2 ** 20, n) * 2.0 ** -22).astype(np.float32)
    # identical replicas, weights summing to 1 (powers of two), no gradient: x exactly
    out = oracle.dcd_mix([x, x, x], [0.5, 0.25, 0.25], np.zeros(n, np.float32), 0.1)
    assert np.array_equal(out, x)
    # one replica with weight 1: a plain SGD step, x - lr g, each term rounded once
    g = rng.normal(0, 1, n).astype(np.float32)
    out = oracle.dcd_mix([x], [1.0], g, 0.5)
    assert np.array_equal(out, (x.astype(np.float64) - 0.5 * g.astype(np.float64)).astype(np.float32))


def test_ecd_t2_codes_equal_dcd_of_x():
    """At t = 2 Eq. (3) sends C(x_t) itself (1 - t/2 = 0): the same bytes as
    quantizing the difference x_t - 0 with the same seed and step."""
    rng = np.random.default_rng(4)
    n = 3001
    xp = rng.normal(0, 1, n).astype(np.float32)
    x = rng.normal(0, 1, n).astype(np.float32)
    sc, codes = oracle.ecd_compress(xp, x, 2, 4, 512, seed=77)
    _, sc2, codes2 = oracle.dcd(np.zeros(n, np.float32), x, 4, 512, seed=77, step=2)
    assert np.array_equal(sc, sc2) and np.array_equal(codes, codes2)


@pytest.mark.parametrize("t", [1, 4])
def test_ecd_lossless_reconstruction(t):
    """With a lossless C (every |z| a grid level), Eqs. (3) and (4) recover
    x_t exactly from x~_{t-1} = x_{t-1} (the coefficients at t = 1 and 4 are
    exact in fp32)."""
    rng = np.random.default_rng(t)
    n = 4096
    a, b = 1 - t / 2, t / 2
    # pick integer z on the 8-bit grid of each bucket (max 127) and x_prev, then x
    z = rng.integers(-127, 128, n).astype(np.float64)
    z[::512] = 127
    xp = rng.integers(-64, 64, n).astype(np.float64)
    x = (z - a * xp) / b
    sc, codes = oracle.ecd_compress(xp, x, t, 8, 512, seed=1)
    assert np.all(sc == 127)
    xt = oracle.ecd_update(sc, codes, xp, t, 8, 512)
    assert np.array_equal(xt.astype(np.float64), x)


def test_ecd_estimate_unbiased():
    """E[x~_t] = x_t when x~_{t-1} = x_{t-1} (C is unbiased, Eqs. (3) and (4)
    are linear in z): the mean over many seeds approaches x_t."""
    rng = np.random.default_rng(9)
    n = 1024
    t = 3
    xp = rng.uniform(-1, 1, n).astype(np.float32)
    x = (xp + rng.uniform(-0.1, 0.1, n)).astype(np.float32)
    acc = np.zeros(n)
    T = 400
    for seed in range(T):
        sc, codes = oracle.ecd_compress(xp, x, t, 4, 512, seed=seed)
        acc += oracle.ecd_update(sc, codes, xp, t, 4, 512)
    mean = acc / T
    z = (1 - t / 2) * xp.astype(np.float64) + (t / 2) * x
    step = np.abs(z).max() / 7
    # C's per-element sd <= step / 2; x~ scales it by 2/t; plus fp32 rounding of the coefficients
    assert np.max(np.abs(mean - x)) < 5 * (2 / t) * step / (2 * np.sqrt(T)) + 1e-5
