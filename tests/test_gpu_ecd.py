"""GPU parity of the replica side of DCD-PSGD (replica decode, mixing) and of
ECD-PSGD (Eq. 3 extrapolate-and-compress, Eq. 4 estimate update), through
the C ABI against the oracle, bit for bit, over sizes with ragged tails,
both code widths, several buckets and unaligned pointers; and at the
DeepSpeech-scale model size."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W
from tests.gpu_util import same_bits, say, to_dev, ulp_report

pytestmark = pytest.mark.gpu

SIZES = [1, 3, 4, 5, 511, 513, 4096, 4097, 100_003]


def shifted(a, offset):
    """A device copy of a at a float offset inside a larger buffer (offset 0:
    256-byte aligned)."""
    buf = torch.zeros(len(a) + offset, dtype=torch.float32, device="cuda")
    buf[offset:] = torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    return buf, buf[offset:]


def stream_of(n, bits, bucket, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 0.05, n).astype(np.float32)
    xh = (x - np.float32(0.1) * rng.normal(0, 1e-3, n).astype(np.float32)).astype(np.float32)
    _, sc, codes = oracle.dcd(x, xh, bits, bucket, seed=seed, step=3)
    return x, sc, codes


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("bucket", [4, 512, 4096])
def test_dcd_decode_parity(n, bits, bucket):
    x, sc, codes = stream_of(n, bits, bucket, n + bits + bucket)
    rep = np.random.default_rng(n).normal(0, 0.05, n).astype(np.float32)
    want = oracle.dcd_decode(sc, codes, rep, bits, bucket)
    for offset in (0, 1):
        say(f"dcd_decode n={n} bits={bits} bucket={bucket} offset={offset}")
        _, xd = shifted(rep, offset)
        B.gc_dcd_decode(to_dev(sc), to_dev(codes, torch.uint8), xd, bits, bucket)
        torch.cuda.synchronize()
        got = xd.cpu().numpy()
        assert same_bits(got, want), ulp_report(got, want)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("K", [1, 3, 16])
def test_dcd_mix_parity(n, K):
    rng = np.random.default_rng(n * 3 + K)
    reps = [rng.normal(0, 0.05, n).astype(np.float32) for _ in range(K)]
    w = rng.dirichlet(np.ones(K)).astype(np.float32)
    g = rng.normal(0, 1e-2, n).astype(np.float32)
    want = oracle.dcd_mix(reps, w, g, 0.1)
    for offset in (0, 3):
        say(f"dcd_mix n={n} K={K} offset={offset}")
        dreps = [shifted(r, offset)[1] for r in reps]
        _, gd = shifted(g, offset)
        _, out = shifted(np.zeros(n, np.float32), offset)
        B.gc_dcd_mix(dreps, w, gd, 0.1, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert same_bits(got, want), ulp_report(got, want)


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("t", [1, 2, 3, 7, 1000])
def test_ecd_parity(n, bits, t):
    rng = np.random.default_rng(n * 5 + bits + t)
    bucket = 512 if n > 600 else 4
    xp = rng.normal(0, 0.05, n).astype(np.float32)
    x = (xp + rng.normal(0, 1e-3, n)).astype(np.float32)
    xt0 = (xp + rng.normal(0, 1e-4, n)).astype(np.float32)
    seed = int(rng.integers(0, 2 ** 63))
    sc, codes = oracle.ecd_compress(xp, x, t, bits, bucket, seed)
    xt = oracle.ecd_update(sc, codes, xt0, t, bits, bucket)
    for offset in (0, 1):
        say(f"ecd n={n} bits={bits} t={t} offset={offset}")
        _, xpd = shifted(xp, offset)
        _, xd = shifted(x, offset)
        gsc = torch.zeros(len(sc) + 1, dtype=torch.float32, device="cuda")
        gcodes = torch.zeros(len(codes) + 8, dtype=torch.uint8, device="cuda")
        B.gc_ecd_compress(xpd, xd, t, bits, bucket, seed, gsc, gcodes)
        _, xtd = shifted(xt0, offset)
        B.gc_ecd_update(gsc, gcodes, xtd, t, bits, bucket)
        torch.cuda.synchronize()
        assert same_bits(gsc[:len(sc)].cpu().numpy(), sc)
        gc_ = gcodes.cpu().numpy()
        assert np.array_equal(gc_[:len(codes)], codes)
        assert np.all(gc_[len(codes):] == 0), "wrote past the codes"
        got = xtd.cpu().numpy()
        assert same_bits(got, xt), ulp_report(got, xt)


def test_replica_hand_examples_on_gpu(golden_dir):
    with open(os.path.join(golden_dir, "dcd_replica_hand.json")) as f:
        g = json.load(f)
    for c in g["decode"]:
        xd = to_dev(np.array(c["x_hat"], np.float32))
        B.gc_dcd_decode(to_dev(np.array(c["scales"], np.float32)), to_dev(np.array(c["codes"], np.uint8), torch.uint8),
                        xd, c["bits"], c["bucket"])
        torch.cuda.synchronize()
        assert xd.cpu().numpy().tolist() == c["expect"], c["name"]
    for c in g["ecd"]:
        n = len(c["x"])
        sc = torch.zeros(1, dtype=torch.float32, device="cuda")
        codes = torch.zeros(4, dtype=torch.uint8, device="cuda")
        B.gc_ecd_compress(to_dev(np.array(c["x_prev"], np.float32)), to_dev(np.array(c["x"], np.float32)),
                          c["t"], c["bits"], c["bucket"], 5, sc, codes)
        xt = to_dev(np.array(c["x_prev"], np.float32))
        B.gc_ecd_update(sc, codes, xt, c["t"], c["bits"], c["bucket"])
        torch.cuda.synchronize()
        assert codes.cpu().numpy()[:n].tolist() == c["expect_codes"], c["name"]
        assert xt.cpu().numpy().tolist() == c["expect_x_tilde"], c["name"]


def test_errors_leave_buffers_untouched():
    x = torch.ones(100, dtype=torch.float32, device="cuda")
    sc = torch.ones(1, dtype=torch.float32, device="cuda")
    codes = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.GCError):
        B.gc_dcd_decode(sc, codes, x, 5, 512)
    with pytest.raises(B.GCError):
        B.gc_ecd_update(sc, codes, x, 0, 4, 512)
    with pytest.raises(B.GCError):
        B.gc_dcd_mix([x], [1.0], x, 0.1, x)  # output aliases the gradient
    torch.cuda.synchronize()
    assert torch.all(x == 1)


def test_deepspeech_scale_ring_round():
    """One DCD-PSGD round on a ring of 3 at the DeepSpeech model size (122M
    parameters): mix, compress, a neighbour's replica decode; then an ECD-PSGD
    send and receive, all against the oracle."""
    w = W.make_config("deepspeech")
    n = w.n_total
    x = W.dcd_model(w)
    g = W.gradient(w, 0)
    rng = np.random.default_rng(6)
    left = (x + rng.normal(0, 1e-4, n)).astype(np.float32)
    right = (x + rng.normal(0, 1e-4, n)).astype(np.float32)
    weights = [0.5, 0.25, 0.25]
    say("deepspeech ring: oracle")
    xh = oracle.dcd_mix([x, left, right], weights, g, 0.1)
    xo, sc, codes = oracle.dcd(x, xh, 4, 512, 0x5EED, 1)
    rep = oracle.dcd_decode(sc, codes, x, 4, 512)
    esc, ecodes = oracle.ecd_compress(x, xo, 2, 4, 512, 0x5EED)
    xt = oracle.ecd_update(esc, ecodes, x, 2, 4, 512)
    say("deepspeech ring: hip")
    xd, ld, rd, gd = (to_dev(a) for a in (x, left, right, g))
    xhd = torch.empty_like(xd)
    B.gc_dcd_mix([xd, ld, rd], weights, gd, 0.1, xhd)
    gsc = torch.zeros(len(sc), dtype=torch.float32, device="cuda")
    gcodes = torch.zeros(len(codes), dtype=torch.uint8, device="cuda")
    xod = torch.empty_like(xd)
    B.gc_dcd_compress(xd, xhd, xod, 4, 512, 0x5EED, 1, gsc, gcodes)
    repd = xd.clone()
    B.gc_dcd_decode(gsc, gcodes, repd, 4, 512)
    B.gc_ecd_compress(xd, xod, 2, 4, 512, 0x5EED, gsc, gcodes)
    xtd = xd.clone()
    B.gc_ecd_update(gsc, gcodes, xtd, 2, 4, 512)
    torch.cuda.synchronize()
    assert same_bits(xhd.cpu().numpy(), xh)
    assert same_bits(xod.cpu().numpy(), xo)
    assert same_bits(repd.cpu().numpy(), rep) and same_bits(rep, xo)
    assert np.array_equal(gcodes.cpu().numpy(), ecodes) and same_bits(gsc.cpu().numpy(), esc)
    assert same_bits(xtd.cpu().numpy(), xt)
