"""Seeded synthetic workloads: segment tables and input arrays.

This module only builds inputs.  It holds none of the compression arithmetic,
so both the HIP path's tests and the oracle can take their inputs from it.

The layer shapes stand in for the models the pages train (the datasets and
trained weights are not used; values are seeded random draws):
  fc1m       one fully connected layer gradient of 1,048,576 elements
  resnet50   ResNet-50 (torchvision parameter order): 161 tensors, 25,557,032
  lstm_lm    2-layer LSTM LM, hidden 1500, 10k x 1500 embedding and softmax
             (untied): 11 tensors, 66,034,000
  resnet50x8 eight ResNet-50 learners in one buffer: 1,288 segments
  deepspeech DeepSpeech-style model: 5 conv layers, 7 bidirectional GRU layers
             of hidden 800 and an FC layer: 68 tensors, 121,893,373

Every array is drawn in float64 with NumPy's PCG64 generator and cast once
to float32, so every consumer sees identical bits.  gradient_device() draws
the same distributions on a GPU with torch's seeded generator (float64, cast
once to float32), for runs that need a fresh full-size gradient per step:
NumPy takes about 11 s per DeepSpeech-scale gradient on one host core.  Its
values differ from gradient()'s; a consumer copies them to the host when the
oracle needs them.

A segment table is an int64 array of rows (offset, length, bin_len, k);
k is the 0.1%-density count ceil(length / 1000) unless a config says otherwise.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def topk_count(n: int, per_mille: int = 1) -> int:
    """ceil(n * per_mille / 1000) in integers (at least 1)."""
    return max(1, (n * per_mille + 999) // 1000)


# ----------------------------------------------------------------- shapes
def resnet50_shapes():
    """(name, shape, fan_in) in torchvision's parameter order."""
    out = [("conv1.weight", (64, 3, 7, 7), 3 * 49), ("bn1.weight", (64,), 1),
           ("bn1.bias", (64,), 1)]
    inp = 64
    for li, (w, blocks) in enumerate([(64, 3), (128, 4), (256, 6), (512, 3)], start=1):
        for b in range(blocks):
            p = f"layer{li}.{b}."
            out += [(p + "conv1.weight", (w, inp, 1, 1), inp),
                    (p + "bn1.weight", (w,), 1), (p + "bn1.bias", (w,), 1),
                    (p + "conv2.weight", (w, w, 3, 3), w * 9),
                    (p + "bn2.weight", (w,), 1), (p + "bn2.bias", (w,), 1),
                    (p + "conv3.weight", (4 * w, w, 1, 1), w),
                    (p + "bn3.weight", (4 * w,), 1), (p + "bn3.bias", (4 * w,), 1)]
            if b == 0:
                out += [(p + "downsample.0.weight", (4 * w, inp, 1, 1), inp),
                        (p + "downsample.1.weight", (4 * w,), 1),
                        (p + "downsample.1.bias", (4 * w,), 1)]
            inp = 4 * w
    out += [("fc.weight", (1000, 2048), 2048), ("fc.bias", (1000,), 1)]
    return out


def lstm_lm_shapes():
    out = [("embedding", (10000, 1500))]
    for layer in range(2):
        out += [(f"lstm.weight_ih_l{layer}", (6000, 1500)),
                (f"lstm.weight_hh_l{layer}", (6000, 1500)),
                (f"lstm.bias_ih_l{layer}", (6000,)),
                (f"lstm.bias_hh_l{layer}", (6000,))]
    out += [("softmax.weight", (10000, 1500)), ("softmax.bias", (10000,))]
    return out


def deepspeech_shapes():
    out = []
    convs = [(32, 1), (32, 32), (96, 32), (96, 96), (192, 96)]
    for i, (co, ci) in enumerate(convs):
        kh = 41 if i == 0 else 21
        out += [(f"conv{i}.weight", (co, ci, kh, 11)), (f"conv{i}.bias", (co,))]
    for layer in range(7):
        inp = 192 * 45 if layer == 0 else 1600
        for d in ("fwd", "rev"):
            p = f"gru{layer}.{d}."
            out += [(p + "weight_ih", (2400, inp)), (p + "weight_hh", (2400, 800)),
                    (p + "bias_ih", (2400,)), (p + "bias_hh", (2400,))]
    out += [("fc.weight", (29, 1600)), ("fc.bias", (29,))]
    return out


def make_table(lengths, bin_lens, ks=None, gaps=None) -> np.ndarray:
    lengths = [int(v) for v in lengths]
    bin_lens = [int(v) for v in bin_lens]
    ks = [topk_count(n) for n in lengths] if ks is None else [int(v) for v in ks]
    gaps = [0] * len(lengths) if gaps is None else [int(v) for v in gaps]
    rows, off = [], 0
    for n, lt, k, g in zip(lengths, bin_lens, ks, gaps):
        off += g
        rows.append((off, n, lt, k))
        off += n
    return np.array(rows, dtype=np.int64).reshape(-1, 4)


def table_extent(table) -> int:
    t = np.asarray(table).reshape(-1, 4)
    return int(t[-1, 0] + t[-1, 1]) if len(t) else 0


# ---------------------------------------------------------------- configs
@dataclass
class Workload:
    name: str
    table: np.ndarray
    n_total: int
    params: dict = field(default_factory=dict)
    fan_in: np.ndarray | None = None
    two_d: np.ndarray | None = None
    rows: np.ndarray | None = None

    @property
    def nseg(self) -> int:
        return len(self.table)


def _numel(shape):
    return int(math.prod(shape))


def make_config(name: str) -> Workload:
    if name == "fc1m":
        n = 1 << 20
        return Workload(name, make_table([n], [50]), n,
                        dict(bin_len=50, momentum=0.9, thr_G=0.0, num_nodes=1, steps=1, K=1))
    if name in ("resnet50", "resnet50x8"):
        sh = resnet50_shapes()
        reps = 8 if name == "resnet50x8" else 1
        lengths = [_numel(s) for _, s, _ in sh] * reps
        fan = np.array([f for _, _, f in sh] * reps, dtype=np.float64)
        t = make_table(lengths, [500] * len(lengths))
        return Workload(name, t, table_extent(t),
                        dict(momentum=0.9, thr_G=1.0, num_nodes=8 if reps == 8 else 1,
                             steps=1 if reps == 8 else 10, K=reps, learner_len=sum(lengths) // reps),
                        fan_in=fan)
    if name == "lstm_lm":
        sh = lstm_lm_shapes()
        lengths = [_numel(s) for _, s in sh]
        two = np.array([len(s) == 2 for _, s in sh])
        t = make_table(lengths, [500 if d else 50 for d in two])
        return Workload(name, t, table_extent(t), dict(steps=20, scale_factor=2.0),
                        two_d=two, rows=np.array([s[0] for _, s in sh]))
    if name == "deepspeech":
        sh = deepspeech_shapes()
        lengths = [_numel(s) for _, s in sh]
        t = make_table(lengths, [500] * len(lengths))
        return Workload(name, t, table_extent(t),
                        dict(momentum=0.9, thr_G=1.0, num_nodes=1, steps=10, bin_len=500,
                             dcd_bits=4, dcd_bucket=512, dcd_seed=0x5EED))
    raise KeyError(name)


CONFIG_NAMES = ("fc1m", "resnet50", "lstm_lm", "resnet50x8", "deepspeech")


def gradient(w: Workload, step: int = 0, learner: int = 0) -> np.ndarray:
    """The seeded fp32 gradient of a workload at a step (and learner)."""
    if w.name == "fc1m":
        return _rng(1 + step).normal(0.0, 1e-3, w.n_total).astype(np.float32)
    if w.name == "resnet50":
        return _resnet_grad(w, 2000 + step, 0, w.n_total)
    if w.name == "resnet50x8":
        out = np.empty(w.n_total, np.float32)
        per = w.params["learner_len"]
        for j in range(8):
            out[j * per:(j + 1) * per] = _resnet_grad(w, 4000 + j, j * per, per)
        return out
    if w.name == "lstm_lm":
        rng = _rng(3000 + step)
        g = rng.normal(0.0, 1e-3, w.n_total)
        for s, (off, n, _, _) in enumerate(w.table):
            if not w.two_d[s]:
                continue
            rows = int(w.rows[s])
            cols = int(n) // rows
            heavy = np.nonzero(rng.random(rows) < 0.02)[0]
            block = g[off:off + n].reshape(rows, cols)
            block[heavy] = 1e-3 * rng.standard_t(3.0, size=(heavy.size, cols))
        return g.astype(np.float32)
    if w.name == "deepspeech":
        rng = _rng(5000 + step)
        sigma = 1e-3 * np.exp(rng.normal(0.0, 1.0, w.nseg))
        g = rng.standard_normal(w.n_total)
        for s, (off, n, _, _) in enumerate(w.table):
            g[off:off + n] *= sigma[s]
        return g.astype(np.float32)
    raise KeyError(w.name)


def gradient_device(w: Workload, step: int = 0, device="cuda"):
    """A seeded fp32 gradient drawn on `device` (torch tensor): the same
    recipe and seeds as gradient() (fc1m 1 + step, resnet50 2000 + step,
    lstm_lm 3000 + step, deepspeech 5000 + step), with torch's generator for
    the per-element draws and NumPy's PCG64 for the few per-tensor and
    per-row ones (DeepSpeech's layer scales, the LSTM's heavy rows)."""
    import torch

    def gen(seed):
        return torch.Generator(device=device).manual_seed(seed)

    f64 = dict(dtype=torch.float64, device=device)
    if w.name == "fc1m":
        return (torch.randn(w.n_total, generator=gen(1 + step), **f64) * 1e-3).float()
    if w.name == "resnet50":
        u = torch.rand(w.n_total, generator=gen(2000 + step), **f64) - 0.5
        g = -1e-3 * torch.sign(u) * torch.log1p(-2.0 * u.abs())  # Laplace(0, 1e-3) by inversion
        for s, (off, n, _, _) in enumerate(w.table):
            g[off:off + n] *= float(w.fan_in[s]) ** -0.5
        return g.float()
    if w.name == "lstm_lm":
        gg = gen(3000 + step)
        rng = _rng(3000 + step)
        g = torch.randn(w.n_total, generator=gg, **f64) * 1e-3
        for s, (off, n, _, _) in enumerate(w.table):
            if not w.two_d[s]:
                continue
            rows = int(w.rows[s])
            cols = int(n) // rows
            heavy = torch.from_numpy(np.nonzero(rng.random(rows) < 0.02)[0]).to(device)
            z = torch.randn(heavy.numel(), cols, generator=gg, **f64)
            chi2 = torch.randn(3, heavy.numel(), cols, generator=gg, **f64).square().sum(0)
            block = g[off:off + n].view(rows, cols)
            block[heavy] = 1e-3 * z * torch.sqrt(3.0 / chi2)  # Student-t, nu = 3
        return g.float()
    if w.name == "deepspeech":
        sigma = 1e-3 * np.exp(_rng(5000 + step).normal(0.0, 1.0, w.nseg))
        g = torch.randn(w.n_total, generator=gen(5000 + step), **f64)
        for s, (off, n, _, _) in enumerate(w.table):
            g[off:off + n] *= float(sigma[s])
        return g.float()
    raise KeyError(w.name)


def _resnet_grad(w: Workload, seed: int, base: int, count: int) -> np.ndarray:
    g = _rng(seed).laplace(0.0, 1e-3, count)
    for s, (off, n, _, _) in enumerate(w.table):
        if base <= off < base + count:
            g[off - base:off - base + n] *= w.fan_in[s] ** -0.5
    return g.astype(np.float32)


def dcd_model(w: Workload) -> np.ndarray:
    """Model replica x_t for the compressed-difference step: N(0, 0.05^2)."""
    return _rng(5999).normal(0.0, 0.05, w.n_total).astype(np.float32)


def dcd_half_step(x: np.ndarray, g: np.ndarray, lr: float = 0.1) -> np.ndarray:
    """A synthetic x_{t+1/2}: the local model after one SGD step, in fp32."""
    return (x - np.float32(lr) * g).astype(np.float32)


# ------------------------------------------------------------- test tables
def random_table(rng: np.random.Generator, nseg: int, max_len: int = 5000,
                 bin_lens=(1, 7, 50, 64, 500), per_mille=(1, 10, 100, 1000),
                 gaps: bool = False, special_lengths=(1, 2, 63, 64, 65, 4095, 4096, 4097)):
    """A random segment table with odd offsets and lengths for parity tests."""
    lengths, bls, ks, gp = [], [], [], []
    for _ in range(nseg):
        if rng.random() < 0.3:
            n = int(rng.choice(special_lengths))
        else:
            n = int(rng.integers(1, max_len + 1))
        lengths.append(n)
        bls.append(int(rng.choice(bin_lens)))
        pm = int(rng.choice(per_mille))
        ks.append(min(n, topk_count(n, pm)))
        gp.append(int(rng.integers(0, 5)) if gaps else 0)
    return make_table(lengths, bls, ks, gp)


def random_values(rng: np.random.Generator, n: int, kind: str = "normal",
                  scale: float = 1e-3) -> np.ndarray:
    """fp32 values with a few distributions (ties, zeros, denormals)."""
    if kind == "normal":
        return rng.normal(0.0, scale, n).astype(np.float32)
    if kind == "laplace":
        return rng.laplace(0.0, scale, n).astype(np.float32)
    if kind == "ties":
        return (rng.integers(-3, 4, n) * scale).astype(np.float32)
    if kind == "zeros":
        v = rng.normal(0.0, scale, n)
        v[rng.random(n) < 0.7] = 0.0
        return v.astype(np.float32)
    if kind == "denormal":
        return (rng.normal(0.0, 1.0, n) * 1e-40).astype(np.float32)
    if kind == "const":
        return np.full(n, scale, np.float32)
    raise KeyError(kind)
