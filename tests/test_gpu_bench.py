"""bench.py end to end on the GPU, short: the deepspeech step through the
library, and its one JSON line checked field by field (the numbers must be
consistent with one another; their size is what the benchmark measures)."""
import json

import numpy as np
import pytest
import torch

import bench
from gradient_compression_dnn_amd import binding as B
from gradient_compression_dnn_amd import workloads as W

pytestmark = pytest.mark.gpu


def test_bench_line_schema_and_consistency(capsys):
    assert bench.main(["--steps", "2", "--warmup", "1", "--no-cpu-baseline", "--no-variants"]) == 0
    lines = [ln for ln in capsys.readouterr().out.splitlines() if ln.strip()]
    assert len(lines) == 1
    r = json.loads(lines[0])
    n = W.make_config("deepspeech").n_total

    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline", "methods"):
        assert key in r, key
    assert r["n_gpus"] == 1 and r["steps"] == 2 and r["warmup"] == 1
    assert r["higher_is_better"] is True and r["scaling"] == "weak" and r["data"] == "synthetic"
    assert r["dtype"] == "f32" and r["unit"] == "GB/s" and r["vs_baseline"] is None
    assert "workload" in r["config"] and "deepspeech" in r["config"]["workload"]
    assert r["cpu_baseline"] is None  # --no-cpu-baseline

    # value is the step's fp32 gradient bytes (DGC and AdaComp each read n) per second
    ms = r["ms_per_step"]
    assert ms > 0
    assert r["value"] == pytest.approx(2 * 4 * n / (ms / 1000.0) / 1e9, rel=1e-3)
    assert r["step_ms_min"] <= r["step_ms_median"]

    roof = r["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["kernel"] == "dgc_update"
    assert roof["algorithmic_bytes_per_launch"] == 20 * n
    assert roof["achieved"] == pytest.approx(20 * n / (roof["avg_us"] * 1e-6) / 1e9, rel=1e-3)
    assert roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    assert 0.0 < roof["frac"] < 1.0
    # counters are reported only for the sources they were taken on
    if roof["traffic"] is not None:
        assert r["source_digest"] == bench.source_digest()
        assert 0.9 * 20 * n < roof["traffic"] < 1.5 * 20 * n

    sc = r["stream_ceiling"]
    assert sc["unit"] == "GB/s" and sc["achieved"] > 0 and 0.0 < sc["frac"] < 1.0
    assert sc["dominant_share"] == pytest.approx(roof["achieved"] / sc["achieved"], rel=1e-3)
    assert 0.5 < sc["dominant_share"] < 1.3

    for name in ("dgc", "adacomp", "pack_both", "decode_both", "dcd"):
        m = r["methods"][name]
        assert m["ms"] > 0 and m["alg_bytes"] > 0
        assert m["alg_hbm_frac"] == pytest.approx(m["alg_bytes"] / (m["ms"] / 1000.0) / 1e9 / 8000.0, rel=2e-3)
    # the calls timed alone add up to about one step
    assert sum(m["ms"] for m in r["methods"].values()) == pytest.approx(ms, rel=0.15)

    msgs = r["messages"]
    assert msgs["dgc_entries"] == sum(W.topk_count(int(s[1])) for s in W.make_config("deepspeech").table)
    # per-kernel fractions: the bytes of all the kernel's launches in a step
    # over its time in the step (two decodes, each its own message)
    kf, kus = r["kernel_alg_hbm_frac"], r["kernel_us_per_step"]
    dec = 2 * 4 * n + 8 * (msgs["dgc_entries"] + msgs["adacomp_entries"])
    assert kf["decode"] == pytest.approx(dec / (kus["decode"] * 1e-6) / 1e9 / 8000.0, rel=2e-3)
    assert kf["dgc_update"] == pytest.approx(20 * n / (kus["dgc_update"] * 1e-6) / 1e9 / 8000.0, rel=2e-3)
    # each step of the run draws its own gradient
    assert "fresh seeded gradient per step" in r["config"]["gradients"]
    assert 0 < msgs["adacomp_entries"] <= n
    assert msgs["dgc_packed_bytes"] > 8 * msgs["dgc_entries"] // 2


def test_stream_probe_arithmetic_and_bounds():
    """The streaming reference computes d = a + b and e = c + d in fp32 and
    writes nothing past n (ragged chunk tails included)."""
    rng = np.random.default_rng(5)
    for n in (1, 4095, 4096 * 3 + 7):
        a, b, c = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
        d = torch.full((n + 64,), 7.0, device="cuda")
        e = torch.full((n + 64,), 7.0, device="cuda")
        B.gc_stream_probe(*(torch.from_numpy(x).cuda() for x in (a, b, c)), d[:n], e[:n])
        torch.cuda.synchronize()
        want_d = (a + b).astype(np.float32)
        want_e = (c + want_d).astype(np.float32)
        assert np.array_equal(d[:n].cpu().numpy().view(np.uint32), want_d.view(np.uint32))
        assert np.array_equal(e[:n].cpu().numpy().view(np.uint32), want_e.view(np.uint32))
        assert torch.all(d[n:] == 7.0) and torch.all(e[n:] == 7.0)
