"""bench.py's host-side logic, on the CPU: the one-GPU refusal, the
algorithmic byte counts per unit, and the committed counter readings that
are used only while the HIP sources match the ones they were taken on."""
import json
import os

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    err = capsys.readouterr().err
    assert "one GPU" in err and "--gpus 2" in err


def test_world_size_above_one_is_refused(monkeypatch, capsys):
    monkeypatch.setenv("WORLD_SIZE", "4")
    assert bench.main([]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_algorithmic_bytes_per_unit():
    n, nbins, k, ada, bucket = 1_000_000, 2_000, 1_000, 150_000, 512
    a = bench.algorithmic_bytes(n, nbins, k, ada, bucket)
    # (bytes per step over all launches, launches per step)
    assert a["dgc_update"] == (20 * n, 1)          # read G, U, V; write U, V
    assert a["dgc_norm"] == (4 * n, 1)             # read G
    assert a["ada_fold"] == (12 * n, 1)            # read R, dW; write R
    assert a["ada_emit"] == (8 * ada, 1)           # idx and val per entry
    assert a["dcd"] == (12 * n + n // 2 + 4 * ((n + bucket - 1) // bucket), 1)  # 12.5 B/elt + scales
    # two decodes, each writing the dense update and reading its message (idx + val)
    assert a["decode"] == (2 * 4 * n + 8 * (k + ada), 2)
    assert a["dgc_emit"] == (16 * k, 1)            # message and masking writes


def test_source_digest_is_stable_and_covers_the_sources():
    d = bench.source_digest()
    assert d == bench.source_digest() and len(d) == 16
    int(d, 16)


def _write_profile(root, digest):
    os.makedirs(os.path.join(root, "profiles"))
    data = {
        "source_digest": digest,
        "steps_in_run": 4,
        "step_hbm_bytes": 1234,
        "kernels": {
            "dgc_update": {"hbm_bytes_per_launch": 100, "launches": 4},
            "dgc_norm": {"hbm_bytes_per_launch": 10, "launches": 4},
            "ada_fold": {"hbm_bytes_per_launch": 7, "launches": 4},
            "pack_count": {"hbm_bytes_per_launch": 3, "launches": 8},
        },
    }
    with open(os.path.join(root, "profiles", "pmc_traffic_deepspeech.json"), "w") as f:
        json.dump(data, f)


def test_counter_readings_only_for_matching_sources(tmp_path, monkeypatch):
    _write_profile(str(tmp_path), "abcdef0123456789")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("dgc_update", "abcdef0123456789") == 100
    assert bench.stored_traffic("dgc_update", "0000000000000000") is None
    assert bench.stored_traffic("no_such_kernel", "abcdef0123456789") is None
    assert bench.stored_step_traffic("abcdef0123456789") == 1234
    assert bench.stored_step_traffic("0000000000000000") is None
    # per step: launches / steps_in_run of each matching kernel
    assert bench.stored_call_traffic(("dgc_",), "abcdef0123456789") == 110
    assert bench.stored_call_traffic(("pack_",), "abcdef0123456789") == 6
    assert bench.stored_call_traffic(("dgc_",), "0000000000000000") is None


def test_missing_profile_reads_as_unmeasured(tmp_path, monkeypatch):
    d = bench.source_digest()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.stored_traffic("dgc_update", d) is None
    assert bench.stored_step_traffic(d) is None
    assert bench.stored_call_traffic(("dgc_",), d) is None
