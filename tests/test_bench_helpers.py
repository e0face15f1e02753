"""CPU checks of the benchmark's arithmetic and of the committed profile
summaries it reads: the roofline of the dominant kernel must follow from
profiles/ with the formulas below, whoever recomputes it."""
import glob
import os
import re
import sys
from types import SimpleNamespace

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

WORKLOAD = "codellama7b_doc16k_p256"
# the headline's document kernel (d = 128, 2 query blocks, 8 waves, decode,
# non-temporal key/value loads)
DOC_KERNEL = "doc_mfma_bf16_kernel<128, 2, 8, false, true>"


def _kv(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    return kv


def _profile_digest(path):
    return _kv(path)["kernel_source_digest"]


def test_median_and_geomean_intervals():
    m, (lo, hi) = bench.median_ci(list(range(1, 10)))
    assert m == 5.0 and lo <= m <= hi
    g, (glo, ghi) = bench.geomean_ci([2.0, 8.0, 2.0, 8.0])
    assert abs(g - 4.0) < 1e-12 and glo <= g <= ghi
    # a constant sample has a degenerate interval
    assert bench.median_ci([3.0] * 20)[1] == [3.0, 3.0]


def test_algorithmic_bytes_of_the_headline_step():
    # doc 16k, P = 256, H = 32, d = 128, bf16: the document's K and V once plus Q
    case = SimpleNamespace(q=torch.empty(0, dtype=torch.bfloat16), H=32, D=128, P=256, doc_len=16384,
                           seq_len=31825, own_slots=[list(range(59))] * 256)
    by = bench.step_bytes(case)
    st = bench.stage_algorithmic_bytes(by)
    assert st["document"] == 2 * 16384 * 32 * 128 * 2 + 256 * 32 * 128 * 2 == 270_532_608
    assert st["plan"] == 4 * 31825
    assert st["own_slots_merge"] == 2 * 59 * 256 * 32 * 128 * 2 + 2 * 256 * 32 * 128 * 2
    assert by["doc_flops"] == 4 * 128 * 32 * 256 * 16384


@pytest.mark.parametrize("flops_per_byte, bound", [(254.0, "hbm"), (400.0, "mfma")])
def test_roofline_bound_follows_the_ridge(monkeypatch, flops_per_byte, bound):
    monkeypatch.setattr(bench, "read_trace_avg_us", lambda *a: None)
    monkeypatch.setattr(bench, "read_pmc_traffic", lambda *a: None)
    monkeypatch.setattr(bench, "read_sq_counters", lambda *a: None)
    nbytes = 1.0e8
    us = 50.0
    gbs = nbytes / (us * 1e-6) / 1e9
    tflops = flops_per_byte * nbytes / (us * 1e-6) / 1e12
    kernels = {"document": {"us": us, "algorithmic_bytes": nbytes, "gbs": gbs, "flops": flops_per_byte * nbytes,
                            "mfma_tflops": tflops, "mfma_frac": tflops / bench.MFMA_BF16_PEAK_TFLOPS}}
    e = bench.roofline_entry("document", kernels, WORKLOAD, None)
    assert e["bound"] == bound
    assert abs(e["ridge_flop_per_byte"] - 312.5) < 1e-9
    if bound == "hbm":
        assert e["unit"] == "GB/s" and abs(e["frac"] - gbs / 8000.0) < 1e-12
    else:
        assert e["unit"] == "TFLOP/s" and abs(e["frac"] - tflops / 2500.0) < 1e-12


def test_kernel_trace_summary_gives_the_roofline(monkeypatch):
    path = os.path.join(ROOT, "profiles", f"kernels_{WORKLOAD}.txt")
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: _profile_digest(path))
    avg = bench.read_trace_avg_us("document", WORKLOAD)
    assert avg is not None and 20.0 < avg < 500.0
    # the row the reader picked is the document kernel's
    row = next(ln for ln in open(path) if ln.startswith(DOC_KERNEL))
    assert float(row.split(">", 1)[1].split()[1]) == avg
    # frac = algorithmic bytes / average duration / 8 TB/s
    frac = 270_532_608 / (avg * 1e-6) / 1e9 / 8000.0
    assert 0.0 < frac < 1.0
    # another source digest: the summary is not used
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 16)
    assert bench.read_trace_avg_us("document", WORKLOAD) is None


@pytest.mark.parametrize("stage", ["document", "own_slots_merge", "plan"])
def test_pmc_traffic_is_the_scaled_counter_sum(monkeypatch, stage):
    path = os.path.join(ROOT, "profiles", f"pmc_{stage}_{WORKLOAD}.txt")
    kv = _kv(path)
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: kv["kernel_source_digest"])
    got = bench.read_pmc_traffic(stage, WORKLOAD)
    want = 1024.0 * (float(kv["FETCH_SIZE_KiB"]) * float(kv["fetch_factor"]) +
                     float(kv["WRITE_SIZE_KiB"]) * float(kv["write_factor"]))
    # (the factors are printed rounded; the bytes use the exact ratio)
    assert got is not None and abs(got - want) <= 1e-4 * want
    assert abs(float(kv["traffic_over_algorithmic"]) - got / float(kv["algorithmic_bytes_per_launch"])) < 1e-3


def test_read_calibration_factors_match_the_profiles():
    kv = _kv(os.path.join(ROOT, "profiles", "pmc_read_calibration.txt"))
    text = open(os.path.join(ROOT, "profiles", "pmc_read_calibration.txt")).read()
    factors = {k: float(v.split()[0]) for k, v in kv.items() if k in ("fetch_factor", "write_factor")}
    for stage in ("document", "own_slots_merge", "plan"):
        pk = _kv(os.path.join(ROOT, "profiles", f"pmc_{stage}_{WORKLOAD}.txt"))
        assert abs(float(pk["fetch_factor"]) - factors["fetch_factor"]) < 5e-3, text
        assert abs(float(pk["write_factor"]) - factors["write_factor"]) < 5e-3, text


def test_sq_counter_ratios_follow_their_definitions(monkeypatch):
    path = os.path.join(ROOT, "profiles", f"pmc_sq_{WORKLOAD}.txt")
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: _profile_digest(path))
    c = bench.read_sq_counters("document", WORKLOAD)
    assert c is not None
    # recompute MfmaUtil from the raw counters of the document block
    block, inside = {}, False
    for ln in open(path):
        if ln and not ln.startswith((" ", "#")):
            inside = ln.startswith("document (")
            continue
        m = re.match(r"\s+(SQ_\w+|GRBM_\w+)\s+(\d+)\s*$", ln)
        if inside and m:
            block[m.group(1)] = int(m.group(2))
    cycles = block["GRBM_GUI_ACTIVE"] / 8.0
    mfma = block["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * 1024.0)
    lds = block["SQ_LDS_IDX_ACTIVE"] / (cycles * 256.0)
    assert abs(c["MfmaUtil"] - mfma) < 1.5e-3
    assert abs(c["LdsUtil"] - lds) < 1.5e-3


def _kernel_profiles():
    # every summary of this library's decode-path kernels (the counter
    # calibration and the streaming-read ceiling measure the chip on kernels
    # of known size, whatever the sources)
    return [p for p in glob.glob(os.path.join(ROOT, "profiles", "*.txt"))
            if os.path.basename(p) not in ("pmc_read_calibration.txt", "hbm_read_ceiling.txt")]


def test_profile_commands_run_committed_files_only():
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.txt")):
        text = open(path).read()
        assert "_work" not in text, path
        if os.path.basename(path).startswith(("kernels_", "pmc_")):
            assert "rocprofv3" in text, path
    for path in _kernel_profiles():
        assert "kernel_source_digest:" in open(path).read(), path


def test_profiles_share_one_source_digest():
    digests = {_profile_digest(p) for p in _kernel_profiles()}
    assert len(digests) == 1, digests


def test_headline_trace_and_counters_agree_on_the_kernel_time():
    # the counter run's cycles over the trace's average give a plausible
    # shader clock (the two runs measure the same kernel)
    sq = open(os.path.join(ROOT, "profiles", f"pmc_sq_{WORKLOAD}.txt")).read()
    m = re.search(r"document \(" + re.escape(DOC_KERNEL) + r"\): dispatches \d+, kernel-trace avg ([\d.]+) us", sq)
    assert m
    avg_sq = float(m.group(1))
    kt = open(os.path.join(ROOT, "profiles", f"kernels_{WORKLOAD}.txt")).read()
    row = next(ln for ln in kt.splitlines() if ln.startswith(DOC_KERNEL))
    assert abs(float(row.split(">", 1)[1].split()[1]) - avg_sq) < 0.05 * avg_sq
    g = re.search(r"document \(doc_mfma.*?GRBM_GUI_ACTIVE\s+(\d+)", sq, re.S)
    ghz = int(g.group(1)) / 8.0 / (avg_sq * 1e3)
    assert 1.0 < ghz < 2.6
    assert np.isfinite(ghz)
