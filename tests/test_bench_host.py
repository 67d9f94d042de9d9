"""Host-side checks of bench.py's measurement arithmetic (no GPU).

The rocprofv3 summary that profiles/kernels_<workload>.md holds is written by
bench.summarize_profile from the profiler's CSV files, and bench.py reads the
attention's HBM bytes per launch back from it.  These tests feed the
summariser small CSV files in rocprofv3's column layout, with counter values
chosen so that every derived figure has a hand-computed value, and check the
read-back's source-hash guard.
"""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

WL = "unit_test_workload"
ATTN = "void xattn::(anonymous namespace)::attn_pp<128, 3>(xattn::AttnArgs, int)"
EST = "void xattn::(anonymous namespace)::est_gemm_bf16<128, 8, 256, 256, 8, 2, 64, false, 1>(xattn::EstArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>, std::array<char*, 3ul> >"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _profile_dir(tmp_path, with_pmc=True):
    base = tmp_path / "prof"
    # kernel trace statistics: attention 800 us, estimate 70 us on average
    _write_csv(str(base / ("prof_%s" % WL) / "host" / "trace_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
               [[ATTN, 10, 8000000, 800000, 91.0, 790000, 810000, 1.0],
                [EST, 10, 700000, 70000, 9.0, 69000, 71000, 1.0]])
    line = {"ms_per_step": 0.9, "value": 4.5e6, "config": {"density": [1.0]},
            "stages": {"step_ms_median": 0.89, "attn_kernel_ms": 0.8, "estimate_ms": 0.07,
                       "estimate_flops": 64.0e9},
            "roofline": {"flops_per_launch": 1000.0e9}}
    (base / ("prof_%s.json" % WL)).write_text("warm-up output\n" + json.dumps(line) + "\n")
    if with_pmc:
        hdr = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
        # the copy kernel moves 512 MiB each way: FETCH_SIZE reads half of it
        # (factor 2), WRITE_SIZE all of it (factor 1)
        _write_csv(str(base / ("pmc_fetch_%s" % WL) / "host" / "pmc_counter_collection.csv"), hdr,
                   [[1, 1, COPY, "FETCH_SIZE", 262144.0],
                    [2, 2, ATTN, "FETCH_SIZE", 100000.0], [3, 3, ATTN, "FETCH_SIZE", 120000.0],
                    [4, 4, EST, "FETCH_SIZE", 70000.0]])
        _write_csv(str(base / ("pmc_write_%s" % WL) / "host" / "pmc_counter_collection.csv"), hdr,
                   [[1, 1, COPY, "WRITE_SIZE", 524288.0],
                    [2, 2, ATTN, "WRITE_SIZE", 40000.0], [3, 3, ATTN, "WRITE_SIZE", 40000.0],
                    [4, 4, EST, "WRITE_SIZE", 8000.0]])
        _write_csv(str(base / ("pmc_mfma_%s" % WL) / "host" / "pmc_counter_collection.csv"), hdr,
                   [[2, 2, ATTN, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0e9],
                    [4, 4, EST, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.125e9]])
        # LDS / MFMA busy pass: the attention's GRBM_GUI_ACTIVE over 8 XCDs is
        # 1.3e6 clocks (1.625 GHz over its 800 us), its MFMA pipes busy 1.0e9
        # SIMD-cycles of 1024 x 1.3e6
        _write_csv(str(base / ("pmc_lds_%s" % WL) / "host" / "pmc_counter_collection.csv"), hdr,
                   [[2, 2, ATTN, "SQ_LDS_IDX_ACTIVE", 1.0e8], [2, 2, ATTN, "SQ_LDS_BANK_CONFLICT", 5.0e4],
                    [2, 2, ATTN, "SQ_VALU_MFMA_BUSY_CYCLES", 1.0e9], [2, 2, ATTN, "GRBM_GUI_ACTIVE", 1.04e7],
                    [4, 4, EST, "SQ_LDS_IDX_ACTIVE", 6.0e6], [4, 4, EST, "SQ_LDS_BANK_CONFLICT", 3.0e6],
                    [4, 4, EST, "SQ_VALU_MFMA_BUSY_CYCLES", 6.5e7], [4, 4, EST, "GRBM_GUI_ACTIVE", 1.0e6]])
    return str(base)


def _row(text, name):
    for line in text.splitlines():
        if line.startswith("| %s |" % name):
            return [c.strip() for c in line.strip("|").split("|")]
    raise AssertionError("no row for %s" % name)


def test_summary_calibrates_bytes_and_rates(tmp_path):
    out = tmp_path / "profiles"
    out.mkdir()
    bench.summarize_profile(_profile_dir(tmp_path), WL, out_dir=str(out))
    text = (out / ("kernels_%s.md" % WL)).read_text()
    assert "FETCH_SIZE is scaled by 2.000 and WRITE_SIZE by 1.000" in text
    # every command that made the summary is listed, for this workload
    assert text.count("--workload %s" % WL) == len(bench.PROFILE_COMMANDS)
    assert "attention.hip %s" % bench.source_hash("attention.hip") in text

    # durations: the trace's averages in microseconds
    attn = _row(text, "attn_pp<128, 3>")
    assert attn[1:5] == ["10", "800.0", "790.0", "810.0"]

    # bytes: FETCH_SIZE mean 110000 KiB x 2, WRITE_SIZE mean 40000 KiB x 1
    rb, wb = 110000 * 1024 * 2.0, 40000 * 1024 * 1.0
    rows = [r for r in text.splitlines() if r.startswith("| attn_pp<128, 3> |")]
    hbm = [c.strip() for c in rows[1].strip("|").split("|")]
    assert hbm[1:3] == ["110000", "40000"]
    assert float(hbm[3]) == pytest.approx(rb / 2 ** 20, abs=0.05)
    assert float(hbm[4]) == pytest.approx(wb / 2 ** 20, abs=0.05)
    gbs = (rb + wb) / 800e-6 / 1e9
    assert float(hbm[5]) == pytest.approx(gbs, abs=0.5)
    assert float(hbm[6]) == pytest.approx(gbs / 8000.0, abs=5e-4)
    # algorithmic rate: 1000 GFLOP per launch over 800 us = 1250 TFLOP/s, 0.5 of 2500
    assert hbm[7] == "1250" and hbm[8] == "0.500"
    assert "attention traffic_bytes_per_launch: %d" % int(rb + wb) in text

    # executed MFMA flops: 512 per counted unit
    mf = [c.strip() for c in rows[2].strip("|").split("|")]
    assert mf[1] == "1024.0" and mf[2] == "1000.0"
    assert float(mf[3]) == pytest.approx(1024e9 / 800e-6 / 1e12, abs=0.5)
    est = [r for r in text.splitlines() if r.startswith("| est_gemm_bf16<")]
    assert [c.strip() for c in est[2].strip("|").split("|")][1] == "64.0"  # 0.125e9 x 512

    # LDS / MFMA busy cycles
    lds = [c.strip() for c in rows[3].strip("|").split("|")]
    assert lds[3] == "0.001"            # 5e4 conflict cycles of 1e8 LDS-active cycles (0.0005)
    assert float(lds[5]) == pytest.approx(1.3e6, rel=1e-3)   # shader clocks per XCD
    assert lds[6] == "1.62" or lds[6] == "1.63"              # 1.3e6 clocks over 800 us
    assert float(lds[7]) == pytest.approx(1.0e9 / (1024 * 1.3e6), abs=1e-3)
    assert [c.strip() for c in est[3].strip("|").split("|")][3] == "0.500"


def test_traffic_read_back_is_tied_to_the_attention_source(tmp_path):
    out = tmp_path / "profiles"
    out.mkdir()
    bench.summarize_profile(_profile_dir(tmp_path), WL, out_dir=str(out))
    assert bench.profiled_traffic(WL, profiles_dir=str(out)) == int(110000 * 1024 * 2.0 + 40000 * 1024)
    # a summary made from another attention source gives no traffic figure
    md = out / ("kernels_%s.md" % WL)
    text = md.read_text().replace("attention.hip %s" % bench.source_hash("attention.hip"),
                                  "attention.hip 0000000000000000")
    md.write_text(text)
    assert bench.profiled_traffic(WL, profiles_dir=str(out)) is None
    assert bench.profiled_traffic("no_such_workload", profiles_dir=str(out)) is None


def test_summary_without_counters_has_durations_only(tmp_path):
    out = tmp_path / "profiles"
    out.mkdir()
    bench.summarize_profile(_profile_dir(tmp_path, with_pmc=False), WL, out_dir=str(out))
    text = (out / ("kernels_%s.md" % WL)).read_text()
    assert "## Kernel durations" in text
    assert "## HBM traffic" not in text and "traffic_bytes_per_launch" not in text
    assert "## LDS and MFMA busy" not in text
    assert bench.profiled_traffic(WL, profiles_dir=str(out)) is None


def test_committed_profiles_match_their_workloads():
    """Every committed kernel summary names its own workload in each command
    and carries the source hashes it was made from."""
    pdir = os.path.join(ROOT, "profiles")
    names = [n for n in os.listdir(pdir) if n.startswith("kernels_") and n.endswith(".md")]
    assert names
    for n in names:
        wl = n[len("kernels_"):-len(".md")]
        text = open(os.path.join(pdir, n)).read()
        assert text.count("--workload %s" % wl) == len(bench.PROFILE_COMMANDS), n
        assert "source sha256[:16]: attention.hip " in text, n
