"""bench.py's counter report on synthetic profiler databases (CPU only).

Each database holds rows of (dispatch, kernel, counter, value, duration) in the shape rocprofv3
writes: marker spins delimit the workload segments, in the driver's order, and a plain copy
(a multiply by one) calibrates the byte counters. The report's columns are checked against the
definitions it states: bytes scaled by the copy, percentages of the GPU cycles
(GRBM_GUI_ACTIVE over 8 XCDs) per SIMD (1024) or per CU (256), waits over wave cycles.
"""
import os
import sqlite3

import pytest

import bench

KERNEL = "void bfp::rowk::row_gemv_kernel<4, 2, true, 5, false, 1>(bfp::rowk::RowArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>, at::detail::Array<char*, 3> >(int, at::native::MulFunctor<float>, at::detail::Array<char*, 3>)"
SPIN = "void at::cuda::spin_kernel(long)"


def _db(path, counters):
    """One pass: a segment (two dispatches of KERNEL) between two markers, then the copy."""
    os.makedirs(path)
    con = sqlite3.connect(os.path.join(path, "run_results.db"))
    con.execute("create table counters_collection (dispatch_id int, kernel_name text, counter_name text, "
                "value real, duration int)")
    rows, did = [], 0

    def dispatch(name, vals, dur):
        nonlocal did
        did += 1
        for cn, v in vals.items():
            rows.append((did, name, cn, v, dur))

    marker = {c: 0.0 for c in counters}
    dispatch(SPIN, marker, 2000)
    dispatch(KERNEL, counters, 20_000)
    dispatch(KERNEL, counters, 22_000)
    dispatch(SPIN, marker, 2000)
    copy = {c: v for c, v in counters.items()}
    if "FETCH_SIZE" in copy:
        copy["FETCH_SIZE"] = bench.COPY_BYTES / 1024 / 2     # the counter reads half the bytes
    if "WRITE_SIZE" in copy:
        copy["WRITE_SIZE"] = bench.COPY_BYTES / 1024
    dispatch(COPY, copy, 100_000)
    con.executemany("insert into counters_collection values (?, ?, ?, ?, ?)", rows)
    con.commit()
    con.close()


def test_counter_report_columns(tmp_path, capsys):
    cyc = 2.4e9 * 20e-6 * 8                  # GRBM_GUI_ACTIVE: 20 us at 2.4 GHz, summed over 8 XCDs
    _db(str(tmp_path / "c1"), {"FETCH_SIZE": 50_000.0})
    _db(str(tmp_path / "c2"), {"WRITE_SIZE": 100.0})
    _db(str(tmp_path / "c3"), {"TCC_HIT_sum": 30.0, "TCC_MISS_sum": 70.0, "SQ_INSTS_VALU": 0.25 * 1024 * cyc / 8 / 4,
                               "GRBM_GUI_ACTIVE": cyc})
    _db(str(tmp_path / "c4"), {"SQ_VALU_MFMA_BUSY_CYCLES": 0.06 * 1024 * cyc / 8, "SQ_LDS_IDX_ACTIVE": 0.12 * 256 * cyc / 8,
                               "SQ_LDS_BANK_CONFLICT": 0.02 * 256 * cyc / 8, "SQ_WAIT_ANY": 390.0, "SQ_WAVE_CYCLES": 1000.0,
                               "TA_ADDR_STALLED_BY_TC_CYCLES": 256 * 1234.0, "GRBM_GUI_ACTIVE": cyc})
    bench.counter_report([str(tmp_path / f"c{i}") for i in range(1, 5)])
    out = capsys.readouterr().out
    row = [l for l in out.splitlines() if l.startswith("| dense BFP4 MLP M=1 |")]
    assert len(row) == 1, out
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "`rowk::row_gemv_kernel<4, 2, true, 5, false, 1>`"
    assert cells[2] == "2"                                   # dispatches
    assert cells[3] == "21.00"                               # mean duration, us
    assert cells[4] == f"{50_000 * 1024 * 2 / 1e6:.2f}"      # FETCH_SIZE x the copy's factor 2
    assert cells[5] == f"{100 * 1024 / 1e6:.3f}"             # WRITE_SIZE x 1
    assert cells[6:13] == ["30%", "25%", "6%", "12%", "2%", "39%", "1,234"]
    assert "FETCH_SIZE factor 2.0000, WRITE_SIZE factor 1.0000" in out


def test_marker_is_short_spin():
    assert bench.is_marker(SPIN, 2000)
    assert not bench.is_marker(SPIN, bench.MARKER_MAX_NS + 1)      # the longer spin ahead of a timed graph
    assert not bench.is_marker(KERNEL, 100)
