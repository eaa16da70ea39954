"""CPU: bench.py's measurement helpers.  Kernel names map to the families
the bench line and the profiles report; trace and counter summaries are
computed from small synthetic rocprofv3 CSV files whose answers are known;
the layer's compulsory bytes per token, with every read on a distinct row,
equal the worst-case figures of the hot-path scope table (Million 437 252,
Mid 120 324, Long 115 460 bytes per token)."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sparse_weight_memory_sub_amd.workloads import WORKLOADS  # noqa: E402

NS = "void fwpkm::(anonymous namespace)::"


@pytest.mark.parametrize("name,family", [
    (NS + "k_scatter<1, 8, 16>(fwpkm::ScatterArgs)", "scatter"),
    (NS + "k_fixup<1, 8>(fwpkm::ScatterArgs)", "scatter"),
    (NS + "k_gather<1, 8>(fwpkm::GatherArgs)", "gather"),
    (NS + "k_gather_split<1, 8>(fwpkm::GatherArgs)", "gather"),
    (NS + "k_sort_count<2>(fwpkm::SortArgs)", "sort"),
    (NS + "k_sort_scatter<8>(fwpkm::SortArgs)", "sort"),
    (NS + "k_score<1, 8, 3, 3, 16, false>(fwpkm::ScoreArgs)", "score_select"),
    (NS + "k_score<1, 8, 1, 4, 16, false>(fwpkm::ScoreArgs)", "score_rowstat"),
    (NS + "k_score<1, 8, 1, 2, 16, false>(fwpkm::ScoreArgs)", "score_stats"),
    (NS + "k_rows<1, 8, false>(fwpkm::ScoreArgs)", "score_select"),
    (NS + "k_row_m<1, false>(fwpkm::ScoreArgs)", "score_rowstat"),
    (NS + "k_row_colsum<false>(fwpkm::ScoreArgs)", "score_rowstat"),
    (NS + "k_select<1, false>(fwpkm::SelectArgs)", "select"),
    (NS + "k_select_rows(fwpkm::SelectArgs)", "select"),
    (NS + "k_select_ovf<1>(fwpkm::SelectArgs)", "select"),
    (NS + "k_kgrad<1, 8, false, true>(fwpkm::KgradArgs)", "kgrad"),
    (NS + "k_kgrad_finish<1, 8, false>(fwpkm::KgradArgs)", "kgrad"),
    (NS + "k_qt<1>(fwpkm::QtArgs)", "qt"),
    (NS + "k_knorm<1>(fwpkm::KnormArgs)", "knorm"),
    ("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>", None),
])
def test_kernel_family(name, family):
    assert bench.kernel_family(name) == family


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)


def _trace_row(name, start_ns, end_ns, queue):
    return {"Kernel_Name": NS + name + "(fwpkm::X)", "Start_Timestamp": start_ns, "End_Timestamp": end_ns,
            "Queue_Id": queue}


def test_summarize_trace_last_call(tmp_path, capsys):
    # two calls; the second has two chunks on two streams (times in ns)
    rows = [
        _trace_row("k_knorm<1>", 0, 500, 1),
        _trace_row("k_select_rows", 600, 900, 1),
        _trace_row("k_knorm<1>", 10_000, 10_100, 1),                 # the last call starts here
        _trace_row("k_rows<1, 8, false>", 10_100, 11_100, 1),
        _trace_row("k_select_rows", 11_100, 12_100, 1),
        _trace_row("k_sort_count<2>", 12_500, 13_000, 2),
        _trace_row("k_gather_split<1, 8>", 13_000, 14_000, 2),
        _trace_row("k_kgrad<1, 8, false, true>", 12_100, 14_100, 1),
        _trace_row("k_rows<1, 8, false>", 14_600, 15_600, 1),
        _trace_row("k_select_rows", 15_600, 16_600, 1),               # next chunk: 4.5 us after the first
        _trace_row("k_gather_split<1, 8>", 17_000, 18_000, 2),
    ]
    # an unrelated kernel of the input generation is left out
    rows.append({"Kernel_Name": "void at::native::normal_kernel", "Start_Timestamp": 9_000,
                 "End_Timestamp": 9_500, "Queue_Id": 1})
    _write_csv(tmp_path / "run_kernel_trace.csv", rows)
    bench.summarize_trace(str(tmp_path), last_call=True)
    out = capsys.readouterr().out
    # 9 library kernels from the last k_knorm on, spanning 10.0 .. 18.0 us
    assert "Last call: 9 kernels over 0.008 ms" in out
    # busy: [10.0, 14.1] and [14.6, 16.6] and [17.0, 18.0] -> 4.1 + 2.0 + 1.0 us
    assert "some kernel running for 0.007 ms" in out
    # stream 1: 6 kernels, 0.1+1+1+2+1+1 = 6.1 us of kernels, gaps 0 + 0 + 0 + 0.5 + 0 = 0.5 us
    assert "| 1 | 6 | 0.006 | 0.001 |" in out
    # stream 2: 3 kernels, 0.5+1+1 = 2.5 us, gaps 0 + 3.0 = 3.0 us
    assert "| 2 | 3 | 0.003 | 0.003 |" in out
    assert "mean 4.5 us, min 4.5, max 4.5" in out
    # the per-family table counts the last call only: 2 selections
    assert "Per chunk step (2 selections)" in out
    assert "| gather | 1.0 |" in out          # 2 us over 2 chunk steps


def test_summarize_trace_whole(tmp_path, capsys):
    rows = [_trace_row("k_select<1, false>", 0, 1000, 1), _trace_row("k_select<1, false>", 2000, 3000, 1),
            _trace_row("k_scatter<1, 8, 16>", 1000, 5000, 2), _trace_row("k_fixup<1, 8>", 5000, 6000, 2)]
    _write_csv(tmp_path / "run_kernel_trace.csv", rows)
    bench.summarize_trace(str(tmp_path))
    out = capsys.readouterr().out
    assert "| `k_scatter<1, 8, 16>` | 1 | 4000.0 | 4.00 |" not in out  # durations are in us
    assert "| `k_scatter<1, 8, 16>` | 1 | 4.0 | 0.00 |" in out
    assert "Per chunk step (2 selections)" in out
    assert "| scatter | 2.5 |" in out           # (4 + 1) us over 2 steps
    assert "Last call" not in out


def test_summarize_decode_calls(tmp_path, capsys):
    # four decode calls 10 us apart: scoring 3 us, selection and read 5 us;
    # the third call also runs a 20 us chunk write
    rows = []
    for c in range(4):
        t0 = 1_000 + c * 10_000
        rows.append(_trace_row("k_rows<1, 8, false>", t0, t0 + 3_000, 1))
        rows.append(_trace_row("k_select_gather<1, 8>", t0 + 3_000, t0 + 8_000, 1))
    rows.append(_trace_row("k_scatter<1, 8, 16>", 21_000 + 8_500, 21_000 + 28_500, 1))
    _write_csv(tmp_path / "run_kernel_trace.csv", rows)
    bench.summarize_decode_calls(str(tmp_path), 1, 2)  # calls 1 and 2
    out = capsys.readouterr().out
    # (3 + 5) * 2 + 20 = 36 us of kernels over 2 calls, starts 10 us apart
    assert "Calls 1 .. 2: 18.0 us of kernels per call, calls 10.0 us apart." in out
    assert "| `k_scatter<1, 8, 16>` | 1 | 20.00 | 10.00 |" in out
    assert "| `k_rows<1, 8, false>` | 2 | 3.00 | 3.00 |" in out
    with pytest.raises(SystemExit):
        bench.summarize_decode_calls(str(tmp_path), 2, 2)  # needs a fifth call's start


def _pmc_row(dispatch, name, counter, value):
    return {"Dispatch_Id": dispatch, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value}


def test_summarize_pmc_scales(tmp_path, capsys):
    # calibration: torch.neg over 1 GiB reads FETCH 512 Ki KiB (scale 2) and writes 1 Gi (scale 1)
    neg = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>"
    fetch = [_pmc_row(1, neg, "FETCH_SIZE", 1 << 19)]
    write = [_pmc_row(1, neg, "WRITE_SIZE", 1 << 20)]
    d = 2
    for step in range(2):
        for name, f_kib, w_kib in (("k_select<1, false>", 100, 10), ("k_sort_count<8>", 30, 0),
                                   ("k_sort_scatter<8>", 50, 40)):
            fetch.append(_pmc_row(d, NS + name + "(x)", "FETCH_SIZE", f_kib))
            write.append(_pmc_row(d, NS + name + "(x)", "WRITE_SIZE", w_kib))
            d += 1
    os.makedirs(tmp_path / "f")
    os.makedirs(tmp_path / "w")
    _write_csv(tmp_path / "f" / "run_counter_collection.csv", fetch)
    _write_csv(tmp_path / "w" / "run_counter_collection.csv", write)
    # only families without committed per-kernel files, so nothing is written under profiles/
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "synthetic")
    out = capsys.readouterr().out
    assert "fetch scale 2.0000, write scale 1.0000; 2 chunk steps" in out
    # select: (100 * 2 + 10 * 1) KiB = 210 KiB = 0.2 MB per step
    assert "| select | 100 | 10 | 0.2 MB |" in out
    # sort: count + scatter, (80 * 2 + 40) KiB = 200 KiB
    assert "| sort | 80 | 40 | 0.2 MB |" in out


def test_summarize_mfma(tmp_path, capsys):
    # two dispatches of a 10 us sweep, each executing 2^30 bf16 MFMA flops
    # (2^21 MOPS of 512): 107.4 TFLOP/s, 4.3% of 2500; GRBM_GUI_ACTIVE of
    # 8 XCDs x 24000 cycles, MFMA busy 6144000 cycles = 25% of 24000 x 1024 SIMDs
    rows = []
    for d in (1, 2):
        base = {"Kernel_Name": NS + "k_score<1, 8, 3, 3, 16, 1, false>(fwpkm::ScoreArgs)",
                "Start_Timestamp": 1_000_000 * d, "End_Timestamp": 1_000_000 * d + 10_000}
        for counter, value in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1 << 21), ("SQ_INSTS_VALU_MFMA_MOPS_F32", 0),
                               ("SQ_VALU_MFMA_BUSY_CYCLES", 6_144_000), ("GRBM_GUI_ACTIVE", 8 * 24_000)):
            rows.append({**_pmc_row(d, base["Kernel_Name"], counter, value), **base})
        # a kernel outside the MFMA families is left out
        rows.append({**base, **_pmc_row(10 + d, NS + "k_gather<1, 8>(fwpkm::GatherArgs)", "GRBM_GUI_ACTIVE", 8)})
    _write_csv(tmp_path / "run_counter_collection.csv", rows)
    bench.summarize_mfma(str(tmp_path))
    out = capsys.readouterr().out
    assert "| `k_score<1, 8, 3, 3, 16, 1, false>` | 2 | 10.0 | 1.07 | 107 | 4.3 | 25.0 |" in out
    assert "k_gather" not in out


@pytest.mark.parametrize("name,worst", [("million", 437_252), ("mid", 120_324), ("long", 115_460)])
def test_layer_bytes_worst_case(name, worst):
    cfg = WORKLOADS[name].cfg
    U = cfg.chunk * cfg.heads * cfg.k  # every read of a chunk on a distinct row
    assert bench.layer_bytes_per_token(cfg, U) == pytest.approx(worst, abs=0.5)


def test_layer_bytes_reuse_lowers_the_write():
    cfg = WORKLOADS["million"].cfg
    full = bench.layer_bytes_per_token(cfg, cfg.chunk * cfg.heads * cfg.k)
    half = bench.layer_bytes_per_token(cfg, cfg.chunk * cfg.heads * cfg.k // 2)
    # half as many rows written: the read-modify-write term halves, nothing else moves
    rmw = 2 * cfg.chunk * cfg.heads * cfg.k * cfg.d_v * 2 / cfg.chunk
    assert full - half == pytest.approx(rmw / 2)
