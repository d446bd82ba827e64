"""Host logic of the measurement code (no GPU): the benchmark's FLOP and byte
counts, its command-line contract, and the rocprofv3 summariser."""
import csv
import importlib.util
import os
import subprocess
import sys

import numpy as np

from sparse_attention_diffusion_amd import profsum

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_kept_flops_and_bytes_by_hand():
    bench = _bench()
    # one head, N = 150 (blocks of 64, 64, 22), keep 2
    idx = np.array([[[[0, 2], [1, 2], [0, 1]]]], dtype=np.int32)
    d, D, N = 64, 64, 150
    # rows x kept keys per query block: 64*(64+22) + 64*(64+22) + 22*(64+64)
    assert bench.kept_flops(idx, N, d) == 4 * d * (64 * 86 + 64 * 86 + 22 * 128)
    # Q, O (bf16), R (f32), m/Z_full/Z_sparse (f32) per row, K and V of blocks {0,1,2} once, the lists
    rows = N
    want = rows * D * 2 * 2 + rows * D * 4 + rows * 12 + 150 * D * 2 * 2 + idx.size * 4
    assert bench.sparse_call_bytes(idx, N, D, 2) == want


def test_oracle_full_timing_tiny():
    bench = _bench()
    r = bench.oracle_full_timing("tiny")
    assert r["config"] == "tiny" and r["dtype"] == "f32" and r["heads"] == 2
    assert r["calibrate_layers"] == [0] and len(r["calibrate_s"]) == 1
    assert r["sparse_step_s"] > 0 and r["sparse_kept_tflops"] > 0 and r["calibrate_dense_tflops"] > 0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_profile_summary_from_csv(tmp_path):
    trace = tmp_path / "trace"
    trace.mkdir()
    _write_csv(trace / "run_kernel_stats.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "MinNs", "MaxNs"], [
        ["void rettn::(anonymous namespace)::sparse_occ_kernel<64, false, false>(rettn::AttnArgs)", 10, 3e6, 3e5,
         2.9e5, 3.1e5],
        ["void rettn::(anonymous namespace)::calib_kernel<64, 2, 2, false>(rettn::AttnArgs)", 1, 6e6, 6e6, 6e6, 6e6],
        ["some_other_kernel", 3, 1e3, 3e2, 2e2, 4e2],
    ])
    stats = {s["kernel"]: s for s in profsum.trace_stats(str(trace))}
    assert set(stats) == {"sparse reshape R1 (d_pad 64)", "calibration (d_pad 64)"}
    assert stats["sparse reshape R1 (d_pad 64)"]["avg_us"] == 300.0
    assert stats["calibration (d_pad 64)"]["total_ms"] == 6.0
    # counters: a 512 MiB copy read back as 262144 KiB means a fetch scale of 2
    pmc = tmp_path / "pmc"
    pmc.mkdir()
    _write_csv(pmc / "run_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"], [
        ["copyBuffer", "FETCH_SIZE", 262144.0],
        ["sparse_occ_kernel<64, false, false>", "FETCH_SIZE", 500000.0],
        ["sparse_occ_kernel<64, false, false>", "FETCH_SIZE", 700000.0],
    ])
    scale, per, raw = profsum.counters(str(pmc), "FETCH_SIZE")
    assert raw == 262144.0 and abs(scale - 2.0) < 1e-12
    assert abs(per["sparse reshape R1 (d_pad 64)"] - 600000.0 * 1024 * 2) < 1e-3
    # every kernel of the library has a label, and the bf16/R2 variants are not merged with R1
    names = ["sparse_occ_kernel<64, true, false>", "sparse_occ_kernel<64, false, true>",
             "sparse_occ_kernel<80, true, true>", "calib_kernel<80, 2, 2, true>", "pool_k_kernel<__bf16, 64>",
             "select_kernel<__bf16, 64, 5, 4>", "attn_f32_kernel<64, 1>", "permute_kernel"]
    labels = [profsum.short_name(n) for n in names]
    assert None not in labels and len(set(labels)) == len(labels)


def test_unit_utilisation_summary(tmp_path):
    """GRBM_GUI_ACTIVE is summed over 8 XCDs: 8000 cycles means 1000 per XCD, so
    512000 MFMA-busy cycles over 1024 SIMDs is 50%, and 64000 TA-busy cycles over
    256 CUs is 25%; a read latency sum of 2560000 cycles over 1000 cycles and 256
    CUs is 10 reads in flight per CU."""
    d1, d2 = tmp_path / "u1", tmp_path / "u2"
    d1.mkdir()
    d2.mkdir()
    k = "sparse_occ_kernel<64, false, false>"
    _write_csv(d1 / "run_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"], [
        [k, "GRBM_GUI_ACTIVE", 8000], [k, "SQ_VALU_MFMA_BUSY_CYCLES", 512000], [k, "SQ_ACTIVE_INST_VALU", 64000],
        [k, "SQ_VALU_MFMA_COEXEC_CYCLES", 102400]])
    _write_csv(d2 / "run_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"], [
        [k, "GRBM_GUI_ACTIVE", 8000], [k, "TA_TA_BUSY_sum", 64000], [k, "TD_TD_BUSY_sum", 128000],
        [k, "TCP_TCC_READ_REQ_sum", 5000], [k, "TCP_TCC_READ_REQ_LATENCY_sum", 2560000],
        [k, "TCP_PENDING_STALL_CYCLES_sum", 25600]])
    rows = profsum.unit_table(profsum.unit_counters([str(d1), str(d2)]))
    cells = [x.strip() for x in rows[-1].split("|")[1:-1]]
    assert cells == ["sparse reshape R1 (d_pad 64)", "50%", "25%", "10%", "25%", "50%", "10%", "0.0 M", "512", "10"]
    # wave states are fractions of SQ_WAVE_CYCLES; the instruction mix is per MFMA instruction
    d3, d4 = tmp_path / "u3", tmp_path / "u4"
    d3.mkdir()
    d4.mkdir()
    _write_csv(d3 / "run_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"], [
        [k, "GRBM_GUI_ACTIVE", 8000], [k, "SQ_WAVE_CYCLES", 1000], [k, "SQ_WAIT_ANY", 360],
        [k, "SQ_WAIT_INST_ANY", 400], [k, "SQ_ACTIVE_INST_ANY", 230]])
    _write_csv(d4 / "run_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"], [
        [k, "GRBM_GUI_ACTIVE", 8000], [k, "SQ_INSTS_MFMA", 100], [k, "SQ_INSTS_VALU", 1030],
        [k, "SQ_INSTS_LDS", 160], [k, "SQ_INSTS_SALU", 450], [k, "SQ_INSTS_VMEM", 60]])
    rows = profsum.unit_table(profsum.unit_counters([str(d1), str(d2), str(d3), str(d4)]))
    cells = [x.strip() for x in rows[-1].split("|")[1:-1]]
    assert cells == ["sparse reshape R1 (d_pad 64)", "36%", "40%", "23%", "10.3", "1.6", "4.5", "0.6"]
