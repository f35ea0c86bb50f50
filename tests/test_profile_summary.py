"""Host logic of the rocprofv3 summariser: label matching, grouping and copy calibration."""
import csv

import pytest

from skinny_gemm_nvfp4_amd import profile_summary as ps

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id",
              "Kernel_Id", "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp",
              "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
              "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X",
              "Grid_Size_Y", "Grid_Size_Z"]
PMC_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]
GEMM = "void nvfp4::gemv_stream_kernel<1, 16, 4, true, false>(nvfp4::GemmArgs, nvfp4::Lay)"
PACK = "void nvfp4::pack_quant_kernel(int, int, float const*)"


def _trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, TRACE_COLS)
        w.writeheader()
        for i, (name, start, ns) in enumerate(rows):
            w.writerow({**{c: 0 for c in TRACE_COLS}, "Dispatch_Id": i + 1, "Kernel_Name": name,
                        "Start_Timestamp": start, "End_Timestamp": start + ns,
                        "Grid_Size_X": 256, "Grid_Size_Y": 1, "Workgroup_Size_X": 1024})


def _pmc(path, rows, counter):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, PMC_COLS)
        w.writeheader()
        for i, (name, values) in enumerate(rows):
            for v in values:   # several rows per dispatch are summed
                w.writerow({**{c: 0 for c in PMC_COLS}, "Dispatch_Id": i + 1,
                            "Kernel_Name": name, "Grid_Size": 256, "Counter_Name": counter,
                            "Counter_Value": v})


def test_trace_groups_by_label(tmp_path):
    # out-of-order rows are sorted by start time; pack kernels are not GEMMs
    _trace(tmp_path / "t.csv", [(GEMM, 300, 4000), (PACK, 50, 10), (GEMM, 100, 2000),
                                (GEMM, 200, 3000)])
    (tmp_path / "l.txt").write_text("a M=1 N=16 K=64\nb M=1 N=16 K=64\na M=1 N=16 K=64\n")
    out = ps.trace_summary(str(tmp_path / "t.csv"), str(tmp_path / "l.txt"))
    lines = out.splitlines()
    assert len(lines) == 3
    assert lines[1].startswith("a M=1") and " 2 " in lines[1]
    # a = dispatches starting at 100 and 300: mean (2 + 4) / 2 us
    assert "    3.00" in lines[1] and "    3.00" in lines[2]


def test_label_count_mismatch_is_an_error(tmp_path):
    _trace(tmp_path / "t.csv", [(GEMM, 100, 2000)])
    (tmp_path / "l.txt").write_text("a\nb\n")
    with pytest.raises(ValueError):
        ps.trace_summary(str(tmp_path / "t.csv"), str(tmp_path / "l.txt"))


def test_traffic_is_scaled_by_the_calibration_copy(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    nbytes = 1 << 20
    # the counter sees half of every byte: 512 KiB for the 1 MiB copy (a small copy is ignored)
    _pmc(tmp_path / "f.csv", [(copy, [1.0]), (copy, [256.0, 256.0]), (GEMM, [100.0]),
                              (GEMM, [300.0]), (GEMM, [200.0])], "FETCH_SIZE")
    _pmc(tmp_path / "w.csv", [(copy, [128.0]), (GEMM, [1.0]), (GEMM, [1.0]), (GEMM, [1.0])],
         "WRITE_SIZE")
    (tmp_path / "l.txt").write_text("g M=1 N=16 K=64\n" * 3)
    kf, kw, rows = ps.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                      str(tmp_path / "l.txt"), nbytes)
    assert kf == pytest.approx(2.0) and kw == pytest.approx(8.0)
    r = rows["g M=1 N=16 K=64"]
    assert r["fetch_bytes"] == 200 * 1024 * 2       # median of 100, 300, 200 KiB, x2
    assert r["write_bytes"] == 1 * 1024 * 8
    assert r["bytes_per_launch"] == r["fetch_bytes"] + r["write_bytes"]


BATCH = "void nvfp4::mfma_slab_kernel<8, 4, 1, 0>(nvfp4::GemmArgs, nvfp4::SlabLayout)"
FINALIZE = ("nvfp4::argmax_finalize_kernel(unsigned long long const*, int, int*, float*)")


def test_follow_on_counters_are_summed(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    _pmc(tmp_path / "f.csv", [(copy, [512.0]), (BATCH, [100.0]), (FINALIZE, [50.0])], "FETCH_SIZE")
    _pmc(tmp_path / "w.csv", [(copy, [1024.0]), (BATCH, [10.0]), (FINALIZE, [5.0])], "WRITE_SIZE")
    (tmp_path / "l.txt").write_text("s M=128 N=16 K=64\n")
    _, _, rows = ps.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                    str(tmp_path / "l.txt"), 1 << 20)
    assert rows["s M=128 N=16 K=64"]["fetch_bytes"] == 150 * 1024 * 2
    assert rows["s M=128 N=16 K=64"]["write_bytes"] == 15 * 1024


def test_follow_on_without_a_gemm_is_an_error(tmp_path):
    _trace(tmp_path / "t.csv", [(FINALIZE, 100, 500)])
    (tmp_path / "l.txt").write_text("s\n")
    with pytest.raises(ValueError):
        ps.trace_summary(str(tmp_path / "t.csv"), str(tmp_path / "l.txt"))


def test_mfma_busy_fraction(tmp_path):
    # 1000 MFMAs of 16 busy cycles on one SIMD's share: busy = 16000 over 1024 SIMDs of a
    # dispatch active for 8 XCDs x 100 cycles -> 16000 / (1024 * 100) = 15.6 %
    with open(tmp_path / "c.csv", "w", newline="") as f:
        w = csv.DictWriter(f, PMC_COLS)
        w.writeheader()
        for name, value in (("SQ_INSTS_MFMA", 1000.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 16000.0),
                            ("GRBM_GUI_ACTIVE", 800.0)):
            w.writerow({**{c: 0 for c in PMC_COLS}, "Dispatch_Id": 1, "Kernel_Name": BATCH,
                        "Grid_Size": 256, "Counter_Name": name, "Counter_Value": value})
    (tmp_path / "l.txt").write_text("m M=128 N=16 K=64\n")
    lines = ps.mfma_summary(str(tmp_path / "c.csv"), str(tmp_path / "l.txt")).splitlines()
    assert lines[1].startswith("m M=128") and lines[1].rstrip().endswith("15.6")


def test_argmax_follow_on_dispatches_are_folded(tmp_path):
    # greedy-token call: GEMM 0..1000 then finalize 1100..1300 (1.3 us); a 128-row greedy-token
    # call: slab kernel 2000..4000, finalize 4500..4600 (2.6 us); a plain GEMM
    _trace(tmp_path / "t.csv", [(GEMM, 0, 1000), (FINALIZE, 1100, 200), (BATCH, 2000, 2000),
                                (FINALIZE, 4500, 100), (GEMM, 6000, 1000)])
    (tmp_path / "l.txt").write_text("a M=1 N=16 K=64\nb M=128 N=16 K=64\np M=1 N=16 K=64\n")
    lines = ps.trace_summary(str(tmp_path / "t.csv"), str(tmp_path / "l.txt")).splitlines()
    assert len(lines) == 4
    assert "+argmax" in lines[1] and "    1.30" in lines[1]
    assert "+argmax" in lines[2] and "    2.60" in lines[2]
    assert "+argmax" not in lines[3] and "    1.00" in lines[3]


def test_calibration_is_the_first_copy_of_its_size(tmp_path):
    copy = "__amd_rocclr_copyBuffer"
    # calibration 512 KiB counted for 1 MiB; a later, larger clone of weights must not be taken
    _pmc(tmp_path / "f.csv", [(copy, [512.0]), (GEMM, [100.0]), (copy, [4096.0])], "FETCH_SIZE")
    _pmc(tmp_path / "w.csv", [(copy, [1024.0]), (GEMM, [1.0]), (copy, [8192.0])], "WRITE_SIZE")
    (tmp_path / "l.txt").write_text("g M=1 N=16 K=64\n")
    kf, kw, _ = ps.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                   str(tmp_path / "l.txt"), 1 << 20)
    assert kf == pytest.approx(2.0) and kw == pytest.approx(1.0)


NORM = "nvfp4::rmsnorm_rows_kernel(unsigned short const*, unsigned short const*, float, int, unsigned short*)"


def test_fused_lead_dispatch_is_folded(tmp_path):
    # fused call above the dot-product rows: RMSNorm 0..500, slab GEMM (SiLU * up epilogue)
    # 600..2600 (2.6 us); then a plain GEMM
    _trace(tmp_path / "t.csv", [(NORM, 0, 500), (BATCH, 600, 2000), (GEMM, 5000, 1000)])
    (tmp_path / "l.txt").write_text("f M=128 N=16 K=64\np M=1 N=16 K=64\n")
    lines = ps.trace_summary(str(tmp_path / "t.csv"), str(tmp_path / "l.txt")).splitlines()
    assert len(lines) == 3
    assert "+norm" in lines[1] and "    2.60" in lines[1]
    assert "+norm" not in lines[2] and "    1.00" in lines[2]
