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
