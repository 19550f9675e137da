"""The rocprofv3 summary's split of a sweep into cases (host logic, synthetic CSV)."""
import csv
import json

import pytest

from ternary_weight_decode_amd import rocprof_summary as rs

FIELDS = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Start_Timestamp", "End_Timestamp",
          "Arch_VGPR_Count"]


def _write(tmp_path, dispatches, rows):
    d = tmp_path / "prof" / "host"
    d.mkdir(parents=True)
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        t = 0
        for i, (name, grid, ns) in enumerate(dispatches):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Grid_Size": grid, "Workgroup_Size": 512,
                        "Start_Timestamp": t, "End_Timestamp": t + ns, "Arch_VGPR_Count": 32})
            t += ns + 100
    out = tmp_path / "bench.out"
    out.write_text("noise\n" + json.dumps({"mode": "x", "rows": rows}) + "\n")
    return str(tmp_path / "prof"), str(out)


def test_runs_split_label_and_drop_first_pass(tmp_path, capsys):
    a, b, q = "void tern::gemv_a<1>(int)", "void tern::gemv_b<true>(int)", "void quant(int)"
    # case 1: 2 copies x 3 passes of kernel a; a quantize launch between; case 2: kernel b
    # run as two launches per call (x2), same grid
    disp = [(a, 512 * 4, 9000)] * 2 + [(a, 512 * 4, 3000)] * 4 + [(q, 512, 50)] + \
           [(b, 512 * 4, 1000), (b, 512 * 4, 2000)] * 6
    rows = [{"proj": "q", "M": 1, "act": "bf16"}, {"proj": "q", "M": 1, "act": "int8"}]
    d, out = _write(tmp_path, disp, rows)
    rs.main(["runs", d, "--bench", out, "--kernel", "gemv", "--passes", "3"])
    lines = capsys.readouterr().out.strip().splitlines()
    assert len(lines) == 2
    assert "gemv_a" in lines[0] and "median_us=   3.00" in lines[0] and "M= 1" in lines[0]
    assert "gemv_b x2" in lines[1] and "median_us=   3.00" in lines[1]


def test_runs_mismatch_exits(tmp_path):
    d, out = _write(tmp_path, [("void k1(int)", 512, 10), ("void k2(int)", 512, 10)], [{"proj": "q"}])
    with pytest.raises(SystemExit):
        rs.main(["runs", d, "--bench", out])


def test_runs_counters_scaled_against_row_bytes(tmp_path, capsys):
    d = tmp_path / "pmc" / "host"
    d.mkdir(parents=True)
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                               "Counter_Value"])
        w.writeheader()
        for i in range(4):
            # one counter reported per XCD-like instance: the rows of a dispatch add up
            for part in (600.0, 400.0):
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": "void tern::gemv_a<1>(int)", "Grid_Size": 2048,
                            "Workgroup_Size": 512, "Counter_Name": "FETCH_SIZE", "Counter_Value": part})
    out = tmp_path / "bench.out"
    out.write_text(json.dumps({"rows": [{"unit": "qkv", "format": "fv5", "act": "bf16", "M": 4,
                                         "bytes": 2048000}]}) + "\n")
    rs.main(["runs", str(tmp_path / "pmc"), "--bench", str(out), "--passes", "2", "--scale", "FETCH_SIZE=2.0"])
    line = capsys.readouterr().out.strip()
    # 1000 KiB x 1024 x 2.0 = 2.048 MB measured against 2.048 MB algorithmic
    assert "FETCH_SIZE     1000.0 KiB" in line and "ratio 1.000" in line and "fv5" in line


def test_runs_merges_counter_directories(tmp_path, capsys):
    for cn, val in (("FETCH_SIZE", 1500.0), ("WRITE_SIZE", 500.0)):
        d = tmp_path / cn / "host"
        d.mkdir(parents=True)
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                                   "Counter_Value"])
            w.writeheader()
            for i in range(2):
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": "void gemv_a(int)", "Grid_Size": 512,
                            "Workgroup_Size": 512, "Counter_Name": cn, "Counter_Value": val})
    out = tmp_path / "bench.out"
    out.write_text(json.dumps({"rows": [{"proj": "o", "act": "int8", "M": 1, "bytes": 2048000}]}) + "\n")
    rs.main(["runs", str(tmp_path / "FETCH_SIZE"), str(tmp_path / "WRITE_SIZE"), "--bench", str(out),
             "--passes", "2", "--scale", "FETCH_SIZE=1.0", "--scale", "WRITE_SIZE=1.0"])
    line = capsys.readouterr().out
    assert "FETCH_SIZE     1500.0 KiB" in line and "WRITE_SIZE      500.0 KiB" in line and "ratio 1.000" in line


def test_runs_sq_counters_per_wave(tmp_path, capsys):
    d = tmp_path / "sq" / "host"
    d.mkdir(parents=True)
    vals = {"SQ_WAVES": 8.0, "SQ_INSTS_VALU": 800.0, "SQ_INSTS_MFMA": 160.0, "SQ_WAIT_INST_ANY": 250.0,
            "SQ_WAVE_CYCLES": 1000.0, "SQ_BUSY_CYCLES": 100.0, "SQ_VALU_MFMA_BUSY_CYCLES": 80.0}
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name",
                               "Counter_Value"])
        w.writeheader()
        for i in range(2):
            for cn, v in vals.items():
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": "void gemv_a(int)", "Grid_Size": 512,
                            "Workgroup_Size": 512, "Counter_Name": cn, "Counter_Value": v})
    with open(d / "run_agent_info.csv", "w", newline="") as f:
        w = csv.DictWriter(f, ["Name", "Simd_Count", "Num_Shader_Banks"])
        w.writeheader()
        w.writerow({"Name": "AMD EPYC", "Simd_Count": 0, "Num_Shader_Banks": 0})
        w.writerow({"Name": "gfx950", "Simd_Count": 8, "Num_Shader_Banks": 2})
    out = tmp_path / "bench.out"
    out.write_text(json.dumps({"rows": [{"proj": "q", "act": "bf16", "M": 8}]}) + "\n")
    rs.main(["runs", str(tmp_path / "sq"), "--bench", str(out), "--passes", "2"])
    line = capsys.readouterr().out
    assert "valu/wave   100.0" in line and "mfma/wave    20.0" in line
    # busy 100 cycles summed over 2 engines of 4 SIMDs: 400 SIMD-cycles; 80 MFMA cycles, 800 VALU x 4
    assert "wait  25.0%" in line and "mfma busy  20.0%" in line and "valu issue 800.0%" in line
