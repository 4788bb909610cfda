"""Host logic of the rocprofv3 summaries (hpc_linear_algebra_amd/profiling.py)
on small synthetic CSV files: kernel-name shortening, per-grid trace
statistics, and HBM traffic scaled by a plain copy's counter reading."""
import csv
import math
import os

from hpc_linear_algebra_amd import profiling as P


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_short_names():
    assert P._short("void tlr::(anonymous namespace)::grouped_gemm_kernel<double, 3, 1, 8>(tlr::DevTask const*)") \
        == "grouped_gemm_kernel<double, 3, 1, 8>"
    assert P._short("_ZN3tlr12_GLOBAL__N_121grouped_gemm16_kernelIDF16_Li3ELi4EEEvPKNS_7DevTaskE") \
        == "grouped_gemm16_kernel<half, 3, 4>"
    assert P._short("_ZN3tlr12_GLOBAL__N_121grouped_gemm16_kernelIDF16bLi2ELi2EEEvPKNS_7DevTaskE") \
        == "grouped_gemm16_kernel<bfloat16, 2, 2>"
    assert P._short("_ZN3tlr12_GLOBAL__N_118wide_gemm16_kernelIDF16_EEvPKNS_7DevTaskEPKNS_7DevTileE") \
        == "wide_gemm16_kernel<half>"
    assert P._short("_ZN3tlr12_GLOBAL__N_118wide_gemm16_kernelIDF16_Li3EEEvPKNS_7DevTaskEPKNS_7DevTileE") \
        == "wide_gemm16_kernel<half, 3>"
    assert P._short("_ZN3tlr12_GLOBAL__N_119strip_gemm16_kernelIDF16bEEvPKNS_7DevTaskEPKNS_7DevTileE") \
        == "strip_gemm16_kernel<bfloat16>"
    assert P._short("_ZN3tlr12_GLOBAL__N_119grouped_gemm_kernelIfLi1ELi0ELi4EEEvPK") \
        == "grouped_gemm_kernel<float, 1, 0, 4>"
    assert P._short("_ZN3tlr12_GLOBAL__N_117strip_gemm_kernelIdLi1EEEvPKNS_7DevTaskEPKNS_7DevTileEPKlNS_5BasesE") \
        == "strip_gemm_kernel<double, 1>"


def test_trace_stats_groups_by_kernel_and_grid(tmp_path):
    name = "void tlr::(anonymous namespace)::grouped_gemm_kernel<double, 3, 1, 8>(x)"
    rows = []
    # three launches of 16384 workgroups lasting 10, 12 and 20 us; one of 64 lasting 4 us
    for dur, grid in ((10, 16384), (12, 16384), (20, 16384), (4, 64)):
        rows.append([name, grid * 256, 256, 1000, 1000 + dur * 1000])
    _write(str(tmp_path / "d" / "run_kernel_trace.csv"),
           ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"], rows)
    out = P.stats([str(tmp_path / "d")], "cmd")
    lines = [l for l in out.splitlines() if l.startswith("| grouped")]
    assert len(lines) == 2
    big = [l for l in lines if "| 16384 |" in l][0].split("|")
    # kernel, workgroups, calls, total ms, avg, median, min, max, %
    assert big[3].strip() == "3"
    assert math.isclose(float(big[4]), 0.042, abs_tol=1e-3)
    assert math.isclose(float(big[5]), 14.0, abs_tol=0.05)
    assert math.isclose(float(big[6]), 12.0, abs_tol=0.05)
    assert math.isclose(float(big[7]), 10.0, abs_tol=0.05) and math.isclose(float(big[8]), 20.0, abs_tol=0.05)
    assert out.startswith("Command: `cmd`")


def test_traffic_scales_by_the_copy(tmp_path):
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "void tlr::(anonymous namespace)::grouped_gemm_kernel<double, 3, 1, 8>(x)"
    # the copy of 1 GiB reads FETCH_SIZE 0.5 GiB and WRITE_SIZE 1 GiB (in KiB)
    _write(str(tmp_path / "cf" / "run_counter_collection.csv"), hdr, [["copyBuffer", "FETCH_SIZE", 524288.0]])
    _write(str(tmp_path / "cw" / "run_counter_collection.csv"), hdr, [["copyBuffer", "WRITE_SIZE", 1048576.0]])
    _write(str(tmp_path / "f" / "run_counter_collection.csv"), hdr,
           [[k, "FETCH_SIZE", 1000.0], [k, "FETCH_SIZE", 3000.0], ["other", "FETCH_SIZE", 7.0]])
    _write(str(tmp_path / "w" / "run_counter_collection.csv"), hdr, [[k, "WRITE_SIZE", 500.0]])
    t = P.traffic(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "cf"), str(tmp_path / "cw"),
                  r"grouped_gemm_kernel<double, 3")
    assert math.isclose(t["fetch_scale"], 2.0) and math.isclose(t["write_scale"], 1.0)
    assert math.isclose(t["read_bytes"], 2000.0 * 1024 * 2.0)      # mean of the two dispatches, scaled
    assert math.isclose(t["write_bytes"], 500.0 * 1024)
    assert math.isclose(t["bytes_per_launch"], t["read_bytes"] + t["write_bytes"])
    assert t["kernel_hash"] == P.kernel_source_hash(False)


def test_mfma_busy_fraction(tmp_path):
    """Busy fraction = MFMA busy cycles summed over the 1024 SIMDs over (1024 x
    one XCD's active cycles); GRBM_GUI_ACTIVE reads as the sum over 8 XCDs."""
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    k = "void tlr::(anonymous namespace)::grouped_gemm_kernel<double, 3, 1, 8>(x)"
    # 8e6 active cycles per XCD; every SIMD busy 6e6 of them -> 0.75
    _write(str(tmp_path / "p" / "run_counter_collection.csv"), hdr,
           [[k, "GRBM_GUI_ACTIVE", 8 * 8e6], [k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 6e6],
            ["other", "SQ_VALU_MFMA_BUSY_CYCLES", 1.0]])
    m = P.mfma_busy(str(tmp_path / "p"), r"grouped_gemm_kernel<double, 3")
    assert math.isclose(m["mfma_busy"], 0.75)
    assert m["kernel_hash"] == P.kernel_source_hash(False)
