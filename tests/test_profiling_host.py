"""Host checks of the rocprofv3 summary helpers (synthetic CSVs, no GPU)."""

import csv

from blockwise_fp8_linear_quant_amd import profiling

GEMM = ("void fp8blk::(anonymous namespace)::block_gemm_f16_kernel<256, 128, 64, 64, 0, 1, 8, 3>"
        "(unsigned char const*, long, float const*, long)")
KGROUPS = ("void fp8blk::(anonymous namespace)::block_gemm_f16_kgroups_kernel<1, 2>"
           "(unsigned char const*, long, float const*, long)")
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>>(int, float*)"


def test_short_name_keeps_template_arguments():
    assert profiling.short_name(GEMM) == "block_gemm_f16_kernel<256, 128, 64, 64, 0, 1, 8, 3>"
    q = "fp8blk::(anonymous namespace)::quant_rows_kernel(unsigned short const*, long)"
    assert profiling.short_name(q) == "quant_rows_kernel"


def _counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, name, v in rows:
            w.writerow([d, name, counter, v])


def test_traffic_scales_by_the_copy_probe(tmp_path):
    copy_bytes = 1 << 30
    # counters read half the true bytes for the copy, so the scale is 2048 B per unit
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # both exact-path kernels count as GEMM launches
    _counters(fetch, "FETCH_SIZE", [(1, COPY, 524288.0), (2, GEMM, 1000.0), (3, KGROUPS, 3000.0)])
    _counters(write, "WRITE_SIZE", [(1, COPY, 1048576.0), (2, GEMM, 10.0), (3, KGROUPS, 30.0)])
    text = profiling.traffic_summary(str(fetch), str(write), copy_bytes, "cmd", 4096.0 * 1000)
    kv = dict(line.split(": ", 1) for line in text.strip().splitlines())
    assert float(kv["fetch_scale_bytes_per_kib"]) == 2048.0
    assert float(kv["write_scale_bytes_per_kib"]) == 1024.0
    assert int(kv["gemm_fetch_bytes_per_launch"]) == 2000 * 2048
    assert int(kv["gemm_write_bytes_per_launch"]) == 20 * 1024
    assert int(kv["gemm_dispatches"]) == 2
    assert kv["source_sha256"] == profiling.source_digest()


def test_read_traffic_rejects_another_source(tmp_path):
    p = tmp_path / "t.txt"
    p.write_text("source_sha256: 0000\ngemm_hbm_bytes_per_launch: 5\n")
    assert profiling.read_traffic(str(p)) is None
    p.write_text(f"source_sha256: {profiling.source_digest()}\ngemm_hbm_bytes_per_launch: 5\n")
    assert profiling.read_traffic(str(p))["gemm_hbm_bytes_per_launch"] == "5"
    assert profiling.read_traffic(str(tmp_path / "missing.txt")) is None


def test_stats_summary_sets_rocprof_beside_the_bench_figure(tmp_path):
    stats = tmp_path / "s.csv"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writerow([GEMM, 11, 1150000, 104545, 76.0])
        w.writerow([KGROUPS, 1, 50000, 50000, 4.0])
        w.writerow([COPY, 4, 300000, 75000, 20.0])
    bench = tmp_path / "b.json"
    bench.write_text('noise\n{"roofline": {"avg_launch_us": 125.0, "launches_per_step": 12, "achieved": 900.0}}\n')
    text = profiling.stats_summary(str(stats), "cmd", str(bench))
    assert "12 calls, average 100.00 us" in text
    assert "bench.py in the same run: average launch 125.00 us over 12 launches per step" in text
    assert text.strip().endswith("rocprofv3 average / bench.py average: 0.800")


def test_stats_summary_covers_the_fp8_matrix_path(tmp_path):
    stats = tmp_path / "s.csv"
    with open(stats, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"])
        w.writerow([GEMM, 12, 1200000, 100000, 50.0])
        w.writerow(["void fp8blk::block_gemm_fp8_kernel<256, 128>(...)", 12, 840000, 70000, 50.0])
    bench = tmp_path / "b.json"
    bench.write_text('{"roofline": {"avg_launch_us": 100.0, "launches_per_step": 12, "achieved": 1000.0}, '
                     '"fp8_matrix_core_path": {"avg_launch_us": 72.0, "launches_per_step": 12, "gemm_tflops": 1400.0}}\n')
    text = profiling.stats_summary(str(stats), "cmd", str(bench))
    assert "block_gemm_fp8_kernel (all instantiations): 12 calls, average 70.00 us" in text
    assert "average launch 72.00 us over 12 launches per step, 1400.0 TFLOP/s" in text
    assert text.strip().endswith("rocprofv3 average / bench.py average: 0.972")
