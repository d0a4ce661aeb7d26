"""Host-side reduction of rocprofv3 counter runs to per-launch HBM bytes."""
import csv
import os

from offloaded_pipeline_stage_amd import pmc

GEMM = ("void rp::(anonymous namespace)::gemm_mfma_kernel<256, 256, 2, 4, true, true, 0, true, 0>"
        "(rp::(anonymous namespace)::GemmParams)")
NORM = "void rp::rmsnorm_fwd_kernel<rp::bf16>(rp::bf16 const*, rp::bf16*, int, int, float)"


def _write(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, v) in enumerate(rows):
            w.writerow([i + 1, i + 1, k, counter, v])


def test_norm_name():
    assert pmc.norm_name(GEMM) == "gemm_mfma_kernel<256, 256, 2, 4, 1, 1, 0, 1, 0>"
    assert pmc.norm_name(NORM) == "rmsnorm_fwd_kernel<bf16>"
    assert pmc.base_name(pmc.norm_name(NORM)) == "rmsnorm_fwd_kernel"


def test_summary_calibrates_and_averages(tmp_path):
    # the copy of 1 MiB reads as 512 KiB fetched / 2048 KiB written, so the
    # scales are x2 and x0.5; the product's two launches average 100 and 300 KiB
    _write(str(tmp_path / "f"), "FETCH_SIZE",
           [(pmc.COPY_KERNEL, 512.0), (GEMM, 100.0), (NORM, 10.0), (GEMM, 300.0), (pmc.COPY_KERNEL, 7.0)])
    _write(str(tmp_path / "w"), "WRITE_SIZE",
           [(pmc.COPY_KERNEL, 2048.0), (GEMM, 40.0), (NORM, 4.0), (GEMM, 40.0), (pmc.COPY_KERNEL, 7.0)])
    txt = pmc.summarize(str(tmp_path / "f"), str(tmp_path / "w"), 1, "t", ["cmd"])
    out = tmp_path / "sum.txt"
    out.write_text(txt)
    d = pmc.load(str(out))
    assert d["factors"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 0.5}
    g = d["kernels"]["gemm_mfma_kernel<256, 256, 2, 4, 1, 1, 0, 1, 0>"]
    assert g["launches"] == 2
    assert g["fetch_bytes"] == 200.0 * 1024 * 2.0
    assert g["write_bytes"] == 40.0 * 1024 * 0.5
    assert g["source"] == "gemm.hip"
    want = 200.0 * 1024 * 2.0 + 40.0 * 1024 * 0.5
    assert pmc.traffic_for(str(out), "gemm_mfma_kernel<256, 256, 2, 4, 1, 1, 0, 1, 0>") == want
    # the library traces some kernels by their base name only
    assert pmc.traffic_for(str(out), "rmsnorm_fwd_kernel") == 10.0 * 1024 * 2 + 4.0 * 1024 * 0.5


def test_stale_source_gives_none(tmp_path):
    _write(str(tmp_path / "f"), "FETCH_SIZE", [(pmc.COPY_KERNEL, 1024.0), (GEMM, 100.0)])
    _write(str(tmp_path / "w"), "WRITE_SIZE", [(pmc.COPY_KERNEL, 1024.0), (GEMM, 40.0)])
    txt = pmc.summarize(str(tmp_path / "f"), str(tmp_path / "w"), 1, "t", [])
    name = "gemm_mfma_kernel<256, 256, 2, 4, 1, 1, 0, 1, 0>"
    out = tmp_path / "sum.txt"
    out.write_text(txt.replace('"source_sha": "', '"source_sha": "0'))
    assert pmc.traffic_for(str(out), name) is None
    assert pmc.traffic_for(str(tmp_path / "missing.txt"), name) is None


def test_kernel_trace_summary(tmp_path):
    """The kernel-trace summary: one line per kernel in the library's name
    form, durations in microseconds, and the bench line's roofline quoted."""
    d = tmp_path / "kt"
    d.mkdir()
    with open(d / "run_kernel_stats.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write('"void rp::(anonymous namespace)::gemm_mfma_kernel<256, 256, 2, 4, true, true, 0, true, 0>'
                '(rp::(anonymous namespace)::GemmParams)",4,6000000,1500000.0,60.0,1400000,1600000,1.0\n')
        f.write('"rp::(anonymous namespace)::flash_dkdv_kernel(rp::(anonymous namespace)::FlashParams)",'
                '2,2000000,1000000.0,20.0,990000,1010000,1.0\n')
    bench = ('{"ms_per_step": 40.0, "value": 204800.0, "unit": "tokens/s", "roofline": {"kernel": "k", '
             '"avg_launch_ms": 1.5, "achieved": 1154.7, "unit": "TFLOP/s", "frac": 0.462, "peak": 2500}}')
    txt = pmc.summarize_kernels(str(tmp_path), "t", ["cmd"], bench)
    assert "    4      6.00    1500.0    1400.0    1600.0  60.0  gemm_mfma_kernel<256, 256, 2, 4, 1, 1, 0, 1, 0>" in txt
    assert "flash_dkdv_kernel" in txt and "1000.0" in txt
    assert "0.462 of the 2500 TFLOP/s peak" in txt
