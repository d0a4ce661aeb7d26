"""Host-side reduction of rocprofv3 counter runs to per-launch HBM bytes."""
import csv
import json
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


def test_configs_summary():
    """A bench line with configurations, the ablation, the optimizer and the
    streamed figures gives both tables, every call on its own row."""
    line = json.dumps({
        "configs": {"a": {"tokens": 8, "fwd": {"ms": 2.0, "tokens_per_s": 4000.0, "tflops": 1.5},
                          "note": "n1"},
                    "b": {"tokens": 4, "x": {"ms": 1.0, "tokens_per_s": 4000.0, "tflops": None, "note": "n2"}}},
        "optimizer": {"s_per_step": 0.3},
        "streamed": {"ms_per_step": 60.0},
        "ablation": {"workload": "w", "weights_GB_per_stage": 0.4, "grads_GB_per_bwd_stage": 0.8, "mbs": [1, 2],
                     "no_prefetch": [10.0, 20.0], "prefetch": [11.0, 21.0], "windowed": [12.0, 22.0],
                     "windowed_over_no_prefetch": [1.2, 1.1], "windowed_over_prefetch": [1.09, 1.05]}})
    txt, abl = pmc.summarize_configs(line, ["cmd"])
    assert "command: cmd" in txt
    assert any(l.startswith("a ") and "fwd" in l and "2.00" in l for l in txt.splitlines())
    assert any(l.startswith("b ") and l.rstrip().endswith("-") for l in txt.splitlines())
    assert "a: n1" in txt and "b x: n2" in txt and "host optimizer step" in txt and "streamed step, fp32" in txt
    assert "| 2 | 20 | 21 | 22 | 1.100 | 1.050 |" in abl
    _, none = pmc.summarize_configs(json.dumps({"configs": {}}), [])
    assert none is None
