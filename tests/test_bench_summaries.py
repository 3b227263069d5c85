"""Host logic of bench.py's profile summaries, on small synthetic rocprofv3
CSV files: kernel matching (the dequantiser is not taken for the quantiser),
the copy calibration (the last three copies), and per-grid kernel statistics
(the forward GEMM's line at the bench shape)."""

import csv
import json

import bench

CNT_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=CNT_FIELDS)
        w.writeheader()
        for d, name, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


def test_hbm_summary_matches_kernels_and_calibrates(tmp_path):
    kib = bench.CALIB_BYTES / 1024.0
    n = 11008 * 4096
    q = "qlora::quantize_nf4_kernel(float const*, long, long, unsigned char*, float*)"
    dq = "qlora::dequantize_nf4_kernel(unsigned int const*, signed char const*)"
    # an early, larger copy and quantisation that the summary must skip
    fetch = [(1, "__amd_rocclr_copyBuffer", 10 * kib), (2, q, 5 * n)] + \
        [(3 + i, q, n * 4 / 1024 / 2.0) for i in range(3)] + \
        [(6 + i, dq, (n // 2) / 1024 / 2.0) for i in range(3)] + \
        [(20 + i, "__amd_rocclr_copyBuffer", kib / 2.0) for i in range(3)]
    write = [(1, "__amd_rocclr_copyBuffer", 10 * kib), (2, q, 5 * n)] + \
        [(3 + i, q, (n // 2) / 1024) for i in range(3)] + \
        [(6 + i, dq, 2 * n / 1024) for i in range(3)] + \
        [(20 + i, "__amd_rocclr_copyBuffer", kib) for i in range(3)]
    fc, wc = tmp_path / "f.csv", tmp_path / "w.csv"
    _counter_csv(fc, "FETCH_SIZE", fetch)
    _counter_csv(wc, "WRITE_SIZE", write)
    out = tmp_path / "hbm.txt"
    bench.summarize_hbm(str(out), str(fc), str(wc))
    txt = out.read_text()
    assert "fetch_scale = 2.0000" in txt and "write_scale = 1.0000" in txt
    line = [ln for ln in txt.splitlines() if ln.startswith("quantise, first level")][0]
    assert f"read {4 * n} /" in line  # 3 measured dispatches, the early one skipped
    assert [ln for ln in txt.splitlines() if ln.startswith("dequantise:")]


def test_stats_summary_per_grid(tmp_path):
    trace = tmp_path / "bench_kernel_trace.csv"
    stats = tmp_path / "bench_kernel_stats.csv"
    fields = ["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Start_Timestamp", "End_Timestamp"]
    with open(trace, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=fields)
        w.writeheader()
        t = 0
        for i in range(4):  # two launch grids of the forward GEMM, equally often
            for tiles, us in ((256, 300), (688, 700)):
                w.writerow({"Kernel_Name": f"void qlora::{bench.FWD_GEMM}(qlora::GemmArgs)",
                            "Grid_Size_X": tiles * 256, "Grid_Size_Y": 1, "Start_Timestamp": t,
                            "End_Timestamp": t + us * 1000})
                t += 1_000_000
        w.writerow({"Kernel_Name": "qlora::reduce_partials4_kernel()", "Grid_Size_X": 1024,
                    "Grid_Size_Y": 1, "Start_Timestamp": t, "End_Timestamp": t + 5_000})
    stats.write_text("Name,Calls\n")
    log = tmp_path / "log.txt"
    log.write_text(json.dumps({"metric": "m", "value": 1.0, "ms_per_step": 0.9,
                               "rows": {"llama65b_layer_projections": {}},
                               "roofline": {"us_per_launch": 500.0}}) + "\n")
    out = tmp_path / "stats.txt"
    bench.summarize_stats(str(stats), str(log), str(out))
    txt = out.read_text()
    assert "--no-rows" in txt
    assert "(trace, all grids): 8 calls, mean 500.0 us" in txt
    assert "176128x1" in txt and "65536x1" in txt


def test_layer_forward_algorithmic_bytes():
    """Per launch of the forward GEMM: the NF4 + DQ weight (0.5 + 1/64 B per
    weight and 4 B per 16384), X, U, B and Y in bf16, once each."""
    tot = bench._layer_fwd_algo_bytes()
    M, r = 2048, 64
    ref = 0
    for K, N in [(8192, 8192)] * 4 + [(8192, 22016)] * 2 + [(22016, 8192)]:
        n = K * N
        ref += n * 0.5 + n / 64 + 4 * n / 16384 + 2 * (M * K + M * r + N * r + M * N)
    assert abs(tot - ref) < 1e-6 * ref


def test_gemv_traffic_read_from_the_hbm_summary(tmp_path, monkeypatch):
    """The GEMV roofline's traffic is the summary's counted read + write bytes
    of the few-token GEMV line, and None once the kernel sources differ."""
    good = tmp_path / "hbm.txt"
    good.write_text("# header\n"
                    f"kernel_source_sha256_16 = {bench.hbm_source_hash()}\n"
                    "dequantise: read 10 / 10, write 20 / 20, total 1.000\n"
                    "few-token GEMV, 1 token: read 122789546 / 122101792, write 57344 / 57344, "
                    "total 1.006\n")
    monkeypatch.setattr(bench, "HBM_SUMMARY", str(good))
    assert bench.read_gemv_traffic() == 122789546 + 57344
    stale = tmp_path / "stale.txt"
    stale.write_text(good.read_text().replace(bench.hbm_source_hash(), "0" * 16))
    monkeypatch.setattr(bench, "HBM_SUMMARY", str(stale))
    assert bench.read_gemv_traffic() is None
    monkeypatch.setattr(bench, "HBM_SUMMARY", str(tmp_path / "absent.txt"))
    assert bench.read_gemv_traffic() is None
