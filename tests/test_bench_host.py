"""bench.py's host-side pieces, on the CPU: the rocprofv3 summaries it writes
(counter calibration on the reference copy, per-launch traffic, the
machine-readable block bench.py reads back) from small synthetic csv files,
and the kernel-code hash that keeps a stale summary from being used."""
import csv
import os

import bench


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_traffic_summary_calibration(tmp_path):
    d = tmp_path / "raw"
    d.mkdir()
    out = tmp_path / "out"
    out.mkdir()
    copy = "__amd_rocclr_copyBuffer"
    fq = "void mxk::k_fakequant<true, 0>(void const*, void*, long)"
    _write(d / "trace_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
           [[fq, 10, 22000.0, 21000.0, 23000.0], [copy, 5, 26000.0, 25000.0, 27000.0]])
    # the copy moves 64 MiB each way; FETCH_SIZE sees half of its reads
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Value"]
    _write(d / "fetch_counter_collection.csv", hdr,
           [[copy, 4096, 32768.0], [copy, 64, 1.0], [fq, 8192, 32768.0]])
    _write(d / "write_counter_collection.csv", hdr,
           [[copy, 4096, 65536.0], [copy, 64, 2.0], [fq, 8192, 65536.0]])
    bench.summarize_profiles(str(d), str(out))
    text = (out / os.path.basename(bench.TRAFFIC_FILE)).read_text()
    assert "FETCH_SIZE is scaled by 2.0000 and WRITE_SIZE by 1.0000" in text
    # fake-quant: 32768 KiB fetched x 2 + 65536 KiB written = 128 MiB, its
    # algorithmic bytes exactly
    assert f"traffic_bytes k_fakequant<true, 0> {128 << 20}" in text
    assert "kernel_code_sha256_prefix " + bench.kernel_code_hash() in text
    trace = (out / "mx_bf16_8192x4096_kernel_trace.md").read_text()
    row = next(ln for ln in trace.splitlines() if ln.startswith("| `k_fakequant<true, 0>`"))
    # 134217728 bytes in 22 us = 6101 GB/s = 76.3 % of 8 TB/s
    assert "| 22.00 |" in row and "| 134217728 | 6101 | 76.3 |" in row


def test_algorithmic_bytes_agree_with_the_step():
    n = bench.BENCH_ELEMS
    for op, k in bench.KERNEL_OF.items():
        assert bench.KERNEL_BYTES_PER_ELEM[k] == bench.BYTES_PER_ELEM[op]
    # NVFP4 quantize is its two kernels
    assert (bench.KERNEL_BYTES_PER_ELEM["k_absmax_partials<true>"]
            + bench.KERNEL_BYTES_PER_ELEM["k_quantize_nv<true, false>"]) * n \
        == bench.EXTRA_BYTES_PER_ELEM["quantize_nvfp4"] * n
    assert bench.BYTES_PER_ELEM["fakequant_ocp"] * n == 134217728


def test_kernel_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int a; // one\n/* two */ int b;\n")
    monkeypatch.setattr(bench, "KERNEL_SRCS", (str(src),))
    h1 = bench.kernel_code_hash()
    src.write_text("int a;   // changed comment\n/* other */\nint b;\n")
    assert bench.kernel_code_hash() == h1
    src.write_text("int a; int c;\n")
    assert bench.kernel_code_hash() != h1


def test_more_than_one_gpu_exits_with_a_message():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
