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
    n = bench.STEP_ELEMS
    copy = "void (anonymous namespace)::k_ceiling_copy(u32x4 const*, u32x4*, long)"
    fq = "void mxk::k_fakequant<true, 0, 1, 64>(void const*, void*, long)"
    wg = 256
    grid = n // 2048 * wg  # work-items: one tile of 256 x 8 elements per workgroup
    # two fake-quant dispatches of 1000 us and 1100 us, one copy of 900 us
    _write(d / "step_trace_kernel_trace.csv",
           ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"],
           [[fq, grid, wg, 0, 1_000_000], [fq, grid, wg, 2_000_000, 3_100_000],
            [copy, grid, wg, 4_000_000, 4_900_000]])
    # the copy moves 2n bytes each way; FETCH_SIZE sees half of its reads
    kib = 2 * n / 1024
    hdr = ["Kernel_Name", "Grid_Size", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    _write(d / "step_fetch_counter_collection.csv", hdr,
           [[copy, grid, wg, "FETCH_SIZE", kib / 2], [fq, grid, wg, "FETCH_SIZE", kib / 2]])
    _write(d / "step_write_counter_collection.csv", hdr,
           [[copy, grid, wg, "WRITE_SIZE", kib], [fq, grid, wg, "WRITE_SIZE", kib]])
    bench.summarize_profiles(str(d), str(out))
    text = (out / os.path.basename(bench.TRAFFIC_FILE)).read_text()
    assert "FETCH_SIZE is scaled by 2.0000 and WRITE_SIZE by 1.0000" in text
    # fake-quant: 2n bytes fetched (after scaling) + 2n written = 4n, its
    # algorithmic bytes exactly
    assert f"traffic_bytes k_fakequant<true, 0, 1, 64> {4 * n}" in text
    assert "kernel_code_sha256_prefix " + bench.kernel_code_hash() in text
    trace = (out / (bench.PROFILE_STEM["step"] + "_kernel_trace.md")).read_text()
    row = next(ln for ln in trace.splitlines() if ln.startswith("| `k_fakequant<true, 0, 1, 64>`"))
    # 4n bytes in 1050 us on average
    gbs = 4 * n / 1050e-6 / 1e9
    assert f"| {n // 2048} | {n} | 2 | 1050.00 | 1000.00 | 1100.00 | {4 * n} | {gbs:.0f} |" in row
    assert f"{gbs / 80:.1f} |" in row
    # bench.py reads the figure back for the op whose kernel family matches,
    # while the kernel code is unchanged
    monkey_file = out / os.path.basename(bench.TRAFFIC_FILE)
    old = bench.TRAFFIC_FILE
    try:
        bench.TRAFFIC_FILE = str(monkey_file)
        assert bench.measured_traffic("fakequant_ocp") == ("k_fakequant<true, 0, 1, 64>", 4 * n)
        assert bench.measured_traffic("quantize_ocp") is None
    finally:
        bench.TRAFFIC_FILE = old


def test_kernel_names_and_families():
    short = bench._kernel_short
    assert short("void mxk::k_quantize<true, 3, 4, 256>(void const*, unsigned int*, unsigned char*, "
                 "long)") == "k_quantize<true, 3, 4, 256>"
    assert short("(anonymous namespace)::k_ceiling_copy(u32x4 const*, u32x4*, long) [clone .kd]"
                 ) == "k_ceiling_copy"
    assert short("mxk::k_sum_partials(double const*, long, double*)") == "k_sum_partials"
    fam = bench.kernel_family
    assert fam("k_quantize<true, 3, 4, 256>") == "k_quantize<true, 3, U>"
    assert fam("k_quantize<true, 1, 2, 128>") == "k_quantize<true, 1, U>"
    assert fam("k_dequantize<true, 2, 64>") == "k_dequantize<true, U>"
    assert fam("k_block_mse<true, true, 2>") == "k_block_mse<true, true, U>"
    assert fam("k_quantize_nv<true, false>") == "k_quantize_nv<true, false>"
    assert fam("k_quantize_fused<true, 0, true>") == "k_quantize_fused<true, 0, true>"
    assert bench.items_per_thread("k_fakequant<true, 1, 2, 256>") == 2
    assert bench.items_per_thread("k_fakequant<true, 0, 1, 64>") == 1
    assert bench.threads_per_group("k_fakequant<true, 0, 1, 64>") == 64
    assert bench.threads_per_group("k_block_mse<true, true, 2>") == 256
    assert bench.items_per_thread("k_quantize_fused<true, 0, true>") == bench.FUSED_ITEMS
    assert bench.items_per_thread("k_quantize8<true, 2, 256>") == 2
    assert bench.items_per_thread("k_quantize_nv<true, false>") is None
    # the two-lanes-per-block kernel: 16 elements per item
    assert bench.kernel_family("k_quantize_pair<3, 1>") == "k_quantize_pair<3, U>"
    assert bench.tile_elems("k_quantize_pair<3, 1>", 8192) == 8192 * 4096
    assert bench.tile_elems("k_quantize<true, 3, 2, 256>", 8192) == 8192 * 4096
    assert bench.tile_elems("k_dequantize<true, 2, 64>", 32768) == 32768 * 1024
    assert bench.kernel_bytes_per_elem("k_quantize<true, 0, 1, 256>") == 2 + 0.5 + 1 / 32
    assert bench.kernel_bytes_per_elem("k_ceiling_read") == 2.0


def test_algorithmic_bytes_agree_with_the_step():
    n = bench.STEP_ELEMS
    for op, k in bench.KERNEL_OF.items():
        assert bench.KERNEL_BYTES_PER_ELEM[k] == bench.BYTES_PER_ELEM[op]
        name = k.split("<")[0]
        assert bench.kernel_family(k.replace(", U>", ", 1, 64>" if name in bench.NT_KERNELS
                                              else ", 1>")) == k
    # NVFP4 quantize is its two kernels
    assert (bench.KERNEL_BYTES_PER_ELEM["k_absmax_partials<true>"]
            + bench.KERNEL_BYTES_PER_ELEM["k_quantize_nv<true, false>"]) * n \
        == bench.EXTRA_BYTES_PER_ELEM["quantize_nvfp4"] * n
    # the step's buffer: 196 matrices, 2,818,572,288 elements
    assert n == bench.__dict__["STEP_ELEMS"] == 28 * sum(
        o * i for o, i in ((3072, 3072), (1024, 3072), (1024, 3072), (3072, 3072),
                           (8192, 3072), (8192, 3072), (3072, 8192)))
    assert bench.BYTES_PER_ELEM["fakequant_ocp"] * n == 11274289152
    assert bench.BYTES_PER_ELEM["quantize_ocp"] * n == 7134511104


def test_beside_phase_attributes_by_grid():
    elems = bench.PHASES["beside"]["elems"]
    assert elems("k_quantize<true, 0, 4, 256>", 16384) == 16384 * 8192
    assert elems("k_quantize<true, 3, 4, 256>", 4096) == 8192 * 4096
    assert elems("k_fakequant<true, 0, 2, 256>", 8192) == 8192 * 4096
    assert elems("k_quantize_fused<true, 0, true>", 8192) == 8192 * 4096
    assert elems("k_quantize8<true, 2, 256>", 8192) == 8192 * 4096


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


def test_suite_attribution_by_elements(tmp_path):
    # one dispatch per workload shape; the run ends with the MoE dequantize
    # launches and the untimed QSNR pass after them is left out
    wg = 256
    disp = [("k_quantize<true, 0, 1, 256>", 688128 * 3072 // 2048),
            ("k_quantize<true, 0, 1, 256>", bench.STEP_ELEMS // 2048),
            ("k_quantize<true, 0, 4, 256>", 3072 * 3072 // 8192),
            ("k_quantize<true, 0, 1, 256>", 128 * 3072 * 4096 // 2048),
            ("k_dequantize<true, 2, 64>", 128 * 4096 * 1536 // 1024),
            ("k_dequantize<true, 2, 256>", 16384 * 8192 // 4096)]
    rows = [[f"void mxk::{k}(void const*, long)", g * wg, wg, 10 * i * 1000, (10 * i + 1) * 1000]
            for i, (k, g) in enumerate(disp)]
    _write(tmp_path / "suite_kernel_trace.csv",
           ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"],
           rows)
    bench._summarize_suite(str(tmp_path / "suite_kernel_trace.csv"), "", str(tmp_path))
    text = (tmp_path / "mx_workloads_suite_kernel_trace.md").read_text()
    for label in ("K=3072 [688128, 3072] | `k_quantize<true, 0, 1, 256>`",
                  "one launch [917504, 3072] | `k_quantize<true, 0, 1, 256>`",
                  "q/o [3072, 3072] | `k_quantize<true, 0, 4, 256>`",
                  "MoE w13 [128x3072, 4096] | `k_quantize<true, 0, 1, 256>`",
                  "MoE w2 [128x4096, 1536] | `k_dequantize<true, 2, 64>`"):
        assert label in text, label
    assert "| bf16 Laplace" not in text and "unattributed" not in text


def test_every_op_beside_the_step_has_roofline_kernels():
    # every op run_beside times maps to the kernels whose traffic it reads
    for op in list(bench.EXTRA_BYTES_PER_ELEM) + ["reference_copy", "quantize_ocp",
                                                 "quantize_oas"]:
        fams = [f for g in bench.BESIDE_KERNELS[op] for f in (g if isinstance(g, tuple) else (g,))]
        full = [f.replace(", U>", ", 4, 256>" if f.split("<")[0] in bench.NT_KERNELS else ", 4>")
                for f in fams]
        assert fams and all(bench.kernel_bytes_per_elem(f) is not None
                            or f == "k_ceiling_copy" for f in full), op
        row = {"GB/s": 1.0, "frac_hbm": 0.5, "bytes": 10, "us": 1.0}
        r = bench.beside_roofline(op, row)
        assert r["bound"] == "hbm" and r["peak"] == bench.HBM_PEAK_GBS and r["frac"] == 0.5
        assert r["traffic"] is None or r["traffic"] > 0


def test_suite_attribution_nvfp4_moe(tmp_path):
    # NVFP4 on the MoE experts: the 2,048-workgroup maximum pass alternates
    # w13, w2 in every call; the exponent reduction is one workgroup; the
    # multi-GB block pass (one tile per workgroup) is told apart by elements
    wg = 256
    m13, m2 = 128 * 3072 * 4096, 128 * 4096 * 1536
    disp = []
    for _ in range(2):  # two calls: w13 then w2 each
        for n in (m13, m2):
            disp += [("k_absmax_partials<true>", 2048, wg), ("k_nv_prepare", 1, wg),
                     ("k_quantize_nv_big<true, false, 2, 128>", n // 8 // 256, 128)]
    disp += [("k_dequantize<true, 2, 64>", m2 // 8 // 128, 64)]  # ends the timed part
    rows = [[f"void mxk::{k}(void const*, long)", g * w, w, 10 * i * 1000, (10 * i + 1) * 1000]
            for i, (k, g, w) in enumerate(disp)]
    _write(tmp_path / "suite_kernel_trace.csv",
           ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"],
           rows)
    bench._summarize_suite(str(tmp_path / "suite_kernel_trace.csv"), "", str(tmp_path))
    text = (tmp_path / "mx_workloads_suite_kernel_trace.md").read_text()
    lines = {ln.split("|")[1].strip() + " " + ln.split("|")[2].strip(): ln
             for ln in text.splitlines() if ln.startswith("| ") and "`k_" in ln}
    for wl, n in (("MoE w13 [128x3072, 4096]", m13), ("MoE w2 [128x4096, 1536]", m2)):
        absmax = lines[f"{wl} `k_absmax_partials<true>`"].split("|")
        assert absmax[3].strip() == "2" and int(absmax[7]) == 2 * n  # dispatches, x read once
        block = lines[f"{wl} `k_quantize_nv_big<true, false, 2, 128>`"].split("|")
        assert block[3].strip() == "2" and int(block[7]) == int(n * (2 + 0.5 + 1 / 16))
    assert "NVFP4 tensor-exponent reduction (MoE experts) `k_nv_prepare`" in lines
    assert "unattributed" not in text
