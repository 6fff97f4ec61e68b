"""Benchmark of the MXFP4 hot path on one MI355X.

One step = every operation of the path over one batch of bf16 activations
[8192 tokens, 4096 hidden] (Student-t(3) body, 20 outlier channels x50):
  quantize (OCP scale), quantize (overflow-aware scale), dequantize -> bf16,
  fused fake-quant (OCP), per-block MSE of the OCP result.
Throughput = algorithmic bytes of the step / step time (inputs resident in
HBM). Buffer sets rotate so the working set is >= 1 GiB and the 256 MB
Infinity Cache cannot serve a step from the previous one.

Prints ONE JSON line. --gpus N with N > 1 exits: this path runs on one GPU.

--suite instead times each operation on the other workloads alone (fp32
normal [1024, 4096]; the Llama-3.2-3B-shaped linear stack, per matrix, as one
multi-tensor call and grouped by K; the 128-expert MoE weights; bf16 Laplace
[16384, 8192] with sparse outliers), with per-launch HIP events (median, p10,
p90), warm (cache-resident) and cold (rotated) figures where the tensor fits
the cache, and for the small fp32 case the host-side single-launch latency
and the per-launch time inside a replayed HIP graph. It prints one JSON line
per measurement and a markdown table.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "MXFP4 quantize/fake-quant GB/s (bf16 in) and % of HBM peak, 1× MI355X"
WORKLOAD = ("bf16 activations 8192 tokens x 4096 hidden, Student-t(nu=3), "
            "20 outlier channels x50 (seed 2)")

# algorithmic bytes per element (bf16 input): what each op must move
BYTES_PER_ELEM = {
    "quantize_ocp": 2 + 0.5 + 1 / 32,      # x in, codes + scales out
    "quantize_oas": 2 + 0.5 + 1 / 32,
    "dequantize_bf16": 0.5 + 1 / 32 + 2,   # codes + scales in, y out
    "fakequant_ocp": 2 + 2,                # x in, y out
    "block_mse": 2 + 0.5 + 1 / 32 + 4 / 32,  # x, codes, scales in; fp32/block out
}
OPS = list(BYTES_PER_ELEM)
# measured beside the step (not part of it): the page-faithful
# overflow-aware variants and fake-quant in the overflow-aware modes
EXTRA_BYTES_PER_ELEM = {
    "quantize_oas_bits": 2 + 0.5 + 1 / 32,
    "quantize_oas_nf": 2 + 0.5 + 1 / 32,
    "fakequant_oas": 4.0,
    "fakequant_oas_nf": 4.0,
    # MXFP8 (E4M3): one code byte per element
    "quantize_mxfp8": 2 + 1 + 1 / 32,
    "dequantize_mxfp8_bf16": 1 + 1 / 32 + 2,
    "fakequant_mxfp8": 4.0,
    # NVFP4 comparator: quantize reads x twice (tensor maximum, then blocks)
    "quantize_nvfp4": 2 + 2 + 0.5 + 1 / 16,
    "dequantize_nvfp4_bf16": 0.5 + 1 / 16 + 2,
    # MBS-Static: 16-element sub-block bytes plus one macro byte per 128
    "quantize_mbs": 2 + 0.5 + 1 / 16 + 1 / 128,
    "dequantize_mbs_bf16": 0.5 + 1 / 16 + 1 / 128 + 2,
    # one pass: codes + scales + y + block MSE + tensor sums (quantize,
    # dequantize and block MSE of the step fused; x read once)
    "quantize_fused": 2 + 0.5 + 1 / 32 + 2 + 4 / 32,
    # fused fake-quant of the comparators (NVFP4 reads x twice)
    "fakequant_nvfp4": 2 + 2 + 2,
    "fakequant_mbs": 2 + 2,
}
KERNEL_OF = {"quantize_ocp": "k_quantize<true, 0>", "quantize_oas": "k_quantize<true, 1>",
             "dequantize_bf16": "k_dequantize<true>", "fakequant_ocp": "k_fakequant<true, 0>",
             "block_mse": "k_block_mse<true, true>"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mx_bf16_8192x4096_hbm_traffic.md")
# launches per timing of the multi-GB suite workloads: warm-up, then timed
# twice (per-launch events, then back to back)
BIG_TIMED, BIG_WARM = 20, 3
KERNEL_SRCS = (os.path.join(ROOT, "microscaling_fp4_block_mx_amd", "csrc", "mx_kernels.hip"),
               os.path.join(ROOT, "microscaling_fp4_block_mx_amd", "csrc", "mx_internal.h"))


def kernel_code_hash() -> str:
    """sha256 prefix of the kernel sources (mx_kernels.hip, mx_internal.h)
    with comments and whitespace removed: a comment edit keeps the profiled
    traffic figures valid, any code edit does not."""
    import hashlib
    import re
    text = ""
    for path in KERNEL_SRCS:
        text += open(path).read() + "\n"
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = re.sub(r"\s+", " ", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def measured_traffic(op):
    """HBM bytes per launch of op's kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None if that summary was taken on
    different kernel code than the one built here."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
        h = kernel_code_hash()
    except OSError:
        return None
    if ("kernel_code_sha256_prefix " + h) not in lines:
        return None
    key = "traffic_bytes " + KERNEL_OF[op] + " "
    for ln in lines:
        if ln.startswith(key):
            return int(ln.split()[-1])
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--rotate-gib", type=float, default=1.5,
                    help="minimum working set across rotated buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--suite", action="store_true",
                    help="time the operations on the other workloads instead of the step")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from the rocprofv3 csv files in DIR "
                         "(trace_*, fetch_*, write_*, suite_*) and exit; needs no GPU")
    return ap.parse_args()


def main():
    args = parse()
    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark measures one GPU only; every MX block is independent, "
              "so the path shards by rows with no exchange. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.suite:
        return suite(args, dev)
    torch.cuda.set_device(dev)
    mx.load_library()

    x_host = workloads.bf16_student_t_outlier_channels(2)
    R_, K_ = x_host.shape
    n = x_host.numel()
    per_set = n * (2 + 0.5 * 2 + 2 / 32 + 2 + 2 + 4 / 32 + 1 + 1 / 32 + 1 / 16 + 1 / 16 + 1 / 128)
    n_sets = max(2, int(np.ceil(args.rotate_gib * 2 ** 30 / per_set)))

    x0 = x_host.to(dev)
    sets = []
    for _ in range(n_sets):
        sets.append(dict(
            x=x0.clone(),
            c_ocp=torch.empty((R_, K_ // 2), dtype=torch.uint8, device=dev),
            s_ocp=torch.empty((R_, K_ // 32), dtype=torch.uint8, device=dev),
            c_oas=torch.empty((R_, K_ // 2), dtype=torch.uint8, device=dev),
            s_oas=torch.empty((R_, K_ // 32), dtype=torch.uint8, device=dev),
            y_dq=torch.empty_like(x0),
            y_fq=torch.empty_like(x0),
            bm=torch.empty((R_, K_ // 32), dtype=torch.float32, device=dev),
            c8=torch.empty((R_, K_), dtype=torch.uint8, device=dev),
            s8=torch.empty((R_, K_ // 32), dtype=torch.uint8, device=dev),
            bnv=torch.empty((R_, K_ // 16), dtype=torch.uint8, device=dev),
            tnv=torch.full((1,), 127, dtype=torch.uint8, device=dev),
            smb=torch.empty((R_, K_ // 16), dtype=torch.uint8, device=dev),
            mmb=torch.empty((R_, K_ // 128), dtype=torch.uint8, device=dev),
        ))
    del x0
    sums = torch.empty(2, dtype=torch.float64, device=dev)
    ws_bytes = mx.mx_block_mse_workspace_size(R_, K_)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    wsnv_bytes = mx.mx_nvfp4_workspace_size(R_, K_)
    wsnv = torch.empty(wsnv_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def run(op, b):
        if op == "quantize_ocp":
            st = mx.mx_quantize(b["x"].data_ptr(), mx.MX_BF16, R_, K_, mx.MX_SCALE_OCP,
                                b["c_ocp"].data_ptr(), b["s_ocp"].data_ptr(), sh)
        elif op == "quantize_oas":
            st = mx.mx_quantize(b["x"].data_ptr(), mx.MX_BF16, R_, K_, mx.MX_SCALE_OAS,
                                b["c_oas"].data_ptr(), b["s_oas"].data_ptr(), sh)
        elif op == "dequantize_bf16":
            st = mx.mx_dequantize(b["c_ocp"].data_ptr(), b["s_ocp"].data_ptr(), R_, K_,
                                  mx.MX_BF16, b["y_dq"].data_ptr(), sh)
        elif op == "fakequant_ocp":
            st = mx.mx_fakequant(b["x"].data_ptr(), mx.MX_BF16, R_, K_, mx.MX_SCALE_OCP,
                                 b["y_fq"].data_ptr(), sh)
        elif op in ("quantize_oas_bits", "quantize_oas_nf"):
            mode = mx.MX_SCALE_OAS_BITS if op.endswith("bits") else mx.MX_SCALE_OAS_NF
            st = mx.mx_quantize(b["x"].data_ptr(), mx.MX_BF16, R_, K_, mode,
                                b["c_oas"].data_ptr(), b["s_oas"].data_ptr(), sh)
        elif op == "quantize_mxfp8":
            st = mx.mx_quantize_mxfp8(b["x"].data_ptr(), mx.MX_BF16, R_, K_, b["c8"].data_ptr(),
                                      b["s8"].data_ptr(), sh)
        elif op == "dequantize_mxfp8_bf16":
            st = mx.mx_dequantize_mxfp8(b["c8"].data_ptr(), b["s8"].data_ptr(), R_, K_, mx.MX_BF16,
                                        b["y_dq"].data_ptr(), sh)
        elif op == "fakequant_mxfp8":
            st = mx.mx_fakequant_mxfp8(b["x"].data_ptr(), mx.MX_BF16, R_, K_,
                                       b["y_fq"].data_ptr(), sh)
        elif op == "quantize_nvfp4":
            st = mx.mx_quantize_nvfp4(b["x"].data_ptr(), mx.MX_BF16, R_, K_, b["c_oas"].data_ptr(),
                                      b["bnv"].data_ptr(), b["tnv"].data_ptr(), wsnv.data_ptr(),
                                      wsnv_bytes, sh)
        elif op == "dequantize_nvfp4_bf16":
            st = mx.mx_dequantize_nvfp4(b["c_oas"].data_ptr(), b["bnv"].data_ptr(),
                                        b["tnv"].data_ptr(), R_, K_, mx.MX_BF16,
                                        b["y_dq"].data_ptr(), sh)
        elif op == "quantize_mbs":  # codes land in c_oas; dequantize_mbs_bf16 runs next
            st = mx.mx_quantize_mbs(b["x"].data_ptr(), mx.MX_BF16, R_, K_, b["c_oas"].data_ptr(),
                                    b["smb"].data_ptr(), b["mmb"].data_ptr(), sh)
        elif op == "dequantize_mbs_bf16":
            st = mx.mx_dequantize_mbs(b["c_oas"].data_ptr(), b["smb"].data_ptr(),
                                      b["mmb"].data_ptr(), R_, K_, mx.MX_BF16,
                                      b["y_dq"].data_ptr(), sh)
        elif op == "quantize_fused":
            st = mx.mx_quantize_fused(b["x"].data_ptr(), mx.MX_BF16, R_, K_, mx.MX_SCALE_OCP,
                                      b["c_oas"].data_ptr(), b["s_oas"].data_ptr(),
                                      b["y_fq"].data_ptr(), b["bm"].data_ptr(), sums.data_ptr(),
                                      ws.data_ptr(), ws_bytes, sh)
        elif op == "fakequant_nvfp4":
            st = mx.mx_fakequant_nvfp4(b["x"].data_ptr(), mx.MX_BF16, R_, K_, b["y_fq"].data_ptr(),
                                       wsnv.data_ptr(), wsnv_bytes, sh)
        elif op == "fakequant_mbs":
            st = mx.mx_fakequant_mbs(b["x"].data_ptr(), mx.MX_BF16, R_, K_, b["y_fq"].data_ptr(), sh)
        elif op in ("fakequant_oas", "fakequant_oas_nf"):
            mode = mx.MX_SCALE_OAS if op == "fakequant_oas" else mx.MX_SCALE_OAS_NF
            st = mx.mx_fakequant(b["x"].data_ptr(), mx.MX_BF16, R_, K_, mode,
                                 b["y_fq"].data_ptr(), sh)
        else:
            st = mx.mx_block_mse(b["x"].data_ptr(), mx.MX_BF16, b["c_ocp"].data_ptr(),
                                 b["s_ocp"].data_ptr(), R_, K_, b["bm"].data_ptr(),
                                 sums.data_ptr(), ws.data_ptr(), ws_bytes, sh)
        if st != mx.MX_OK:
            raise RuntimeError(mx.mx_status_string(st))

    def step(i):
        b = sets[i % n_sets]
        for op in OPS:
            run(op, b)

    # warmup (also produces the codes each set's dequantize / block_mse read)
    for i in range(max(args.warmup, n_sets)):
        step(i)
    torch.cuda.synchronize()

    # timed region: K whole steps between two events on the launch stream
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / K

    # per-kernel launch time: each op alone, back to back over the rotating
    # sets, K * n_sets launches between two events on the same stream
    for i in range(n_sets):  # codes for the MXFP8 / NVFP4 dequantize
        run("quantize_mxfp8", sets[i])
        run("quantize_nvfp4", sets[i])
    op_ms = {}
    for op in OPS + list(EXTRA_BYTES_PER_ELEM):
        for i in range(n_sets):
            run(op, sets[i])
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m = max(K, 2 * n_sets)
        a0.record(stream)
        for i in range(m):
            run(op, sets[i % n_sets])
        a1.record(stream)
        torch.cuda.synchronize()
        op_ms[op] = a0.elapsed_time(a1) / m

    # reference: a plain device copy of the same bf16 tensor (read n*2 bytes,
    # write n*2 bytes) timed the same way; it is also the calibration kernel
    # for the HBM traffic counters
    for i in range(n_sets):
        sets[i]["y_fq"].copy_(sets[i]["x"])
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m = max(K, 2 * n_sets)
    c0.record(stream)
    for i in range(m):
        sets[i % n_sets]["y_fq"].copy_(sets[i % n_sets]["x"])
    c1.record(stream)
    torch.cuda.synchronize()
    copy_us = c0.elapsed_time(c1) * 1e3 / m

    bytes_op = {op: BYTES_PER_ELEM[op] * n for op in OPS}
    bytes_step = sum(bytes_op.values())
    value = bytes_step / (ms_per_step * 1e-3) / 1e9

    breakdown = {}
    for op in OPS:
        gbs = bytes_op[op] / (op_ms[op] * 1e-3) / 1e9
        breakdown[op] = {"us": round(op_ms[op] * 1e3, 2), "GB/s": round(gbs, 1),
                         "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
                         "bytes": int(bytes_op[op])}
    extra = {}
    for op, bpe in EXTRA_BYTES_PER_ELEM.items():
        gbs = bpe * n / (op_ms[op] * 1e-3) / 1e9
        extra[op] = {"us": round(op_ms[op] * 1e3, 2), "GB/s": round(gbs, 1),
                     "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "bytes": int(bpe * n)}
    dom = max(OPS, key=lambda o: op_ms[o])
    dom_gbs = bytes_op[dom] / (op_ms[dom] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom),
                "bytes_per_launch": int(bytes_op[dom]),
                "avg_launch_us": round(op_ms[dom] * 1e3, 2)}

    # quantization quality of the bench tensor per scale mode (outside the
    # timed region): tensor MSE and QSNR from the block-error kernel
    quality = {}
    b = sets[0]
    for mode in mx.MODES:
        c, sc = mx.quantize(b["x"], mode)
        _, sums = mx.block_mse(b["x"], c, sc, per_block=False)
        sse, ssq = sums.tolist()
        quality["mxfp4_" + mode] = {"mse": sse / n, "qsnr_db": round(10 * np.log10(ssq / sse), 4)}
    y8 = mx.fakequant_mxfp8(b["x"]).float()
    xf = b["x"].float()
    sse8 = float(((xf - y8).double() ** 2).sum())
    quality["mxfp8"] = {"mse": sse8 / n,
                        "qsnr_db": round(10 * np.log10(float((xf.double() ** 2).sum()) / sse8), 4)}
    cn, bn, tn = mx.quantize_nvfp4(b["x"])
    ynv = mx.dequantize_nvfp4(cn, bn, tn, torch.float32)
    ssenv = float(((xf - ynv).double() ** 2).sum())
    quality["nvfp4"] = {"mse": ssenv / n,
                        "qsnr_db": round(10 * np.log10(float((xf.double() ** 2).sum()) / ssenv), 4)}
    cm, sm, mm = mx.quantize_mbs(b["x"])
    ymb = mx.dequantize_mbs(cm, sm, mm, torch.float32)
    ssemb = float(((xf - ymb).double() ** 2).sum())
    quality["mbs_static"] = {"mse": ssemb / n,
                             "qsnr_db": round(10 * np.log10(float((xf.double() ** 2).sum()) / ssemb), 4)}
    del y8, xf, ynv, ymb

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(x_host, args.cpu_seconds, sets[0]["x"])

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD, "rows": R_, "k": K_, "step": OPS,
                   "bytes_per_step": int(bytes_step),
                   "elements_per_s": round(n / (ms_per_step * 1e-3), 1),
                   "rotation_sets": n_sets,
                   "working_set_gib": round(n_sets * per_set / 2 ** 30, 2),
                   "wall_s_timed": round(wall, 4),
                   "device_copy_reference": {"bytes": 4 * n, "us": round(copy_us, 2),
                                             "GB/s": round(4 * n / copy_us / 1e3, 1)}},
        "breakdown": breakdown,
        "beside_the_step": extra,
        "quality": quality,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "env": {"device": torch.cuda.get_device_name(dev), "torch": torch.__version__,
                "hip": torch.version.hip},
    }
    print(json.dumps(out), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_host, target_s, x_dev):
    """The oracle as it stands, on the host cores, over a bounded sample of
    the same workload (leading rows), running the same step: first on every
    core, then on one thread over a smaller sample. The first sample's oracle
    outputs are also compared with the library's on the same rows (codes and
    scales of both modes, dequantize, fake-quant bit for bit; block MSE and
    tensor sums to a relative 1e-6)."""
    import numpy as np
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import oracle
    import workloads

    oracle.build(force=not os.path.exists(os.path.join(ROOT, "oracle", "libmxref.so")))
    cores = max(1, len(os.sched_getaffinity(0)))
    xs_full = workloads.to_bf16_bits(x_host)
    k = xs_full.shape[1]

    def step(xs, threads):
        c, s = oracle.quantize(xs, "ocp", threads=threads)
        c2, s2 = oracle.quantize(xs, "oas", threads=threads)
        y = oracle.dequantize(c, s, "bf16", threads=threads)
        f = oracle.fakequant(xs, "ocp", threads=threads)
        bm = oracle.block_mse(xs, c, s, threads=threads, with_energy=True)
        return c, s, c2, s2, y, f, bm

    def timed(rows, threads, budget):
        xs = np.ascontiguousarray(xs_full[:rows])
        done, t0, out = 0, time.perf_counter(), None
        while True:
            out = step(xs, threads)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return rows, done, el, out
            if done == 1 and rows < xs_full.shape[0]:  # size the sample to land near the budget
                grow = int(min(xs_full.shape[0], rows * max(1.0, budget / max(el, 1e-3) / 3)))
                if grow > rows:
                    rows = grow
                    xs = np.ascontiguousarray(xs_full[:rows])
                    done, t0 = 0, time.perf_counter()

    bpe = sum(BYTES_PER_ELEM[o] for o in OPS)
    rows, done, el, out = timed(256, cores, 0.7 * target_s)
    gbs = done * bpe * rows * k / el / 1e9
    rows1, done1, el1, _ = timed(16, 1, 0.3 * target_s)
    gbs1 = done1 * bpe * rows1 * k / el1 / 1e9

    # the library on the same rows
    c, s, c2, s2, y, f, (wbm, wsse, wssq) = out
    xd = x_dev[:rows].contiguous()
    gc, gs = mx.quantize(xd, "ocp")
    gc2, gs2 = mx.quantize(xd, "oas")
    gy = mx.dequantize(gc, gs, torch.bfloat16)
    gf = mx.fakequant(xd, "ocp")
    gbm, gsums = mx.block_mse(xd, gc, gs)
    sse, ssq = gsums.tolist()
    same = {
        "codes_scales_ocp": bool(np.array_equal(gc.cpu().numpy(), c) and np.array_equal(gs.cpu().numpy(), s)),
        "codes_scales_oas": bool(np.array_equal(gc2.cpu().numpy(), c2) and np.array_equal(gs2.cpu().numpy(), s2)),
        "dequantize": bool(np.array_equal(workloads.to_bf16_bits(gy), y)),
        "fakequant": bool(np.array_equal(workloads.to_bf16_bits(gf), f)),
        "block_mse_rel_1e-6": bool(np.allclose(gbm.cpu().numpy(), wbm, rtol=1e-6, atol=0)
                                   and abs(sse - wsse) <= 1e-6 * wsse and abs(ssq - wssq) <= 1e-6 * wssq),
    }
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} step(s) over the first {rows} rows x {k} of the same tensor "
                      f"({el:.1f} s, {cores} threads)",
            "single_thread": {"value": round(gbs1, 3), "unit": "GB/s",
                              "sample": f"{done1} step(s) over the first {rows1} rows ({el1:.1f} s)"},
            "cpu_model": cpu_model(),
            "sample_matches_library": same}


# ---- per-workload suite -----------------------------------------------------

def _launch_stats(fn, n_timed, n_warm, stream):
    """Per-launch HIP event times (us) of fn(i) on `stream`: median, p10,
    p90, plus the mean of the same launches issued back to back."""
    import numpy as np
    import torch

    for i in range(n_warm):
        fn(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_timed)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for i in range(n_timed):
        fn(i)
    a1.record(stream)
    torch.cuda.synchronize()
    return {"median_us": float(np.median(t)), "p10_us": float(np.percentile(t, 10)),
            "p90_us": float(np.percentile(t, 90)),
            "back_to_back_us": a0.elapsed_time(a1) * 1e3 / n_timed}


def suite(args, dev):
    import numpy as np
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import workloads

    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    n_timed = max(100, args.steps)
    n_warm = max(10, args.warmup)
    results = []

    def ok(st):
        if st != mx.MX_OK:
            raise RuntimeError(mx.mx_status_string(st))

    def report(workload, op, nbytes, stats, **extra):
        med = stats["median_us"]
        row = {"workload": workload, "op": op, "bytes": int(nbytes),
               **{k: round(v, 2) for k, v in stats.items()},
               "GB/s": round(nbytes / med / 1e3, 1),
               "frac_hbm": round(nbytes / med / 1e3 / HBM_PEAK_GBS, 4), **extra}
        results.append(row)
        print(json.dumps(row), flush=True)

    def nsets_for(per_set):
        return max(2, int(np.ceil(args.rotate_gib * 2 ** 30 / per_set)))

    # -- fp32 normal [1024, 4096] (seed 1): quantize, dequantize -> fp32, block MSE
    x1 = workloads.fp32_normal(1).to(dev)
    R, K = x1.shape
    n = x1.numel()
    per_set = n * (4 + 0.5 + 1 / 32 + 4 + 4 / 32)
    sets = []
    for _ in range(nsets_for(per_set)):
        sets.append(dict(x=x1.clone(),
                         c=torch.empty((R, K // 2), dtype=torch.uint8, device=dev),
                         s=torch.empty((R, K // 32), dtype=torch.uint8, device=dev),
                         y=torch.empty_like(x1),
                         bm=torch.empty((R, K // 32), dtype=torch.float32, device=dev)))
    wsb = mx.mx_block_mse_workspace_size(R, K)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    sums = torch.empty(2, dtype=torch.float64, device=dev)
    W1 = "fp32 normal [1024, 4096] (seed 1)"

    def q1(i, sh=sh):
        b = sets[i % len(sets)]
        ok(mx.mx_quantize(b["x"].data_ptr(), mx.MX_F32, R, K, mx.MX_SCALE_OCP,
                          b["c"].data_ptr(), b["s"].data_ptr(), sh))

    def dq1(i, sh=sh):
        b = sets[i % len(sets)]
        ok(mx.mx_dequantize(b["c"].data_ptr(), b["s"].data_ptr(), R, K, mx.MX_F32,
                            b["y"].data_ptr(), sh))

    def mse1(i, sh=sh):
        b = sets[i % len(sets)]
        ok(mx.mx_block_mse(b["x"].data_ptr(), mx.MX_F32, b["c"].data_ptr(), b["s"].data_ptr(),
                           R, K, b["bm"].data_ptr(), sums.data_ptr(), ws.data_ptr(), wsb, sh))

    def fused1(i, sh=sh):
        b = sets[i % len(sets)]
        ok(mx.mx_quantize_fused(b["x"].data_ptr(), mx.MX_F32, R, K, mx.MX_SCALE_OCP,
                                b["c"].data_ptr(), b["s"].data_ptr(), b["y"].data_ptr(),
                                b["bm"].data_ptr(), sums.data_ptr(), ws.data_ptr(), wsb, sh))

    for i in range(len(sets)):
        q1(i)
    for op, fn, bpe in (("quantize_ocp_f32", q1, 4 + 0.5 + 1 / 32),
                        ("dequantize_f32", dq1, 0.5 + 1 / 32 + 4),
                        ("block_mse_f32", mse1, 4 + 0.5 + 1 / 32 + 4 / 32),
                        ("quantize_fused_f32 (the three above in one pass)", fused1,
                         4 + 0.5 + 1 / 32 + 4 + 4 / 32)):
        report(W1, op, bpe * n, _launch_stats(fn, n_timed, n_warm, stream),
               cache=f"cold ({len(sets)} rotated sets)")
        report(W1, op, bpe * n, _launch_stats(lambda i, fn=fn: fn(0), n_timed, n_warm, stream),
               cache="warm (one set)")
    # single-launch latency: host time of one quantize call until it has run
    lat = []
    for i in range(n_timed):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        q1(i)
        torch.cuda.synchronize()
        lat.append((time.perf_counter() - t0) * 1e6)
    lat = np.array(lat)
    row = {"workload": W1, "op": "quantize_ocp_f32", "single_launch_host_us": {
        "median": round(float(np.median(lat)), 2), "p10": round(float(np.percentile(lat, 10)), 2),
        "p90": round(float(np.percentile(lat, 90)), 2)}}
    results.append(row)
    print(json.dumps(row), flush=True)
    # the same launches captured in one HIP graph and replayed
    gs = torch.cuda.Stream(dev)
    gs.wait_stream(stream)
    with torch.cuda.stream(gs):
        for i in range(len(sets)):
            q1(i, gs.cuda_stream)
    stream.wait_stream(gs)
    torch.cuda.synchronize()
    n_graph = 100
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream(dev).cuda_stream
        for i in range(n_graph):
            q1(i, cs)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    want_c = sets[0]["c"].clone()
    reps = []
    for _ in range(20):
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        g.replay()
        a1.record(stream)
        torch.cuda.synchronize()
        reps.append(a0.elapsed_time(a1) * 1e3 / n_graph)
    q1(0)
    torch.cuda.synchronize()
    assert torch.equal(want_c, sets[0]["c"]), "graph replay changed the codes"
    med = float(np.median(reps))
    row = {"workload": W1, "op": "quantize_ocp_f32", "hip_graph_per_launch_us": round(med, 2),
           "GB/s": round((4 + 0.5 + 1 / 32) * n / med / 1e3, 1),
           "launches_per_graph": n_graph, "cache": f"cold ({len(sets)} rotated sets)"}
    results.append(row)
    print(json.dumps(row), flush=True)
    del sets, x1, g, ws
    torch.cuda.empty_cache()

    # -- Laplace + sparse outliers bf16 [16384, 8192] (seed 5): quantize OCP /
    #    OAS and block MSE of each
    x5 = workloads.bf16_laplace_sparse_outliers(5).to(dev)
    R, K = x5.shape
    n = x5.numel()
    per_set = n * (2 + 2 * (0.5 + 1 / 32) + 4 / 32)
    sets = []
    for _ in range(nsets_for(per_set)):
        sets.append(dict(x=x5.clone(),
                         c=[torch.empty((R, K // 2), dtype=torch.uint8, device=dev) for _ in range(2)],
                         s=[torch.empty((R, K // 32), dtype=torch.uint8, device=dev) for _ in range(2)],
                         bm=torch.empty((R, K // 32), dtype=torch.float32, device=dev)))
    wsb = mx.mx_block_mse_workspace_size(R, K)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    W5 = "bf16 Laplace(0,1) [16384, 8192], 0.1% outliers +-U(20,200) (seed 5)"
    for j, (mode, mname) in enumerate(((mx.MX_SCALE_OCP, "ocp"), (mx.MX_SCALE_OAS, "oas"))):
        def q5(i, mode=mode, j=j):
            b = sets[i % len(sets)]
            ok(mx.mx_quantize(b["x"].data_ptr(), mx.MX_BF16, R, K, mode, b["c"][j].data_ptr(),
                              b["s"][j].data_ptr(), sh))

        def mse5(i, j=j):
            b = sets[i % len(sets)]
            ok(mx.mx_block_mse(b["x"].data_ptr(), mx.MX_BF16, b["c"][j].data_ptr(),
                               b["s"][j].data_ptr(), R, K, b["bm"].data_ptr(), sums.data_ptr(),
                               ws.data_ptr(), wsb, sh))
        for op, fn, bpe in ((f"quantize_{mname}", q5, 2 + 0.5 + 1 / 32),
                            (f"block_mse_{mname}", mse5, 2 + 0.5 + 1 / 32 + 4 / 32)):
            report(W5, op, bpe * n, _launch_stats(fn, n_timed, n_warm, stream),
                   cache=f"cold ({len(sets)} rotated sets)")
            report(W5, op, bpe * n, _launch_stats(lambda i, fn=fn: fn(0), n_timed, n_warm, stream),
                   cache="warm (one set)")
        sse, ssq = sums.tolist()
        row = {"workload": W5, "op": f"tensor_mse_{mname}", "mse": sse / n,
               "qsnr_db": round(10 * np.log10(ssq / sse), 4)}
        results.append(row)
        print(json.dumps(row), flush=True)
    del sets, x5, ws
    torch.cuda.empty_cache()

    # -- Llama-3.2-3B-shaped linear stack, bf16 N(0, 0.02): 196 per-matrix
    #    quantize launches, and two launches grouped by K
    a, b = workloads.llama32_3b_grouped(dev)
    WL = "Llama-3.2-3B linears x28 layers, bf16 N(0,0.02)"
    ca = torch.empty((a.shape[0], a.shape[1] // 2), dtype=torch.uint8, device=dev)
    sa = torch.empty((a.shape[0], a.shape[1] // 32), dtype=torch.uint8, device=dev)
    cb = torch.empty((b.shape[0], b.shape[1] // 2), dtype=torch.uint8, device=dev)
    sb = torch.empty((b.shape[0], b.shape[1] // 32), dtype=torch.uint8, device=dev)
    mats = []  # (tensor, codes, scales, row0, rows, k) in generation order
    ra = rb = 0
    for layer in range(workloads.LLAMA32_3B_LAYERS):
        for which, (_, out_f, in_f) in enumerate(workloads.LLAMA32_3B_LINEARS):
            if in_f == 8192:
                mats.append((b, cb, sb, rb, out_f, in_f))
                rb += out_f
            else:
                mats.append((a, ca, sa, ra, out_f, in_f))
                ra += out_f
    assert ra == a.shape[0] and rb == b.shape[0]
    n = a.numel() + b.numel()
    bytes_q = (2 + 0.5 + 1 / 32) * n

    def per_matrix(_):
        for t, c, s_, r0, rows, k in mats:
            ok(mx.mx_quantize(t[r0].data_ptr(), mx.MX_BF16, rows, k, mx.MX_SCALE_OCP,
                              c[r0].data_ptr(), s_[r0].data_ptr(), sh))

    def grouped(_):
        ok(mx.mx_quantize(a.data_ptr(), mx.MX_BF16, a.shape[0], a.shape[1], mx.MX_SCALE_OCP,
                          ca.data_ptr(), sa.data_ptr(), sh))
        ok(mx.mx_quantize(b.data_ptr(), mx.MX_BF16, b.shape[0], b.shape[1], mx.MX_SCALE_OCP,
                          cb.data_ptr(), sb.data_ptr(), sh))

    descs = (mx.MxTensor * len(mats))()
    for i, (t, c, s_, r0, rows, k) in enumerate(mats):
        descs[i] = mx.MxTensor(t[r0].data_ptr(), None, c[r0].data_ptr(), s_[r0].data_ptr(), rows, k)

    def multi(_):
        ok(mx.mx_quantize_multi(descs, len(mats), mx.MX_BF16, mx.MX_SCALE_OCP, sh))

    report(WL, "quantize_ocp (196 per-matrix launches)", bytes_q,
           _launch_stats(per_matrix, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WL, "quantize_ocp (196 matrices, one multi-tensor call)", bytes_q,
           _launch_stats(multi, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WL, "quantize_ocp (2 launches grouped by K)", bytes_q,
           _launch_stats(grouped, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    del a, b, ca, sa, cb, sb, mats
    torch.cuda.empty_cache()

    # -- MoE experts bf16 N(0, 0.02): quantize, then dequantize -> bf16
    w13, w2 = workloads.moe_weights(dev)
    WM = "MoE 128 experts w13 [128,3072,4096] + w2 [128,4096,1536], bf16 N(0,0.02)"
    shapes = [(w, w.numel() // w.shape[-1], w.shape[-1]) for w in (w13, w2)]
    cs = [torch.empty(w.numel() // 2, dtype=torch.uint8, device=dev) for w in (w13, w2)]
    ss = [torch.empty(w.numel() // 32, dtype=torch.uint8, device=dev) for w in (w13, w2)]
    ys = [torch.empty_like(w) for w in (w13, w2)]
    n = w13.numel() + w2.numel()

    def qm(_):
        for (w, rows, k), c, s_ in zip(shapes, cs, ss):
            ok(mx.mx_quantize(w.data_ptr(), mx.MX_BF16, rows, k, mx.MX_SCALE_OCP, c.data_ptr(),
                              s_.data_ptr(), sh))

    def dqm(_):
        for (w, rows, k), c, s_, y in zip(shapes, cs, ss, ys):
            ok(mx.mx_dequantize(c.data_ptr(), s_.data_ptr(), rows, k, mx.MX_BF16, y.data_ptr(), sh))

    report(WM, "quantize_ocp (w13 + w2)", (2 + 0.5 + 1 / 32) * n,
           _launch_stats(qm, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WM, "dequantize_bf16 (w13 + w2)", (0.5 + 1 / 32 + 2) * n,
           _launch_stats(dqm, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    del w13, w2, cs, ss, ys
    torch.cuda.empty_cache()

    quality = suite_quality(dev)
    results.extend(quality)

    # markdown summary
    print("\n| workload | op | cache | bytes | median us | p10 | p90 | back-to-back us "
          "| GB/s (median) | % of 8 TB/s |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for r in results:
        if "median_us" in r:
            print(f"| {r['workload']} | {r['op']} | {r['cache']} | {r['bytes']} | "
                  f"{r['median_us']} | {r['p10_us']} | {r['p90_us']} | {r['back_to_back_us']} | "
                  f"{r['GB/s']} | {100 * r['frac_hbm']:.1f} |")
    for r in results:
        if "median_us" not in r and r.get("op") != "qsnr_db":
            print("- " + json.dumps(r))
    fmts = list(quality[0]["qsnr_db"])
    print("\nQSNR dB = 10 log10(sum x^2 / sum (x - x_hat)^2) over the whole workload:\n")
    print("| workload | " + " | ".join(fmts) + " |")
    print("|---|" + "---|" * len(fmts))
    for r in quality:
        print(f"| {r['workload']} | " + " | ".join(f"{r['qsnr_db'][f]:.2f}" for f in fmts) + " |")


# ---- rocprofv3 summaries ------------------------------------------------------

# Algorithmic bytes per element of each kernel on the bf16 bench tensor, by
# the name rocprofv3 prints (NVFP4 quantize is two kernels: the tensor-maximum
# pass reads x, the block pass reads it again and writes codes and scales).
KERNEL_BYTES_PER_ELEM = {
    "k_quantize<true, 0>": BYTES_PER_ELEM["quantize_ocp"],
    "k_quantize<true, 1>": BYTES_PER_ELEM["quantize_oas"],
    "k_quantize<true, 2>": EXTRA_BYTES_PER_ELEM["quantize_oas_bits"],
    "k_quantize<true, 3>": EXTRA_BYTES_PER_ELEM["quantize_oas_nf"],
    "k_dequantize<true>": BYTES_PER_ELEM["dequantize_bf16"],
    "k_fakequant<true, 0>": BYTES_PER_ELEM["fakequant_ocp"],
    "k_fakequant<true, 1>": EXTRA_BYTES_PER_ELEM["fakequant_oas"],
    "k_fakequant<true, 3>": EXTRA_BYTES_PER_ELEM["fakequant_oas_nf"],
    "k_block_mse<true, true>": BYTES_PER_ELEM["block_mse"],
    "k_quantize8<true>": EXTRA_BYTES_PER_ELEM["quantize_mxfp8"],
    "k_dequantize8<true>": EXTRA_BYTES_PER_ELEM["dequantize_mxfp8_bf16"],
    "k_fakequant8<true>": EXTRA_BYTES_PER_ELEM["fakequant_mxfp8"],
    "k_absmax_partials<true>": 2.0,
    "k_quantize_nv<true, false>": EXTRA_BYTES_PER_ELEM["quantize_nvfp4"] - 2.0,
    "k_quantize_nv<true, true>": EXTRA_BYTES_PER_ELEM["fakequant_nvfp4"] - 2.0,
    "k_dequantize_nv<true>": EXTRA_BYTES_PER_ELEM["dequantize_nvfp4_bf16"],
    "k_quantize_mbs<true, false>": EXTRA_BYTES_PER_ELEM["quantize_mbs"],
    "k_quantize_mbs<true, true>": EXTRA_BYTES_PER_ELEM["fakequant_mbs"],
    "k_dequantize_mbs<true>": EXTRA_BYTES_PER_ELEM["dequantize_mbs_bf16"],
    "k_quantize_fused<true, 0, true>": EXTRA_BYTES_PER_ELEM["quantize_fused"],
    "__amd_rocclr_copyBuffer": 4.0,  # the reference copy: 2 B in + 2 B out
}
BENCH_ELEMS = 8192 * 4096

PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT -o trace -- \\\n"
             "    python3 $R/bench.py --steps 20 --warmup 5 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT -o fetch -- \\\n"
             "    python3 $R/bench.py --steps 3 --warmup 2 --no-cpu-baseline",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT -o write -- \\\n"
             "    python3 $R/bench.py --steps 3 --warmup 2 --no-cpu-baseline",
    "suite": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT -o suite -- \\\n"
             "    python3 $R/bench.py --suite",
    "sq": "rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR \\\n"
          "    SQ_INSTS_LDS SQ_BUSY_CYCLES SQ_WAVE_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $OUT -o sq -- \\\n"
          "    python3 $R/bench.py --steps 3 --warmup 2 --no-cpu-baseline",
}
# VALU issue model for the instruction-mix summary: a wave64 VALU instruction
# holds its 16-lane SIMD for 4 cycles; 256 CUs x 4 SIMDs at 2.4 GHz
SIMDS, CLOCK_GHZ, VALU_CYCLES = 1024, 2.4, 4
PROFILE_HOW = ("Each rocprofv3 command runs on its own, from a scratch working directory "
               "(`cd /tmp`), with `$R` the repository root and `$OUT` an output directory; "
               "`python3 $R/bench.py --summarize-profiles $OUT` then writes this file.")


def _kernel_short(name: str) -> str:
    for k in KERNEL_BYTES_PER_ELEM:
        if k in name:
            return k
    return name.split("(")[0].replace("void ", "").replace("mxk::", "")


def summarize_profiles(d: str, out_dir: str = os.path.join(ROOT, "profiles")) -> None:
    """The three profiles/ summaries from rocprofv3 csv output in d: the
    bench step's kernel trace, its HBM traffic (FETCH_SIZE and WRITE_SIZE,
    calibrated on the reference copy), and the suite's kernel trace (when d
    holds one), written to out_dir."""
    import collections
    import csv

    h = kernel_code_hash()
    code = ("Kernel code (`csrc/mx_kernels.hip` + `csrc/mx_internal.h`, comments and whitespace "
            f"stripped; `bench.kernel_code_hash`) sha256 prefix: `{h}`\n")
    alg = {k: int(v * BENCH_ELEMS) for k, v in KERNEL_BYTES_PER_ELEM.items()}
    pct = lambda b, us: b / us / 1e3 / HBM_PEAK_GBS * 100  # noqa: E731

    # kernel trace of the bench run
    out = ["# Kernel trace: MXFP4 hot-path kernels, bf16 8192x4096 (bench.py step)\n",
           PROFILE_HOW + "\n", "```\n" + PROFILE_CMDS["trace"] + "\n```\n",
           "Step kernels: `k_quantize<true, 0>` (OCP), `k_quantize<true, 1>` (OAS), "
           "`k_dequantize<true>`, `k_fakequant<true, 0>`, `k_block_mse<true, true>` + "
           "`k_sum_partials`; the rest run beside the step (modes 2/3 = OAS_BITS/OAS_NF, `*8` = "
           "MXFP8, `*_nv` / `k_absmax_partials` = NVFP4, `*_mbs` = MBS-Static; a `true` second "
           "template argument of those two is the fused fake-quant; `k_quantize_fused` = quantize "
           "+ dequantized output + block MSE + tensor sums in one pass). bf16 in, 8192x4096.\n",
           code,
           "| kernel | calls | avg us | min us | max us | algorithmic bytes | GB/s at avg "
           "| % of 8 TB/s |", "|---|---|---|---|---|---|---|---|"]
    with open(os.path.join(d, "trace_kernel_stats.csv")) as f:
        for r in csv.DictReader(f):
            k = _kernel_short(r["Name"])
            if k not in alg and k != "k_sum_partials":
                continue
            avg = float(r["AverageNs"]) / 1e3
            b = alg.get(k)
            out.append(f"| `{k}` | {r['Calls']} | {avg:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                       f"{float(r['MaxNs']) / 1e3:.2f} | {b if b else '-'} | "
                       f"{f'{b / avg / 1e3:.0f}' if b else '-'} | "
                       f"{f'{pct(b, avg):.1f}' if b else '-'} |")
    with open(os.path.join(out_dir, "mx_bf16_8192x4096_kernel_trace.md"), "w") as f:
        f.write("\n".join(out) + "\n")

    # HBM traffic: the reference copy (64 MiB read + 64 MiB written, the
    # largest copyBuffer dispatch) calibrates both counters
    copy = "__amd_rocclr_copyBuffer"
    with open(os.path.join(d, "write_counter_collection.csv")) as f:
        wr = [r for r in csv.DictReader(f) if _kernel_short(r["Kernel_Name"]) == copy]
    ref_grid = max(wr, key=lambda r: float(r["Counter_Value"]))["Grid_Size"]
    per = {}
    for fn, ctr in (("fetch_counter_collection.csv", "FETCH_SIZE"),
                    ("write_counter_collection.csv", "WRITE_SIZE")):
        agg = collections.defaultdict(list)
        with open(os.path.join(d, fn)) as f:
            for r in csv.DictReader(f):
                k = _kernel_short(r["Kernel_Name"])
                if k == copy and r["Grid_Size"] != ref_grid:
                    continue
                agg[k].append(float(r["Counter_Value"]))
        per[ctr] = {k: sum(v) / len(v) for k, v in agg.items()}
    cal_f = 65536.0 / per["FETCH_SIZE"][copy]
    cal_w = 65536.0 / per["WRITE_SIZE"][copy]
    out = ["# HBM traffic: MXFP4 hot-path kernels, bf16 8192x4096 (bench.py step)\n",
           PROFILE_HOW + "\n",
           "```\n" + PROFILE_CMDS["fetch"] + "\n" + PROFILE_CMDS["write"] + "\n```\n", code,
           f"Calibration: the device copy bench.py runs (`{copy}`, 64 MiB read + 64 MiB written "
           f"per dispatch) reads FETCH_SIZE {per['FETCH_SIZE'][copy]:.1f} KiB and WRITE_SIZE "
           f"{per['WRITE_SIZE'][copy]:.1f} KiB, so FETCH_SIZE is scaled by {cal_f:.4f} and "
           f"WRITE_SIZE by {cal_w:.4f}.\n",
           "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled traffic bytes | algorithmic bytes "
           "| traffic / algorithmic |", "|---|---|---|---|---|---|"]
    machine = []
    for k in KERNEL_BYTES_PER_ELEM:
        if k not in per["FETCH_SIZE"] or k not in per["WRITE_SIZE"]:
            continue
        fk, wk = per["FETCH_SIZE"][k], per["WRITE_SIZE"][k]
        t = (fk * cal_f + wk * cal_w) * 1024
        out.append(f"| `{k}` | {fk:.1f} | {wk:.1f} | {t:.0f} | {alg[k]} | {t / alg[k]:.4f} |")
        machine.append(f"traffic_bytes {k} {t:.0f}")
    out += ["\nMachine-readable (read by bench.py while the source hash matches):\n",
            "```\nkernel_code_sha256_prefix " + h] + machine + ["```"]
    with open(os.path.join(out_dir, os.path.basename(TRAFFIC_FILE)), "w") as f:
        f.write("\n".join(out) + "\n")
    if os.path.exists(os.path.join(d, "suite_kernel_trace.csv")):
        _summarize_suite(os.path.join(d, "suite_kernel_trace.csv"), code, out_dir)
    if os.path.exists(os.path.join(d, "sq_counter_collection.csv")):
        _summarize_instruction_mix(d, code, out_dir)


def _summarize_instruction_mix(d: str, code: str, out_dir: str) -> None:
    """Instructions per wave-item (one item = 8 elements per lane, 64 lanes)
    of each kernel from the SQ counters, and the time its VALU instructions
    take at full issue rate next to the kernel's traced duration."""
    import collections
    import csv

    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(os.path.join(d, "sq_counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            agg[_kernel_short(r["Kernel_Name"])][r["Counter_Name"]].append(
                float(r["Counter_Value"]))
    avg_us = {}
    trace = os.path.join(d, "trace_kernel_stats.csv")
    if os.path.exists(trace):
        with open(trace) as f:
            for r in csv.DictReader(f):
                avg_us[_kernel_short(r["Name"])] = float(r["AverageNs"]) / 1e3
    wave_items = BENCH_ELEMS / (8 * 64)
    out = ["# Instruction mix: MXFP4 hot-path kernels, bf16 8192x4096 (bench.py step)\n",
           PROFILE_HOW + "\n", "```\n" + PROFILE_CMDS["sq"] + "\n```\n", code,
           "Counts are chip totals per dispatch (SQ_WAVES equals the waves launched), "
           "averaged over the dispatches of each kernel, per wave-item: one item is 8 "
           "elements in each of a wave's 64 lanes, so the bench tensor is "
           f"{int(wave_items)} wave-items. VALU issue time = SQ_INSTS_VALU x {VALU_CYCLES} "
           f"cycles / ({SIMDS} SIMDs x {CLOCK_GHZ} GHz), the time the kernel's vector "
           "instructions need if every SIMD issued one each cycle slot with nothing else "
           "in the way; kernel time from the kernel trace of the same code.\n",
           "| kernel | waves | VALU / wave-item | SALU / wave-item | VMEM rd / wave-item "
           "| VMEM wr / wave-item | LDS / wave-item | VALU issue us | kernel us | VALU issue / "
           "kernel |", "|---|---|---|---|---|---|---|---|---|---|"]
    for k in KERNEL_BYTES_PER_ELEM:
        if k not in agg or k == "__amd_rocclr_copyBuffer":
            continue
        c = {n: sum(v) / len(v) for n, v in agg[k].items()}
        per = lambda n: c.get(n, 0.0) / wave_items  # noqa: E731
        valu_us = c.get("SQ_INSTS_VALU", 0.0) * VALU_CYCLES / (SIMDS * CLOCK_GHZ * 1e3)
        t = avg_us.get(k)
        out.append(f"| `{k}` | {int(c.get('SQ_WAVES', 0))} | {per('SQ_INSTS_VALU'):.1f} | "
                   f"{per('SQ_INSTS_SALU'):.1f} | {per('SQ_INSTS_VMEM_RD'):.2f} | "
                   f"{per('SQ_INSTS_VMEM_WR'):.2f} | {per('SQ_INSTS_LDS'):.2f} | {valu_us:.2f} | "
                   f"{f'{t:.2f}' if t else '-'} | {f'{valu_us / t:.2f}' if t else '-'} |")
    with open(os.path.join(out_dir, "mx_bf16_8192x4096_instruction_mix.md"), "w") as f:
        f.write("\n".join(out) + "\n")


def _summarize_suite(path: str, code: str, out_dir: str) -> None:
    """Per-workload kernel times of `bench.py --suite` from its kernel trace.
    Launches are told apart by kernel, dtype and grid size; the two
    196,608-workgroup groups by dispatch order (see the note written out)."""
    import collections
    import csv

    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    short = lambda n: n.split("(")[0].replace("void ", "").replace("mxk::", "")  # noqa: E731
    c1, c5 = 1024 * 4096, 16384 * 8192
    l3072, l8192 = 688128 * 3072, 86016 * 8192
    m13, m2 = 128 * 3072 * 4096, 128 * 4096 * 1536
    passes = 2 * BIG_TIMED + BIG_WARM  # dispatches of one big-workload timing
    per_matrix = {384: ("k/v [1024, 3072]", 1024 * 3072), 1152: ("q/o [3072, 3072]", 3072 * 3072),
                  3072: ("gate/up [8192, 3072] and down [3072, 8192]", 8192 * 3072)}

    def bytes_for(kernel, n, f32):
        if kernel.startswith(("k_quantize<", "k_dequantize<")):
            return n * (4.53125 if f32 else 2.53125)
        if kernel.startswith("k_block_mse<"):
            return n * (4.65625 if f32 else 2.65625)
        if kernel.startswith("k_quantize_fused<"):
            return n * (8.65625 if f32 else 4.65625)
        return None

    # the timed part ends with the MoE dequantize launches; the QSNR pass
    # that follows is not timed and is left out
    last = max(i for i, r in enumerate(rows)
               if short(r["Kernel_Name"]) == "k_dequantize<true>"
               and int(r["Grid_Size_X"]) // 256 in (196608, 98304))
    groups = collections.OrderedDict()
    seen196 = 0
    for r in rows[:last + 1]:
        k = short(r["Kernel_Name"])
        if not k.startswith("k_"):
            continue
        grid = int(r["Grid_Size_X"]) // 256
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if k.startswith("k_multi"):
            key = ("MULTI", k, None)
        elif k == "k_sum_partials":
            key = ("tensor-sum pass of block MSE (all workloads)", k, None)
        elif "<false" in k:
            key = ("fp32 normal [1024, 4096]", k, c1)
        elif grid == 16384 or k.startswith("k_block_mse"):
            key = ("bf16 Laplace [16384, 8192]", k, c5)
        elif grid in per_matrix and k.startswith("k_quantize<"):
            key = ("Llama-3.2-3B per-matrix launches: " + per_matrix[grid][0], k,
                   per_matrix[grid][1])
        elif grid == 86016:
            key = ("Llama-3.2-3B grouped by K: K=8192 [86016, 8192]", k, l8192)
        elif grid == 98304:
            key = ("MoE w2 [128x4096, 1536]", k, m2)
        elif grid == 196608 and k.startswith("k_quantize<"):
            seen196 += 1
            key = (("Llama-3.2-3B grouped by K: K=3072 [688128, 3072]", k, l3072)
                   if seen196 <= passes else ("MoE w13 [128x3072, 4096]", k, m13))
        elif grid == 196608 and k.startswith("k_dequantize<"):
            key = ("MOEDQ", k, None)
        elif grid == 196608:
            key = ("MoE w13 [128x3072, 4096]", k, m13)
        else:
            key = (f"unattributed (grid {grid})", k, None)
        groups.setdefault(key, []).append(dur)
    multi = groups.pop(("MULTI", "k_multi<true, 0, false>", None), None)
    moedq = groups.pop(("MOEDQ", "k_dequantize<true>", None), None)
    if moedq:  # w13 and w2 alternate
        groups[("MoE w13 [128x3072, 4096]", "k_dequantize<true>", m13)] = moedq[0::2]
        groups[("MoE w2 [128x4096, 1536]", "k_dequantize<true>", m2)] = moedq[1::2]
    out = ["# Kernel trace: the other workloads (`bench.py --suite`)\n", PROFILE_HOW + "\n",
           "```\n" + PROFILE_CMDS["suite"] + "\n```\n", code,
           "Durations are the GPU's own per-dispatch times from the trace (under the profiler the "
           "host-side event figures of the small fp32 case are inflated by per-dispatch overhead; "
           "these are not). Launches are attributed to their workload by grid size; the K=3072 "
           "Llama group and the MoE w13 tensor both run 196,608 workgroups and are told apart by "
           f"dispatch order (the suite runs the Llama launches first, {passes} of each), and the "
           "MoE dequantize launches (both 196,608 workgroups) alternate w13, w2. Per-matrix Llama "
           "launches are grouped by shape. The suite's QSNR pass, which runs after the timed "
           "launches, is left out.\n",
           "| workload | kernel | dispatches | avg us | min us | max us | algorithmic bytes "
           "| GB/s at avg | % of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for (wl, k, n), v in groups.items():
        avg = sum(v) / len(v)
        b = bytes_for(k, n, "<false" in k) if n else None
        out.append(f"| {wl} | `{k}` | {len(v)} | {avg:.2f} | {min(v):.2f} | {max(v):.2f} | "
                   f"{int(b) if b else '-'} | {f'{b / avg / 1e3:.0f}' if b else '-'} | "
                   f"{f'{b / avg / 1e3 / HBM_PEAK_GBS * 100:.1f}' if b else '-'} |")
    if multi:
        per_pass = sum(multi) / passes
        b = (l3072 + l8192) * 2.53125
        out.append(f"| Llama-3.2-3B, the 196 weights as separate tensors: one `mx_quantize_multi` "
                   f"call per pass ({len(multi) // passes} launches) | `k_multi<true, 0, false>` | "
                   f"{len(multi)} | {per_pass:.2f} per pass | {min(multi):.2f} | {max(multi):.2f} "
                   f"| {int(b)} | {b / per_pass / 1e3:.0f} | "
                   f"{b / per_pass / 1e3 / HBM_PEAK_GBS * 100:.1f} |")
    with open(os.path.join(out_dir, "mx_workloads_suite_kernel_trace.md"), "w") as f:
        f.write("\n".join(out) + "\n")


QUALITY_FORMATS = ("mxfp4_ocp", "mxfp4_oas", "mxfp4_oas_bits", "mxfp4_oas_nf", "mxfp8",
                   "nvfp4", "mbs_static")


def suite_quality(dev, chunk_elems: int = 1 << 27):
    """QSNR of every format and MXFP4 scale mode on each workload, from the
    library's outputs (bit-identical to the oracle's by the parity tests).
    MXFP4 error sums come from the one-pass call; the other formats are
    fake-quantized and differenced in fp64. Block formats are row-local, so
    big tensors go through in row chunks; NVFP4's per-tensor factor is taken
    per weight matrix (per expert for MoE) and per activation tensor."""
    import numpy as np
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import workloads

    mx.load_library()

    def sums_rowwise(x2, acc):
        rows_per = max(1, chunk_elems // x2.shape[1])
        for r0 in range(0, x2.shape[0], rows_per):
            xc = x2[r0:r0 + rows_per]
            xd = xc.double()
            ssq = float((xd * xd).sum())
            for mode in mx.MODES:
                _, _, _, _, sums = mx.quantize_fused(xc, mode, want_y=False,
                                                     want_block_mse=False, want_sums=True)
                acc["mxfp4_" + mode][0] += float(sums[0])
                acc["mxfp4_" + mode][1] += float(sums[1])
            for name, fq in (("mxfp8", mx.fakequant_mxfp8), ("mbs_static", mx.fakequant_mbs)):
                d = fq(xc).double() - xd
                acc[name][0] += float((d * d).sum())
                acc[name][1] += ssq
            del xd

    def sums_nvfp4(x2, acc):
        d = mx.fakequant_nvfp4(x2).double() - x2.double()
        acc["nvfp4"][0] += float((d * d).sum())
        acc["nvfp4"][1] += float((x2.double() ** 2).sum())

    rows = []

    def finish(name, acc):
        q = {f: round(10 * np.log10(acc[f][1] / acc[f][0]), 2) for f in QUALITY_FORMATS}
        row = {"workload": name, "op": "qsnr_db", "qsnr_db": q}
        rows.append(row)
        print(json.dumps(row), flush=True)

    new = lambda: {f: [0.0, 0.0] for f in QUALITY_FORMATS}  # noqa: E731
    for name, x in (("fp32 N(0,1) [1024, 4096]", workloads.fp32_normal(1)),
                    ("bf16 Student-t(3) + 20 outlier channels [8192, 4096]",
                     workloads.bf16_student_t_outlier_channels(2)),
                    ("bf16 Laplace + 0.1% outliers [16384, 8192]",
                     workloads.bf16_laplace_sparse_outliers(5))):
        x = x.to(dev)
        acc = new()
        sums_rowwise(x, acc)
        sums_nvfp4(x, acc)
        finish(name, acc)
        del x
    a, b = workloads.llama32_3b_grouped(dev)
    acc = new()
    sums_rowwise(a, acc)
    sums_rowwise(b, acc)
    ra = rb = 0
    for layer in range(workloads.LLAMA32_3B_LAYERS):
        for _, out_f, in_f in workloads.LLAMA32_3B_LINEARS:
            if in_f == 8192:
                sums_nvfp4(b[rb:rb + out_f], acc)
                rb += out_f
            else:
                sums_nvfp4(a[ra:ra + out_f], acc)
                ra += out_f
    finish("Llama-3.2-3B linears x28, bf16 N(0,0.02)", acc)
    del a, b
    torch.cuda.empty_cache()
    w13, w2 = workloads.moe_weights(dev)
    acc = new()
    for w in (w13, w2):
        sums_rowwise(w.reshape(-1, w.shape[-1]), acc)
        for e in range(w.shape[0]):
            sums_nvfp4(w[e], acc)
    finish("MoE w13 + w2, 128 experts, bf16 N(0,0.02)", acc)
    del w13, w2
    torch.cuda.empty_cache()
    return rows


if __name__ == "__main__":
    main()
