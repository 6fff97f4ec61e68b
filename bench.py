"""Benchmark of the MXFP4 hot path on one MI355X.

One step = every operation of the path over one batch of bf16 activations
[8192 tokens, 4096 hidden] (Student-t(3) body, 20 outlier channels x50):
  quantize (OCP scale), quantize (overflow-aware scale), dequantize -> bf16,
  fused fake-quant (OCP), per-block MSE of the OCP result.
Throughput = algorithmic bytes of the step / step time (inputs resident in
HBM). Buffer sets rotate so the working set is >= 1 GiB and the 256 MB
Infinity Cache cannot serve a step from the previous one.

Prints ONE JSON line. --gpus N with N > 1 exits: this path runs on one GPU.
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
}
KERNEL_OF = {"quantize_ocp": "k_quantize<true, 0>", "quantize_oas": "k_quantize<true, 1>",
             "dequantize_bf16": "k_dequantize<true>", "fakequant_ocp": "k_fakequant<true, 0>",
             "block_mse": "k_block_mse<true, true>"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mx_bf16_8192x4096_hbm_traffic.md")
KERNEL_SRC = os.path.join(ROOT, "microscaling_fp4_block_mx_amd", "csrc", "mx_kernels.hip")


def measured_traffic(op):
    """HBM bytes per launch of op's kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, or None if that summary was taken on a
    different kernel source than the one built here."""
    import hashlib
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
        h = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    if ("source_sha256_prefix " + h) not in lines:
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
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build measures one GPU only; every MX block is independent, "
              "so the path shards by rows with no exchange (see DESIGN.md). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
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
        cpu = cpu_baseline(x_host, args.cpu_seconds)

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
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(x_host, target_s):
    """The oracle as it stands, on the host cores, over a bounded sample of
    the same workload (leading rows), running the same step."""
    import numpy as np

    import oracle
    import workloads

    oracle.build(force=not os.path.exists(os.path.join(ROOT, "oracle", "libmxref.so")))
    cores = max(1, len(os.sched_getaffinity(0)))
    xs_full = workloads.to_bf16_bits(x_host)
    rows = 256
    xs = np.ascontiguousarray(xs_full[:rows])
    n = xs.size
    bytes_step = sum(BYTES_PER_ELEM[o] for o in OPS) * n
    done, t0 = 0, time.perf_counter()
    while True:
        c, s = oracle.quantize(xs, "ocp", threads=cores)
        oracle.quantize(xs, "oas", threads=cores)
        oracle.dequantize(c, s, "bf16", threads=cores)
        oracle.fakequant(xs, "ocp", threads=cores)
        oracle.block_mse(xs, c, s, threads=cores)
        done += 1
        el = time.perf_counter() - t0
        if el >= target_s:
            break
        if done == 1:  # size the sample so the loop lands near the target
            rows_next = int(min(xs_full.shape[0], rows * max(1.0, target_s / max(el, 1e-3) / 3)))
            if rows_next > rows:
                rows = rows_next
                xs = np.ascontiguousarray(xs_full[:rows])
                n = xs.size
                bytes_step = sum(BYTES_PER_ELEM[o] for o in OPS) * n
                done, t0 = 0, time.perf_counter()
    gbs = done * bytes_step / el / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} step(s) over the first {rows} rows x 4096 of the same tensor "
                      f"({el:.1f} s)"}


if __name__ == "__main__":
    main()
