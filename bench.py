"""Benchmark of the MXFP4 hot path on one MI355X.

One step = every operation of the path over one batch of the largest
workload, the Llama-3.2-3B-shaped linear weights: 28 layers x {q, k, v, o,
gate, up, down}, bf16 N(0, 0.02), the 196 matrices end to end in one buffer
(2,818,572,288 elements, 5.6 GB), each matrix quantized along its input
dimension. The operations, one launch each over the whole buffer:
  quantize (OCP scale), quantize (overflow-aware scale), dequantize -> bf16,
  fused fake-quant (OCP), per-block MSE of the OCP result (+ its tensor sums).
Throughput = algorithmic bytes of the step / step time, inputs resident in
HBM; the 5.6 GB input is 22x the 256 MB Infinity Cache, so no step is served
from the previous one.

Beside the step, the same run times (rotated buffer sets of >= 1.5 GiB, so
cold): fake-quant of bf16 activations [8192, 4096] (Student-t(3), 20
outlier channels x50) and the other formats and modes on that tensor;
quantize (OCP and overflow-aware) of bf16 activations [16384, 8192]
(Laplace + 0.1 % outliers); and reference streaming kernels with the
quantize kernel's tiling on the step's buffer (a quantize-shaped skeleton
with no arithmetic, a copy, a read and a write) that show what HBM allows.

Prints ONE JSON line. --gpus N with N > 1 exits: this path runs on one GPU.
--only step|beside runs one part alone (for profiling).

--suite instead times each operation on the other workloads alone (fp32
normal [1024, 4096]; the Llama-3.2-3B-shaped linear stack, per matrix, as one
multi-tensor call, grouped by K and as one buffer; the 128-expert MoE
weights; bf16 Laplace [16384, 8192] with sparse outliers), with per-launch
HIP events (median, p10, p90), warm (cache-resident) and cold (rotated)
figures where the tensor fits the cache, and for the small fp32 case the
host-side single-launch latency, the per-launch time inside a replayed HIP
graph, an empty launch and a copy of the same size. It prints one JSON line
per measurement and a markdown table.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import re
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "MXFP4 quantize/fake-quant GB/s (bf16 in) and % of HBM peak, 1× MI355X"
WORKLOAD = ("Llama-3.2-3B-shaped linear weights, bf16 N(0,0.02), 28 layers x {q 3072x3072, "
            "k 1024x3072, v 1024x3072, o 3072x3072, gate 8192x3072, up 8192x3072, down "
            "3072x8192}: the 196 matrices end to end in one buffer, each quantized along its "
            "input dimension (seed 3)")
STEP_K = 3072            # the buffer is launched as [n / 3072, 3072]; blocks never straddle a matrix
STEP_ELEMS = 2818572288  # 28 layers x 100,663,296
C2_WORKLOAD = ("bf16 activations 8192 tokens x 4096 hidden, Student-t(nu=3), 20 outlier "
               "channels x50 (seed 2)")
C2_ELEMS = 8192 * 4096
C5_WORKLOAD = "bf16 activations 16384 x 8192, Laplace(0,1), 0.1% outliers +-U(20,200) (seed 5)"
C5_ELEMS = 16384 * 8192

# algorithmic bytes per element (bf16 input): what each op must move
BYTES_PER_ELEM = {
    "quantize_ocp": 2 + 0.5 + 1 / 32,      # x in, codes + scales out
    "quantize_oas": 2 + 0.5 + 1 / 32,
    "dequantize_bf16": 0.5 + 1 / 32 + 2,   # codes + scales in, y out
    "fakequant_ocp": 2 + 2,                # x in, y out
    "block_mse": 2 + 0.5 + 1 / 32 + 4 / 32,  # x, codes, scales in; fp32/block out
}
OPS = list(BYTES_PER_ELEM)
# measured beside the step on the Student-t activations: fake-quant (OCP),
# the page-faithful overflow-aware variants, fake-quant in the
# overflow-aware modes, and the other formats
EXTRA_BYTES_PER_ELEM = {
    "fakequant_ocp": 4.0,
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
    # dequantize and block MSE fused; x read once)
    "quantize_fused": 2 + 0.5 + 1 / 32 + 2 + 4 / 32,
    # fused fake-quant of the comparators (NVFP4 reads x twice)
    "fakequant_nvfp4": 2 + 2 + 2,
    "fakequant_mbs": 2 + 2,
}
# on the Laplace activations
C5_BYTES_PER_ELEM = {"quantize_ocp": 2 + 0.5 + 1 / 32, "quantize_oas": 2 + 0.5 + 1 / 32}
# reference kernels (bench_ceiling.hip) on the step's buffer
CEILING_BYTES_PER_ELEM = {"quantize_shape": 2 + 0.5 + 1 / 32, "dequantize_shape": 0.5 + 1 / 32 + 2,
                          "block_mse_shape": 2 + 0.5 + 1 / 32 + 1 / 8,
                          "copy": 4.0, "read": 2.0,
                          "write": 2.0}
# Kernel family of each op (the kernels' template argument U is the number of
# 8-element items per thread, which the library picks by size; the quantize,
# fake-quant and dequantize kernels take the threads per workgroup after it)
KERNEL_OF = {"quantize_ocp": "k_quantize<true, 0, U>", "quantize_oas": "k_quantize<true, 1, U>",
             "dequantize_bf16": "k_dequantize<true, U>",
             "fakequant_ocp": "k_fakequant<true, 0, U>", "block_mse": "k_block_mse<true, true, U>"}
# kernels with items-per-thread as their last template argument (or, for
# NT_KERNELS, U then the threads per workgroup NT), and one tile (NT threads
# x U items x 8 elements; NT = 256 where not given) per workgroup at these sizes
NT_KERNELS = ("k_quantize", "k_fakequant", "k_dequantize", "k_quantize8", "k_dequantize8",
              "k_fakequant8", "k_quantize_mbs", "k_dequantize_mbs", "k_quantize_nv_big")
U_KERNELS = NT_KERNELS + ("k_block_mse", "k_quantize_pair")
ITEM_ELEMS = {"k_quantize_pair": 16}  # elements per item where not 8 (two lanes per block)
FUSED_ITEMS = 2  # items per thread of k_quantize_fused
PROFILE_STEM = {"step": "mx_llama32_3b_linears",
                "beside": "mx_student_t_8192x4096_laplace_16384x8192"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", PROFILE_STEM["step"] + "_hbm_traffic.md")
# launches per timing of the multi-GB suite workloads: warm-up, then timed
# twice (per-launch events, then back to back)
BIG_TIMED, BIG_WARM = 20, 3
KERNEL_SRCS = (os.path.join(ROOT, "microscaling_fp4_block_mx_amd", "csrc", "mx_kernels.hip"),
               os.path.join(ROOT, "microscaling_fp4_block_mx_amd", "csrc", "mx_internal.h"))
CEILING_SRC = os.path.join(ROOT, "bench_ceiling.hip")
CEILING_LIB = os.path.join(ROOT, "libmxceiling.so")


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


def _u_nt(k: str):
    """(name, leading template arguments, U, NT) of a kernel in U_KERNELS,
    else None."""
    m = re.fullmatch(r"(k_\w+)<(.*), (\d+), (\d+)>", k)
    if m and m.group(1) in NT_KERNELS:
        return m.group(1), m.group(2), int(m.group(3)), int(m.group(4))
    m = re.fullmatch(r"(k_\w+)<(.*), (\d+)>", k)
    if m and m.group(1) in U_KERNELS and m.group(1) not in NT_KERNELS:
        return m.group(1), m.group(2), int(m.group(3)), 256
    return None


def kernel_family(k: str) -> str:
    """k_quantize<true, 0, 2, 128> -> k_quantize<true, 0, U>,
    k_block_mse<true, true, 2> -> k_block_mse<true, true, U>; other names
    as they are."""
    p = _u_nt(k)
    return f"{p[0]}<{p[1]}, U>" if p else k


def items_per_thread(k: str):
    """U of a kernel whose grid is one tile per workgroup, else None."""
    p = _u_nt(k)
    if p:
        return p[2]
    if k.startswith("k_quantize_fused<"):
        return FUSED_ITEMS
    return None


def threads_per_group(k: str) -> int:
    """Threads per workgroup of kernel k (256 unless its name gives NT)."""
    p = _u_nt(k)
    return p[3] if p else 256


def _traffic_lines(path):
    """{kernel: HBM bytes per launch} from a committed rocprofv3 traffic
    summary, or None if it was taken on different kernel code than the one
    built here."""
    try:
        lines = open(path).read().splitlines()
        h = kernel_code_hash()
    except OSError:
        return None
    if ("kernel_code_sha256_prefix " + h) not in lines:
        return None
    out = {}
    for ln in lines:
        f = ln.split(" ")
        if f[0] == "traffic_bytes":
            out[" ".join(f[1:-1])] = int(f[-1])
    return out


def measured_traffic(op, path=None, family=None):
    """(kernel, HBM bytes per launch) of op's kernel (or of the kernel family
    given) from the committed FETCH_SIZE/WRITE_SIZE summary of the step (or
    of path), or None while that summary belongs to other kernel code."""
    t = _traffic_lines(path or TRAFFIC_FILE)
    if t is None:
        return None
    fam = family or KERNEL_OF[op]
    for k, b in t.items():
        if kernel_family(k) == fam:
            return k, b
    return None


# Kernel families of the ops timed beside the step (one instantiation each
# there), for their measured traffic; NVFP4 quantize is two kernels, and a
# tuple lists the kernels the library chooses between by tensor size.
BESIDE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", PROFILE_STEM["beside"] + "_hbm_traffic.md")
BESIDE_KERNELS = {
    "fakequant_ocp": ["k_fakequant<true, 0, U>"], "fakequant_oas": ["k_fakequant<true, 1, U>"],
    "fakequant_oas_nf": ["k_fakequant<true, 3, U>"],
    "quantize_oas_bits": ["k_quantize<true, 2, U>"],
    "quantize_oas_nf": [("k_quantize_pair<3, U>", "k_quantize<true, 3, U>")],
    "quantize_mxfp8": ["k_quantize8<true, U>"], "dequantize_mxfp8_bf16": ["k_dequantize8<true, U>"],
    "fakequant_mxfp8": ["k_fakequant8<true, U>"],
    "quantize_nvfp4": ["k_absmax_partials<true>", "k_quantize_nv<true, false>"],
    "dequantize_nvfp4_bf16": ["k_dequantize_nv<true>"],
    "fakequant_nvfp4": ["k_absmax_partials<true>", "k_quantize_nv<true, true>"],
    "quantize_mbs": ["k_quantize_mbs<true, false, U>"],
    "dequantize_mbs_bf16": ["k_dequantize_mbs<true, U>"],
    "fakequant_mbs": ["k_quantize_mbs<true, true, U>"],
    "quantize_fused": ["k_quantize_fused<true, 0, true>"],
    "reference_copy": ["k_ceiling_copy"],
    "quantize_ocp": ["k_quantize<true, 0, U>"], "quantize_oas": ["k_quantize<true, 1, U>"],
}


def beside_roofline(op, row):
    """Roofline fields of one op timed beside the step: its achieved rate
    against the 8 TB/s peak, and the HBM bytes its kernels moved per call
    in the committed profile of this part (None while stale)."""
    traffic = 0
    for fams in BESIDE_KERNELS[op]:  # a tuple: the kernels the library may pick by size
        mt = None
        for fam in (fams if isinstance(fams, tuple) else (fams,)):
            mt = mt or measured_traffic(op, BESIDE_TRAFFIC_FILE, fam)
        if mt is None:
            traffic = None
            break
        traffic += mt[1]
    return {"bound": "hbm", "achieved": row["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": row["frac_hbm"], "traffic": traffic, "bytes_per_launch": row["bytes"],
            "avg_launch_us": row["us"]}


def build_ceiling(verbose: bool = False) -> str:
    """Compile the reference streaming kernels (bench_ceiling.hip) for gfx950
    into libmxceiling.so beside this file."""
    from microscaling_fp4_block_mx_amd import build as mxbuild
    tmp = CEILING_LIB + ".tmp"
    cmd = [mxbuild.hipcc(), f"--offload-arch={mxbuild.ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-command-line-argument", "-o", tmp, CEILING_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libmxceiling.so")
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


def ceiling_lib() -> ctypes.CDLL:
    if not os.path.exists(CEILING_LIB):
        build_ceiling()
    lib = ctypes.CDLL(CEILING_LIB)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.mxc_quantize_shape.argtypes = [p, i64, p, p, p]
    lib.mxc_dequantize_shape.argtypes = [p, p, i64, p, p]
    lib.mxc_block_mse_shape.argtypes = [p, p, p, i64, p, p]
    lib.mxc_copy.argtypes = [p, p, i64, p]
    lib.mxc_read.argtypes = [p, i64, p, p]
    lib.mxc_write.argtypes = [p, i64, p]
    lib.mxc_empty.argtypes = [p]
    for f in ("mxc_quantize_shape", "mxc_dequantize_shape", "mxc_block_mse_shape", "mxc_copy",
              "mxc_read", "mxc_write", "mxc_empty"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate-gib", type=float, default=1.5,
                    help="minimum working set across rotated buffer sets (the activations "
                         "beside the step)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=("step", "beside"),
                    help="run only the step (with its reference kernels) or only the "
                         "measurements beside it; no quality or CPU baseline")
    ap.add_argument("--suite", action="store_true",
                    help="time the operations on the other workloads instead of the step")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write the profiles/ summaries from the rocprofv3 csv files in DIR "
                         "(trace_*, fetch_*, write_*, sq_*, suite_*) and exit; needs no GPU")
    return ap.parse_args()


def _ok(mx, st):
    if st != mx.MX_OK:
        raise RuntimeError(mx.mx_status_string(st) + " " + mx.mx_last_error_detail())


def _timed_launches(fn, m, stream):
    """Mean time (ms) of m calls of fn(i) issued back to back between two
    events on `stream`."""
    import torch
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for i in range(m):
        fn(i)
    a1.record(stream)
    torch.cuda.synchronize()
    return a0.elapsed_time(a1) / m


def _row(nbytes, ms, **extra):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"us": round(ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": int(nbytes), **extra}


def run_step(args, dev, stream):
    """The step on the Llama-3.2-3B linear buffer, each op alone, and the
    reference kernels on the same buffer."""
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import workloads

    sh = stream.cuda_stream
    arena, _ = workloads.llama32_3b_arena(dev)
    x = arena.view(-1, STEP_K)
    R_, K_ = x.shape
    n = x.numel()
    assert n == STEP_ELEMS
    b = dict(c_ocp=torch.empty((R_, K_ // 2), dtype=torch.uint8, device=dev),
             s_ocp=torch.empty((R_, K_ // 32), dtype=torch.uint8, device=dev),
             c_oas=torch.empty((R_, K_ // 2), dtype=torch.uint8, device=dev),
             s_oas=torch.empty((R_, K_ // 32), dtype=torch.uint8, device=dev),
             y_dq=torch.empty_like(x), y_fq=torch.empty_like(x),
             bm=torch.empty((R_, K_ // 32), dtype=torch.float32, device=dev))
    sums = torch.empty(2, dtype=torch.float64, device=dev)
    ws_bytes = mx.mx_block_mse_workspace_size(R_, K_)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    xp = x.data_ptr()

    def run(op):
        if op == "quantize_ocp":
            st = mx.mx_quantize(xp, mx.MX_BF16, R_, K_, mx.MX_SCALE_OCP, b["c_ocp"].data_ptr(),
                                b["s_ocp"].data_ptr(), sh)
        elif op == "quantize_oas":
            st = mx.mx_quantize(xp, mx.MX_BF16, R_, K_, mx.MX_SCALE_OAS, b["c_oas"].data_ptr(),
                                b["s_oas"].data_ptr(), sh)
        elif op == "dequantize_bf16":
            st = mx.mx_dequantize(b["c_ocp"].data_ptr(), b["s_ocp"].data_ptr(), R_, K_,
                                  mx.MX_BF16, b["y_dq"].data_ptr(), sh)
        elif op == "fakequant_ocp":
            st = mx.mx_fakequant(xp, mx.MX_BF16, R_, K_, mx.MX_SCALE_OCP, b["y_fq"].data_ptr(),
                                 sh)
        else:
            st = mx.mx_block_mse(xp, mx.MX_BF16, b["c_ocp"].data_ptr(), b["s_ocp"].data_ptr(),
                                 R_, K_, b["bm"].data_ptr(), sums.data_ptr(), ws.data_ptr(),
                                 ws_bytes, sh)
        _ok(mx, st)

    def step():
        for op in OPS:
            run(op)

    for _ in range(max(1, args.warmup)):  # also produces the codes dequantize / block MSE read
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps between two events on the launch stream
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = e0.elapsed_time(e1) / K

    # each op alone: m launches back to back between two events on the same
    # stream (the average launch duration of its kernel; block MSE is its
    # kernel plus the one-workgroup tensor-sum kernel)
    m = max(K, 10)
    op_ms = {op: _timed_launches(lambda i, op=op: run(op), m, stream) for op in OPS}

    # reference kernels with the quantize kernel's tiling, on the same buffer
    cl = ceiling_lib()
    nit = n // 8
    sink = torch.empty(-(-nit // 256), dtype=torch.int32, device=dev)  # a word per workgroup
    ceil_fn = {
        "quantize_shape": lambda i: cl.mxc_quantize_shape(xp, nit, b["c_oas"].data_ptr(),
                                                          b["s_oas"].data_ptr(), sh),
        "dequantize_shape": lambda i: cl.mxc_dequantize_shape(b["c_ocp"].data_ptr(),
                                                              b["s_ocp"].data_ptr(), nit,
                                                              b["y_dq"].data_ptr(), sh),
        "block_mse_shape": lambda i: cl.mxc_block_mse_shape(xp, b["c_ocp"].data_ptr(),
                                                            b["s_ocp"].data_ptr(), nit,
                                                            b["bm"].data_ptr(), sh),
        "copy": lambda i: cl.mxc_copy(xp, b["y_fq"].data_ptr(), nit, sh),
        "read": lambda i: cl.mxc_read(xp, nit, sink.data_ptr(), sh),
        "write": lambda i: cl.mxc_write(b["y_fq"].data_ptr(), nit, sh),
    }
    ceil_ms = {}
    for name, fn in ceil_fn.items():
        fn(0)
        torch.cuda.synchronize()
        ceil_ms[name] = _timed_launches(fn, m, stream)
    ceilings = {name: _row(CEILING_BYTES_PER_ELEM[name] * n, ceil_ms[name]) for name in ceil_fn}
    ceilings["quantize_ocp_vs_quantize_shape"] = round(ceil_ms["quantize_shape"]
                                                       / op_ms["quantize_ocp"], 4)
    ceilings["dequantize_bf16_vs_dequantize_shape"] = round(ceil_ms["dequantize_shape"]
                                                            / op_ms["dequantize_bf16"], 4)
    ceilings["block_mse_vs_block_mse_shape"] = round(ceil_ms["block_mse_shape"]
                                                     / op_ms["block_mse"], 4)
    ceilings["fakequant_ocp_vs_copy"] = round(ceil_ms["copy"] / op_ms["fakequant_ocp"], 4)
    ceilings["kernels"] = ("bench_ceiling.hip (k_ceiling_*): one 16-byte item per thread, one tile "
                           "per workgroup, no format arithmetic")

    bytes_op = {op: BYTES_PER_ELEM[op] * n for op in OPS}
    bytes_step = sum(bytes_op.values())
    breakdown = {op: _row(bytes_op[op], op_ms[op], elements_per_s=round(n / (op_ms[op] * 1e-3), 1))
                 for op in OPS}
    dom = max(OPS, key=lambda o: op_ms[o])
    dom_gbs = bytes_op[dom] / (op_ms[dom] * 1e-3) / 1e9
    mt = measured_traffic(dom)
    if mt is None:
        print(f"bench.py: roofline.traffic is null: {os.path.relpath(TRAFFIC_FILE, ROOT)} was "
              "taken on other kernel code (python bench.py --summarize-profiles DIR rewrites it)",
              file=sys.stderr)
    roofline = {"bound": "hbm", "kernel": mt[0] if mt else KERNEL_OF[dom], "op": dom,
                "achieved": round(dom_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                "traffic": mt[1] if mt else None,
                "bytes_per_launch": int(bytes_op[dom]),
                "avg_launch_us": round(op_ms[dom] * 1e3, 2)}

    # quality of the step's outputs (outside the timed region)
    run("block_mse")
    torch.cuda.synchronize()
    sse, ssq = sums.tolist()
    quality = {"mxfp4_ocp": {"mse": sse / n, "qsnr_db": round(10 * math.log10(ssq / sse), 4)}}
    run("quantize_oas")  # the reference kernels wrote over the overflow-aware codes
    _ok(mx, mx.mx_block_mse(xp, mx.MX_BF16, b["c_oas"].data_ptr(), b["s_oas"].data_ptr(), R_, K_,
                            None, sums.data_ptr(), ws.data_ptr(), ws_bytes, sh))
    torch.cuda.synchronize()
    sse2, ssq2 = sums.tolist()
    quality["mxfp4_oas"] = {"mse": sse2 / n,
                            "qsnr_db": round(10 * math.log10(ssq2 / sse2), 4)}
    del b, ws, sink
    torch.cuda.empty_cache()
    # block MSE's summing launches: a second level when the workspace holds
    # more than one pair per 4096 elements (16 bytes per 8192 partials)
    sum_launches = 1 + int(ws_bytes // 16 > -(-n // 4096))
    return dict(x=x, n=n, ms_per_step=ms_per_step, wall=wall, bytes_step=bytes_step,
                sum_launches=sum_launches,
                breakdown=breakdown, roofline=roofline, ceilings=ceilings, quality=quality,
                copy_us=ceil_ms["copy"] * 1e3)


def run_beside(args, dev, stream):
    """Fake-quant and the other formats on the Student-t activations, and
    quantize (both modes) on the Laplace activations; rotated buffer sets,
    each op m launches back to back."""
    import numpy as np
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import workloads

    sh = stream.cuda_stream
    K = args.steps
    out = {}

    # -- Student-t activations [8192, 4096]
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
            c=torch.empty((R_, K_ // 2), dtype=torch.uint8, device=dev),
            s=torch.empty((R_, K_ // 32), dtype=torch.uint8, device=dev),
            y_dq=torch.empty_like(x0), y_fq=torch.empty_like(x0),
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

    def run(op, b):
        xp = b["x"].data_ptr()
        if op in ("fakequant_ocp", "fakequant_oas", "fakequant_oas_nf"):
            mode = {"fakequant_ocp": mx.MX_SCALE_OCP, "fakequant_oas": mx.MX_SCALE_OAS,
                    "fakequant_oas_nf": mx.MX_SCALE_OAS_NF}[op]
            st = mx.mx_fakequant(xp, mx.MX_BF16, R_, K_, mode, b["y_fq"].data_ptr(), sh)
        elif op in ("quantize_oas_bits", "quantize_oas_nf"):
            mode = mx.MX_SCALE_OAS_BITS if op.endswith("bits") else mx.MX_SCALE_OAS_NF
            st = mx.mx_quantize(xp, mx.MX_BF16, R_, K_, mode, b["c"].data_ptr(),
                                b["s"].data_ptr(), sh)
        elif op == "quantize_mxfp8":
            st = mx.mx_quantize_mxfp8(xp, mx.MX_BF16, R_, K_, b["c8"].data_ptr(),
                                      b["s8"].data_ptr(), sh)
        elif op == "dequantize_mxfp8_bf16":
            st = mx.mx_dequantize_mxfp8(b["c8"].data_ptr(), b["s8"].data_ptr(), R_, K_, mx.MX_BF16,
                                        b["y_dq"].data_ptr(), sh)
        elif op == "fakequant_mxfp8":
            st = mx.mx_fakequant_mxfp8(xp, mx.MX_BF16, R_, K_, b["y_fq"].data_ptr(), sh)
        elif op == "quantize_nvfp4":
            st = mx.mx_quantize_nvfp4(xp, mx.MX_BF16, R_, K_, b["c"].data_ptr(),
                                      b["bnv"].data_ptr(), b["tnv"].data_ptr(), wsnv.data_ptr(),
                                      wsnv_bytes, sh)
        elif op == "dequantize_nvfp4_bf16":
            st = mx.mx_dequantize_nvfp4(b["c"].data_ptr(), b["bnv"].data_ptr(),
                                        b["tnv"].data_ptr(), R_, K_, mx.MX_BF16,
                                        b["y_dq"].data_ptr(), sh)
        elif op == "quantize_mbs":  # codes land in c; dequantize_mbs_bf16 runs next
            st = mx.mx_quantize_mbs(xp, mx.MX_BF16, R_, K_, b["c"].data_ptr(),
                                    b["smb"].data_ptr(), b["mmb"].data_ptr(), sh)
        elif op == "dequantize_mbs_bf16":
            st = mx.mx_dequantize_mbs(b["c"].data_ptr(), b["smb"].data_ptr(),
                                      b["mmb"].data_ptr(), R_, K_, mx.MX_BF16,
                                      b["y_dq"].data_ptr(), sh)
        elif op == "quantize_fused":
            st = mx.mx_quantize_fused(xp, mx.MX_BF16, R_, K_, mx.MX_SCALE_OCP,
                                      b["c"].data_ptr(), b["s"].data_ptr(),
                                      b["y_fq"].data_ptr(), b["bm"].data_ptr(), sums.data_ptr(),
                                      ws.data_ptr(), ws_bytes, sh)
        elif op == "fakequant_nvfp4":
            st = mx.mx_fakequant_nvfp4(xp, mx.MX_BF16, R_, K_, b["y_fq"].data_ptr(),
                                       wsnv.data_ptr(), wsnv_bytes, sh)
        elif op == "fakequant_mbs":
            st = mx.mx_fakequant_mbs(xp, mx.MX_BF16, R_, K_, b["y_fq"].data_ptr(), sh)
        else:
            raise KeyError(op)
        _ok(mx, st)

    m = max(K, 2 * n_sets)
    for op, bpe in EXTRA_BYTES_PER_ELEM.items():
        for i in range(n_sets):  # warm the code paths; produce the codes the decoders read
            run(op, sets[i])
        torch.cuda.synchronize()
        ms = _timed_launches(lambda i, op=op: run(op, sets[i % n_sets]), m, stream)
        row = _row(bpe * n, ms, workload=C2_WORKLOAD, cache=f"cold ({n_sets} rotated sets)")
        row["roofline"] = beside_roofline(op, row)
        out[f"{op} [8192, 4096]"] = row
    # the reference copy of the same tensor, timed the same way (and the
    # counter calibration kernel of this part's profiles)
    cl = ceiling_lib()
    ms = _timed_launches(lambda i: cl.mxc_copy(sets[i % n_sets]["x"].data_ptr(),
                                               sets[i % n_sets]["y_fq"].data_ptr(), n // 8, sh),
                         m, stream)
    row = _row(4.0 * n, ms, workload=C2_WORKLOAD, cache=f"cold ({n_sets} rotated sets)")
    row["roofline"] = beside_roofline("reference_copy", row)
    out["reference_copy [8192, 4096]"] = row
    del sets, ws, wsnv
    torch.cuda.empty_cache()

    # -- Laplace activations [16384, 8192]: quantize in both modes
    x5 = workloads.bf16_laplace_sparse_outliers(5).to(dev)
    R5, K5 = x5.shape
    n5 = x5.numel()
    per_set = n5 * (2 + 0.5 + 1 / 32)
    n_sets = max(2, int(np.ceil(args.rotate_gib * 2 ** 30 / per_set)))
    sets = [dict(x=x5.clone(), c=torch.empty((R5, K5 // 2), dtype=torch.uint8, device=dev),
                 s=torch.empty((R5, K5 // 32), dtype=torch.uint8, device=dev))
            for _ in range(n_sets)]
    del x5
    m = max(K, 2 * n_sets)
    for op, mode in (("quantize_ocp", mx.MX_SCALE_OCP), ("quantize_oas", mx.MX_SCALE_OAS)):
        def q5(i, mode=mode):
            b = sets[i % n_sets]
            _ok(mx, mx.mx_quantize(b["x"].data_ptr(), mx.MX_BF16, R5, K5, mode,
                                   b["c"].data_ptr(), b["s"].data_ptr(), sh))
        for i in range(n_sets):
            q5(i)
        torch.cuda.synchronize()
        row = _row(C5_BYTES_PER_ELEM[op] * n5, _timed_launches(q5, m, stream),
                   workload=C5_WORKLOAD, cache=f"cold ({n_sets} rotated sets)")
        row["roofline"] = beside_roofline(op, row)
        out[f"{op} [16384, 8192]"] = row
    del sets
    torch.cuda.empty_cache()
    return out


def quality_beside(dev):
    """Tensor MSE and QSNR of every format and MXFP4 mode on the Student-t
    activations, and of both step modes on the Laplace activations."""
    import numpy as np
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import workloads

    q = {}
    x = workloads.bf16_student_t_outlier_channels(2).to(dev)
    n = x.numel()
    for mode in mx.MODES:
        c, sc = mx.quantize(x, mode)
        _, sums = mx.block_mse(x, c, sc, per_block=False)
        sse, ssq = sums.tolist()
        q["mxfp4_" + mode] = {"mse": sse / n, "qsnr_db": round(10 * np.log10(ssq / sse), 4)}
    xf = x.float()
    e = float((xf.double() ** 2).sum())
    for name, y in (("mxfp8", mx.fakequant_mxfp8(x).float()),
                    ("nvfp4", mx.dequantize_nvfp4(*mx.quantize_nvfp4(x), torch.float32)),
                    ("mbs_static", mx.dequantize_mbs(*mx.quantize_mbs(x), torch.float32))):
        sse = float(((xf - y).double() ** 2).sum())
        q[name] = {"mse": sse / n, "qsnr_db": round(10 * np.log10(e / sse), 4)}
    out = {"student_t_8192x4096": q}
    x5 = workloads.bf16_laplace_sparse_outliers(5).to(dev)
    q5 = {}
    for mode in ("ocp", "oas"):
        c, sc = mx.quantize(x5, mode)
        _, sums = mx.block_mse(x5, c, sc, per_block=False)
        sse, ssq = sums.tolist()
        q5["mxfp4_" + mode] = {"mse": sse / x5.numel(), "qsnr_db": round(10 * np.log10(ssq / sse), 4)}
    out["laplace_16384x8192"] = q5
    return out


def main():
    args = parse()
    if args.summarize_profiles:
        return summarize_profiles(args.summarize_profiles)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark measures one GPU only; every MX block is independent, "
              "so the path shards by rows with no exchange. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import microscaling_fp4_block_mx_amd as mx

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.suite:
        return suite(args, dev)
    torch.cuda.set_device(dev)
    mx.load_library()
    stream = torch.cuda.current_stream(dev)

    step = run_step(args, dev, stream) if args.only in (None, "step") else None
    beside = run_beside(args, dev, stream) if args.only in (None, "beside") else None
    quality = cpu = None
    if args.only is None:
        quality = {"llama32_3b_linears": step["quality"], **quality_beside(dev)}
        if not args.no_cpu_baseline:
            cpu = cpu_baseline(step["x"], args.cpu_seconds)

    out = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    if step:
        n = step["n"]
        out.update({
            "value": round(step["bytes_step"] / (step["ms_per_step"] * 1e-3) / 1e9, 1),
            "ms_per_step": round(step["ms_per_step"], 5),
            "config": {"workload": WORKLOAD, "rows": n // STEP_K, "k": STEP_K, "elements": n,
                       "step": OPS, "launches_per_step": len(OPS) + step["sum_launches"],
                       "bytes_per_step": int(step["bytes_step"]),
                       "elements_per_s": round(n / (step["ms_per_step"] * 1e-3), 1),
                       "wall_s_timed": round(step["wall"], 4),
                       "cache": "input 22x the 256 MB Infinity Cache; no rotation needed"},
            "breakdown": step["breakdown"],
            "ceilings": step["ceilings"],
            "roofline": step["roofline"],
        })
    if beside:
        out["beside_the_step"] = beside
    if quality:
        out["quality"] = quality
    if cpu:
        out["cpu_baseline"] = cpu
    out["env"] = {"device": torch.cuda.get_device_name(dev), "torch": torch.__version__,
                  "hip": torch.version.hip}
    print(json.dumps(out), flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x_dev, target_s):
    """The oracle as it stands, on the host cores, over a bounded sample of
    the step's buffer (its leading rows of 3072, i.e. the first matrices),
    running the same step: first on every core, then on one thread over a
    smaller sample. The first sample's oracle outputs are also compared with
    the library's on the same rows (codes and scales of both modes,
    dequantize, fake-quant bit for bit; block MSE and tensor sums to a
    relative 1e-6)."""
    import numpy as np
    import torch

    import microscaling_fp4_block_mx_amd as mx
    import oracle
    import workloads

    oracle.build(force=not os.path.exists(os.path.join(ROOT, "oracle", "libmxref.so")))
    cores = max(1, len(os.sched_getaffinity(0)))
    k = x_dev.shape[1]
    max_rows = min(x_dev.shape[0], 131072)  # at most 403 M elements on the host
    cache = {}

    def host_rows(rows):
        if cache.get("rows", 0) < rows:
            cache["x"] = workloads.to_bf16_bits(x_dev[:rows])
            cache["rows"] = rows
        return np.ascontiguousarray(cache["x"][:rows])

    def step(xs, threads):
        c, s = oracle.quantize(xs, "ocp", threads=threads)
        c2, s2 = oracle.quantize(xs, "oas", threads=threads)
        y = oracle.dequantize(c, s, "bf16", threads=threads)
        f = oracle.fakequant(xs, "ocp", threads=threads)
        bm = oracle.block_mse(xs, c, s, threads=threads, with_energy=True)
        return c, s, c2, s2, y, f, bm

    def timed(rows, threads, budget):
        xs = host_rows(rows)
        done, t0, out = 0, time.perf_counter(), None
        while True:
            out = step(xs, threads)
            done += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return rows, done, el, out
            if done == 1 and rows < max_rows:  # size the sample to land near the budget
                grow = int(min(max_rows, rows * max(1.0, budget / max(el, 1e-3) / 3)))
                if grow > rows:
                    rows = grow
                    xs = host_rows(rows)
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
            "sample": f"{done} step(s) over the first {rows} rows x {k} of the same buffer "
                      f"({rows * k} elements, the first matrices; {el:.1f} s, {cores} threads)",
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
    # the floor of a launch of this size: an empty kernel, and a copy of the
    # fp32 input with the quantize kernel's tiling (16 MiB read + 16 MiB written)
    cl = ceiling_lib()
    report(W1, "empty launch (one workgroup)", 0, _launch_stats(lambda i: cl.mxc_empty(sh),
                                                                 n_timed, n_warm, stream),
           cache="-")
    report(W1, "reference copy of the fp32 input (bench_ceiling.hip)", 8 * n,
           _launch_stats(lambda i: cl.mxc_copy(sets[i % len(sets)]["x"].data_ptr(),
                                               sets[i % len(sets)]["y"].data_ptr(), n // 4, sh),
                         n_timed, n_warm, stream), cache=f"cold ({len(sets)} rotated sets)")
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

    # QAT's weight pass: every weight fake-quantized, into its own output
    ya, yb = torch.empty_like(a), torch.empty_like(b)
    fdescs = (mx.MxTensor * len(mats))()
    for i, (t, c, s_, r0, rows, k) in enumerate(mats):
        y = ya if t is a else yb
        fdescs[i] = mx.MxTensor(t[r0].data_ptr(), y[r0].data_ptr(), None, None, rows, k)

    def multi_fq(_):
        ok(mx.mx_fakequant_multi(fdescs, len(mats), mx.MX_BF16, mx.MX_SCALE_OCP, sh))

    report(WL, "quantize_ocp (196 per-matrix launches)", bytes_q,
           _launch_stats(per_matrix, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WL, "quantize_ocp (196 matrices, one multi-tensor call)", bytes_q,
           _launch_stats(multi, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WL, "quantize_ocp (2 launches grouped by K)", bytes_q,
           _launch_stats(grouped, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WL, "fakequant_ocp (196 matrices, one multi-tensor call)", 4.0 * n,
           _launch_stats(multi_fq, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    del a, b, ca, sa, cb, sb, mats, ya, yb
    torch.cuda.empty_cache()
    # the same 196 matrices end to end in one buffer: one launch (the step's form)
    arena, _ = workloads.llama32_3b_arena(dev)
    xa = arena.view(-1, STEP_K)
    ca = torch.empty((xa.shape[0], STEP_K // 2), dtype=torch.uint8, device=dev)
    sa = torch.empty((xa.shape[0], STEP_K // 32), dtype=torch.uint8, device=dev)

    def one_buffer(_):
        ok(mx.mx_quantize(xa.data_ptr(), mx.MX_BF16, xa.shape[0], STEP_K, mx.MX_SCALE_OCP,
                          ca.data_ptr(), sa.data_ptr(), sh))
    report(WL, "quantize_ocp (one launch over the 196 matrices end to end)", bytes_q,
           _launch_stats(one_buffer, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    del arena, xa, ca, sa
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
    # the same experts in MXFP8 (E4M3, the online path of the vLLM page):
    # quantize, dequantize -> bf16, fake-quant
    c8 = [torch.empty(w.numel(), dtype=torch.uint8, device=dev) for w in (w13, w2)]

    def q8(_):
        for (w, rows, k), c, s_ in zip(shapes, c8, ss):
            ok(mx.mx_quantize_mxfp8(w.data_ptr(), mx.MX_BF16, rows, k, c.data_ptr(),
                                    s_.data_ptr(), sh))

    def dq8(_):
        for (w, rows, k), c, s_, y in zip(shapes, c8, ss, ys):
            ok(mx.mx_dequantize_mxfp8(c.data_ptr(), s_.data_ptr(), rows, k, mx.MX_BF16,
                                      y.data_ptr(), sh))

    def fq8(_):
        for (w, rows, k), y in zip(shapes, ys):
            ok(mx.mx_fakequant_mxfp8(w.data_ptr(), mx.MX_BF16, rows, k, y.data_ptr(), sh))

    report(WM, "quantize_mxfp8 (w13 + w2)", (2 + 1 + 1 / 32) * n,
           _launch_stats(q8, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WM, "dequantize_mxfp8_bf16 (w13 + w2)", (1 + 1 / 32 + 2) * n,
           _launch_stats(dq8, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WM, "fakequant_mxfp8 (w13 + w2)", 4.0 * n,
           _launch_stats(fq8, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    del c8
    # and in MBS-Static (16-element sub-blocks, 8-bit macro mantissas per 128)
    smb = [torch.empty(w.numel() // 16, dtype=torch.uint8, device=dev) for w in (w13, w2)]
    mmb = [torch.empty(w.numel() // 128, dtype=torch.uint8, device=dev) for w in (w13, w2)]

    def qmb(_):
        for (w, rows, k), c, s_, m_ in zip(shapes, cs, smb, mmb):
            ok(mx.mx_quantize_mbs(w.data_ptr(), mx.MX_BF16, rows, k, c.data_ptr(), s_.data_ptr(),
                                  m_.data_ptr(), sh))

    def dqmb(_):
        for (w, rows, k), c, s_, m_, y in zip(shapes, cs, smb, mmb, ys):
            ok(mx.mx_dequantize_mbs(c.data_ptr(), s_.data_ptr(), m_.data_ptr(), rows, k,
                                    mx.MX_BF16, y.data_ptr(), sh))

    def fqmb(_):
        for (w, rows, k), y in zip(shapes, ys):
            ok(mx.mx_fakequant_mbs(w.data_ptr(), mx.MX_BF16, rows, k, y.data_ptr(), sh))

    report(WM, "quantize_mbs (w13 + w2)", (2 + 0.5 + 1 / 16 + 1 / 128) * n,
           _launch_stats(qmb, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WM, "dequantize_mbs_bf16 (w13 + w2)", (0.5 + 1 / 16 + 1 / 128 + 2) * n,
           _launch_stats(dqmb, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WM, "fakequant_mbs (w13 + w2)", 4.0 * n,
           _launch_stats(fqmb, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    del smb, mmb
    # and the NVFP4 comparator (16-element blocks, E4M3 block scales, a
    # per-tensor factor): quantize (x read twice) and fake-quant
    bnv = [torch.empty(w.numel() // 16, dtype=torch.uint8, device=dev) for w in (w13, w2)]
    tnv = torch.empty(16, dtype=torch.uint8, device=dev)
    wsnv = [mx.mx_nvfp4_workspace_size(rows, k) for (_, rows, k) in shapes]
    wnv = [torch.empty(b_, dtype=torch.uint8, device=dev) for b_ in wsnv]

    def qnv(_):
        for (w, rows, k), c, b_, ws, wb in zip(shapes, cs, bnv, wnv, wsnv):
            ok(mx.mx_quantize_nvfp4(w.data_ptr(), mx.MX_BF16, rows, k, c.data_ptr(), b_.data_ptr(),
                                    tnv.data_ptr(), ws.data_ptr(), wb, sh))

    def fqnv(_):
        for (w, rows, k), y, ws, wb in zip(shapes, ys, wnv, wsnv):
            ok(mx.mx_fakequant_nvfp4(w.data_ptr(), mx.MX_BF16, rows, k, y.data_ptr(),
                                     ws.data_ptr(), wb, sh))

    report(WM, "quantize_nvfp4 (w13 + w2)", (2 + 2 + 0.5 + 1 / 16) * n,
           _launch_stats(qnv, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    report(WM, "fakequant_nvfp4 (w13 + w2)", 6.0 * n,
           _launch_stats(fqnv, BIG_TIMED, BIG_WARM, stream), cache="exceeds cache")
    del bnv, wnv
    # MXFP4 dequantize of the codes quantized above (its launches end the
    # timed part of the suite's profile)
    qm(0)
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

# Algorithmic bytes per element of each kernel (bf16 in), by the name
# rocprofv3 prints. NVFP4 quantize is two kernels: the tensor-maximum pass
# reads x, the block pass reads it again and writes codes and scales.
KERNEL_BYTES_PER_ELEM = {
    "k_quantize<true, 0, U>": BYTES_PER_ELEM["quantize_ocp"],
    "k_quantize<true, 1, U>": BYTES_PER_ELEM["quantize_oas"],
    "k_quantize<true, 2, U>": EXTRA_BYTES_PER_ELEM["quantize_oas_bits"],
    "k_quantize<true, 3, U>": EXTRA_BYTES_PER_ELEM["quantize_oas_nf"],
    "k_quantize_pair<3, U>": EXTRA_BYTES_PER_ELEM["quantize_oas_nf"],
    "k_dequantize<true, U>": BYTES_PER_ELEM["dequantize_bf16"],
    "k_fakequant<true, 0, U>": BYTES_PER_ELEM["fakequant_ocp"],
    "k_fakequant<true, 1, U>": EXTRA_BYTES_PER_ELEM["fakequant_oas"],
    "k_fakequant<true, 3, U>": EXTRA_BYTES_PER_ELEM["fakequant_oas_nf"],
    "k_block_mse<true, true, U>": BYTES_PER_ELEM["block_mse"],
    "k_quantize8<true, U>": EXTRA_BYTES_PER_ELEM["quantize_mxfp8"],
    "k_dequantize8<true, U>": EXTRA_BYTES_PER_ELEM["dequantize_mxfp8_bf16"],
    "k_fakequant8<true, U>": EXTRA_BYTES_PER_ELEM["fakequant_mxfp8"],
    "k_absmax_partials<true>": 2.0,
    "k_quantize_nv<true, false>": EXTRA_BYTES_PER_ELEM["quantize_nvfp4"] - 2.0,
    "k_quantize_nv<true, true>": EXTRA_BYTES_PER_ELEM["fakequant_nvfp4"] - 2.0,
    "k_dequantize_nv<true>": EXTRA_BYTES_PER_ELEM["dequantize_nvfp4_bf16"],
    "k_quantize_mbs<true, false, U>": EXTRA_BYTES_PER_ELEM["quantize_mbs"],
    "k_quantize_mbs<true, true, U>": EXTRA_BYTES_PER_ELEM["fakequant_mbs"],
    "k_dequantize_mbs<true, U>": EXTRA_BYTES_PER_ELEM["dequantize_mbs_bf16"],
    "k_quantize_fused<true, 0, true>": EXTRA_BYTES_PER_ELEM["quantize_fused"],
    "k_ceiling_quantize_shape": CEILING_BYTES_PER_ELEM["quantize_shape"],
    "k_ceiling_dequantize_shape": CEILING_BYTES_PER_ELEM["dequantize_shape"],
    "k_ceiling_block_mse_shape": CEILING_BYTES_PER_ELEM["block_mse_shape"],
    "k_ceiling_copy": CEILING_BYTES_PER_ELEM["copy"],
    "k_ceiling_read": CEILING_BYTES_PER_ELEM["read"],
    "k_ceiling_write": CEILING_BYTES_PER_ELEM["write"],
}
CALIBRATION_KERNEL = "k_ceiling_copy"  # reads and writes 2 bytes per element, known exactly


def kernel_bytes_per_elem(k: str):
    """Algorithmic bytes per element of kernel k (a name as _kernel_short gives)."""
    return KERNEL_BYTES_PER_ELEM.get(kernel_family(k))


def tile_elems(k: str, grid: int):
    """Elements a dispatch of k covers when it runs one tile per workgroup
    (NT threads x U items x 8 elements, 16 for the two-lanes-per-block
    kernel), else None."""
    u = items_per_thread(k)
    return grid * threads_per_group(k) * u * ITEM_ELEMS.get(k.split("<")[0], 8) if u else None


# The two parts of bench.py that are profiled, each on its own (--only):
# elements a dispatch covers, from its kernel and grid (workgroups). Beside
# the step only the Laplace quantize launches cover C5_ELEMS.
PHASES = {
    "step": {"title": "Llama-3.2-3B linears, 196 matrices end to end, bf16 [917504, 3072] "
                      "(bench.py step)",
             "elems": lambda k, grid: STEP_ELEMS},
    "beside": {"title": "bf16 Student-t activations [8192, 4096] and Laplace activations "
                        "[16384, 8192] (bench.py, beside the step)",
               "elems": lambda k, grid: C5_ELEMS if tile_elems(k, grid) == C5_ELEMS
               else C2_ELEMS},
}
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT -o {p}_trace -- \\\n"
             "    python3 $R/bench.py --only {p} --steps 20 --warmup 5",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $OUT -o {p}_fetch -- \\\n"
             "    python3 $R/bench.py --only {p} --steps 3 --warmup 2",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $OUT -o {p}_write -- \\\n"
             "    python3 $R/bench.py --only {p} --steps 3 --warmup 2",
    "sq": "rocprofv3 --pmc SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_VMEM_RD SQ_INSTS_VMEM_WR \\\n"
          "    SQ_INSTS_LDS SQ_BUSY_CYCLES SQ_WAVE_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $OUT \\\n"
          "    -o {p}_sq -- python3 $R/bench.py --only {p} --steps 3 --warmup 2",
    "suite": "rocprofv3 --kernel-trace --stats --output-format csv -d $OUT -o suite -- \\\n"
             "    python3 $R/bench.py --suite",
}
# VALU issue model for the instruction-mix summary: a wave64 VALU instruction
# holds its 16-lane SIMD for 4 cycles; 256 CUs x 4 SIMDs at 2.4 GHz
SIMDS, CLOCK_GHZ, VALU_CYCLES = 1024, 2.4, 4
PROFILE_HOW = ("Each rocprofv3 command runs on its own, from a scratch working directory "
               "(`cd /tmp`), with `$R` the repository root and `$OUT` an output directory; "
               "`python3 $R/bench.py --summarize-profiles $OUT` then writes this file.")


def _kernel_short(name: str) -> str:
    """'void mxk::k_quantize<true, 0, 2, 128>(void const*, ...)' -> 'k_quantize<true, 0, 2, 128>'."""
    m = re.search(r"\b(k_\w+(?:<[^()]*>)?)\(", name)
    return m.group(1) if m else name.split("(")[0]


def _dispatch_groups(path: str, elems):
    """(kernel, workgroups, elements) -> list of durations in us, from a
    rocprofv3 kernel-trace csv."""
    import collections
    import csv
    groups = collections.OrderedDict()
    with open(path) as f:
        for r in csv.DictReader(f):
            k = _kernel_short(r["Kernel_Name"])
            grid = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            groups.setdefault((k, grid, elems(k, grid)), []).append(dur)
    return groups


def _counter_groups(path: str, elems):
    """(kernel, workgroups, elements) -> {counter: mean value per dispatch}."""
    import collections
    import csv
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            k = _kernel_short(r["Kernel_Name"])
            grid = int(r["Grid_Size"]) // max(1, int(r.get("Workgroup_Size", 256) or 256))
            agg[(k, grid, elems(k, grid))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {key: {c: sum(v) / len(v) for c, v in d.items()} for key, d in agg.items()}


def summarize_profiles(d: str, out_dir: str = os.path.join(ROOT, "profiles")) -> None:
    """The profiles/ summaries from rocprofv3 csv output in d: per profiled
    part of bench.py (the step; beside the step) its kernel trace, its HBM
    traffic (FETCH_SIZE and WRITE_SIZE, calibrated on the reference copy
    kernel) and its instruction mix (SQ counters), and the suite's kernel
    trace, for whichever raw files d holds."""
    h = kernel_code_hash()
    code = ("Kernel code (`csrc/mx_kernels.hip` + `csrc/mx_internal.h`, comments and whitespace "
            f"stripped; `bench.kernel_code_hash`) sha256 prefix: `{h}`\n")
    pct = lambda b, us: b / us / 1e3 / HBM_PEAK_GBS * 100  # noqa: E731
    for p, ph in PHASES.items():
        stem = os.path.join(out_dir, PROFILE_STEM[p])
        cmd = {k: v.format(p=p) for k, v in PROFILE_CMDS.items()}
        trace = os.path.join(d, f"{p}_trace_kernel_trace.csv")
        avg_us = {}
        if os.path.exists(trace):
            out = [f"# Kernel trace: {ph['title']}\n", PROFILE_HOW + "\n",
                   "```\n" + cmd["trace"] + "\n```\n", code,
                   "Per-dispatch GPU times from the trace, grouped by kernel and grid "
                   "(workgroups); algorithmic bytes = the op's bytes per element x the elements "
                   "one launch covers. `k_ceiling_*` are the reference kernels of "
                   "`bench_ceiling.hip` (the quantize kernel's tiling, no format arithmetic).\n",
                   "| kernel | workgroups | elements | dispatches | avg us | min us | max us "
                   "| algorithmic bytes | GB/s at avg | % of 8 TB/s |",
                   "|---|---|---|---|---|---|---|---|---|---|"]
            for (k, grid, n), v in _dispatch_groups(trace, ph["elems"]).items():
                avg = sum(v) / len(v)
                avg_us[(k, grid)] = avg
                bpe = kernel_bytes_per_elem(k)
                if bpe is None and k != "k_sum_partials":
                    continue
                b = int(bpe * n) if bpe else None
                out.append(f"| `{k}` | {grid} | {n if bpe else '-'} | {len(v)} | {avg:.2f} | "
                           f"{min(v):.2f} | {max(v):.2f} | {b if b else '-'} | "
                           f"{f'{b / avg / 1e3:.0f}' if b else '-'} | "
                           f"{f'{pct(b, avg):.1f}' if b else '-'} |")
            with open(stem + "_kernel_trace.md", "w") as f:
                f.write("\n".join(out) + "\n")
        fetch = os.path.join(d, f"{p}_fetch_counter_collection.csv")
        write = os.path.join(d, f"{p}_write_counter_collection.csv")
        if os.path.exists(fetch) and os.path.exists(write):
            cf = _counter_groups(fetch, ph["elems"])
            cw = _counter_groups(write, ph["elems"])
            cal = [key for key in cf if key[0] == CALIBRATION_KERNEL and key in cw]
            ref = max(cal, key=lambda key: key[2])
            ref_kib = ref[2] * 2.0 / 1024  # the copy reads and writes 2 bytes per element
            cal_f = ref_kib / cf[ref]["FETCH_SIZE"]
            cal_w = ref_kib / cw[ref]["WRITE_SIZE"]
            out = [f"# HBM traffic: {ph['title']}\n", PROFILE_HOW + "\n",
                   "```\n" + cmd["fetch"] + "\n" + cmd["write"] + "\n```\n", code,
                   f"Calibration: the reference copy kernel (`{CALIBRATION_KERNEL}`, "
                   f"{ref[2] * 2} bytes read and as many written per dispatch) reads FETCH_SIZE "
                   f"{cf[ref]['FETCH_SIZE']:.1f} KiB and WRITE_SIZE {cw[ref]['WRITE_SIZE']:.1f} "
                   f"KiB, so FETCH_SIZE is scaled by {cal_f:.4f} and WRITE_SIZE by {cal_w:.4f}.\n",
                   "| kernel | workgroups | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled traffic bytes "
                   "| algorithmic bytes | traffic / algorithmic |",
                   "|---|---|---|---|---|---|---|"]
            machine = []
            for key in cf:
                k, grid, n = key
                bpe = kernel_bytes_per_elem(k)
                if bpe is None or key not in cw:
                    continue
                fk, wk = cf[key]["FETCH_SIZE"], cw[key]["WRITE_SIZE"]
                t = (fk * cal_f + wk * cal_w) * 1024
                alg = bpe * n
                out.append(f"| `{k}` | {grid} | {fk:.1f} | {wk:.1f} | {t:.0f} | {alg:.0f} | "
                           f"{t / alg:.4f} |")
                machine.append(f"traffic_bytes {k} {t:.0f}")
            out += ["\nMachine-readable (read by bench.py while the source hash matches):\n",
                    "```\nkernel_code_sha256_prefix " + h] + machine + ["```"]
            with open(stem + "_hbm_traffic.md", "w") as f:
                f.write("\n".join(out) + "\n")
        sq = os.path.join(d, f"{p}_sq_counter_collection.csv")
        if os.path.exists(sq):
            _summarize_instruction_mix(sq, avg_us, ph, cmd["sq"], code, stem)
    suite_csv = os.path.join(d, "suite_kernel_trace.csv")
    if os.path.exists(suite_csv):
        _summarize_suite(suite_csv, code, out_dir)


def _summarize_instruction_mix(path: str, avg_us: dict, ph: dict, cmd: str, code: str,
                               stem: str) -> None:
    """Instructions per wave-item (one item = 8 elements per lane, 64 lanes)
    of each kernel from the SQ counters, and the time its VALU instructions
    take at full issue rate next to the kernel's traced duration."""
    out = [f"# Instruction mix: {ph['title']}\n", PROFILE_HOW + "\n", "```\n" + cmd + "\n```\n",
           code,
           "Counts are chip totals per dispatch (SQ_WAVES equals the waves launched), "
           "averaged over the dispatches of each kernel and grid, per wave-item: one item is 8 "
           "elements in each of a wave's 64 lanes. VALU issue time = SQ_INSTS_VALU x "
           f"{VALU_CYCLES} cycles / ({SIMDS} SIMDs x {CLOCK_GHZ} GHz), the time the kernel's "
           "vector instructions need if every SIMD issued one each cycle slot with nothing else "
           "in the way; kernel time from the kernel trace of the same code.\n",
           "| kernel | workgroups | waves | VALU / wave-item | SALU / wave-item | VMEM rd / "
           "wave-item | VMEM wr / wave-item | LDS / wave-item | VALU issue us | kernel us | "
           "VALU issue / kernel |", "|---|---|---|---|---|---|---|---|---|---|---|"]
    for (k, grid, n), c in _counter_groups(path, ph["elems"]).items():
        if kernel_bytes_per_elem(k) is None:
            continue
        wave_items = n / (8 * 64)
        per = lambda name: c.get(name, 0.0) / wave_items  # noqa: E731
        valu_us = c.get("SQ_INSTS_VALU", 0.0) * VALU_CYCLES / (SIMDS * CLOCK_GHZ * 1e3)
        t = avg_us.get((k, grid))
        out.append(f"| `{k}` | {grid} | {int(c.get('SQ_WAVES', 0))} | {per('SQ_INSTS_VALU'):.1f} | "
                   f"{per('SQ_INSTS_SALU'):.1f} | {per('SQ_INSTS_VMEM_RD'):.2f} | "
                   f"{per('SQ_INSTS_VMEM_WR'):.2f} | {per('SQ_INSTS_LDS'):.2f} | {valu_us:.2f} | "
                   f"{f'{t:.2f}' if t else '-'} | {f'{valu_us / t:.2f}' if t else '-'} |")
    with open(stem + "_instruction_mix.md", "w") as f:
        f.write("\n".join(out) + "\n")


def _summarize_suite(path: str, code: str, out_dir: str) -> None:
    """Per-workload kernel times of `bench.py --suite` from its kernel trace.
    Launches are told apart by kernel, dtype and the elements their grid
    covers (one tile per workgroup); the Laplace launches' cold and warm
    timings by dispatch order."""
    import collections
    import csv

    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    c1, c5 = 1024 * 4096, 16384 * 8192
    l3072, l8192 = 688128 * 3072, 86016 * 8192
    m13, m2 = 128 * 3072 * 4096, 128 * 4096 * 1536
    by_elems = {
        c5: "bf16 Laplace [16384, 8192]",
        1024 * 3072: "Llama-3.2-3B per-matrix launches: k/v [1024, 3072]",
        3072 * 3072: "Llama-3.2-3B per-matrix launches: q/o [3072, 3072]",
        8192 * 3072: "Llama-3.2-3B per-matrix launches: gate/up [8192, 3072] and down [3072, 8192]",
        l3072: "Llama-3.2-3B grouped by K: K=3072 [688128, 3072]",
        l8192: "Llama-3.2-3B grouped by K: K=8192 [86016, 8192]",
        STEP_ELEMS: "Llama-3.2-3B, 196 matrices end to end: one launch [917504, 3072]",
        m13: "MoE w13 [128x3072, 4096]", m2: "MoE w2 [128x4096, 1536]"}
    passes = 2 * BIG_TIMED + BIG_WARM  # dispatches of one big-workload timing

    def bytes_for(kernel, n, f32):
        if kernel == "k_ceiling_copy":  # the fp32 input copied: 4 bytes in, 4 out
            return n * 8.0
        if kernel.startswith(("k_quantize<", "k_dequantize<")):
            return n * (4.53125 if f32 else 2.53125)
        if kernel.startswith("k_block_mse<"):
            return n * (4.65625 if f32 else 2.65625)
        if kernel.startswith("k_quantize_fused<"):
            return n * (8.65625 if f32 else 4.65625)
        if kernel.startswith(("k_quantize8<", "k_dequantize8<")):
            return n * (5.03125 if f32 else 3.03125)
        if kernel.startswith("k_fakequant8<") or kernel.startswith("k_quantize_mbs<true, true"):
            return n * (8.0 if f32 else 4.0)
        if kernel.startswith(("k_quantize_mbs<", "k_dequantize_mbs<")):
            return n * ((2.0 if f32 else 0.0) + 2 + 0.5 + 1 / 16 + 1 / 128)
        if kernel.startswith("k_quantize_nv_big<true, true"):  # NVFP4 block pass, fake-quant
            return n * 4.0
        if kernel.startswith("k_quantize_nv_big<"):  # NVFP4 block pass, quantize
            return n * (2 + 0.5 + 1 / 16)
        if kernel.startswith("k_absmax_partials<"):  # NVFP4 maximum pass: x read once
            return n * 2.0
        return None

    # the timed part ends with the MoE dequantize launches; the QSNR pass
    # that follows is not timed and is left out
    grid_of = lambda r: int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))  # noqa: E731
    last = max(i for i, r in enumerate(rows)
               if _kernel_short(r["Kernel_Name"]).startswith("k_dequantize<true,")
               and tile_elems(_kernel_short(r["Kernel_Name"]), grid_of(r)) in (m13, m2))
    groups = collections.OrderedDict()
    seen_c5 = collections.Counter()
    seen_abs = collections.Counter()
    per_timing = 10 + 2 * 100  # dispatches of one _launch_stats call at the suite's defaults
    for r in rows[:last + 1]:
        k = _kernel_short(r["Kernel_Name"])
        if not k.startswith("k_"):
            continue
        grid = grid_of(r)
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        n = tile_elems(k, grid)
        if k.startswith("k_multi"):
            key = ("MULTI", k, None)
        elif k == "k_sum_partials":
            key = ("tensor-sum pass of block MSE (all workloads)", k, None)
        elif k == "k_nv_prepare":
            key = ("NVFP4 tensor-exponent reduction (MoE experts)", k, None)
        elif k.startswith("k_absmax_partials<true"):
            # NVFP4's maximum pass (a 2,048-workgroup grid for every size):
            # the suite runs it on w13, then w2, in every call
            which = seen_abs[k] % 2
            seen_abs[k] += 1
            nn = (m13, m2)[which]
            key = (by_elems[nn], k, nn)
        elif k.startswith("k_ceiling"):
            key = ("fp32 normal [1024, 4096]: reference kernels", k, c1)
        elif "<false" in k:
            key = ("fp32 normal [1024, 4096]", k, c1)
        elif n == c5:
            # each op is timed cold (rotated sets), then warm (one set): runs
            # of per_timing dispatches alternate
            cold = (seen_c5[k] // per_timing) % 2 == 0
            seen_c5[k] += 1
            key = (by_elems[c5] + (", cold (rotated sets)" if cold
                                   else ", warm (one set, cache-resident)"), k, c5)
        elif n in by_elems:
            key = (by_elems[n], k, n)
        else:
            key = (f"unattributed (grid {grid})", k, None)
        groups.setdefault(key, []).append(dur)
    # the OCP quantize and fake-quant launches of the multi-tensor calls (bf16)
    multis = []
    for fq, bpe, what in ((False, 2.53125, "one `mx_quantize_multi` call"),
                          (True, 4.0, "one `mx_fakequant_multi` call")):
        key = next((key for key in groups if key[0] == "MULTI" and
                    key[1].startswith(f"k_multi<true, 0, {'true' if fq else 'false'}")), None)
        if key:
            multis.append((key[1], groups.pop(key), bpe, what))
    out = ["# Kernel trace: the other workloads (`bench.py --suite`)\n", PROFILE_HOW + "\n",
           "```\n" + PROFILE_CMDS["suite"] + "\n```\n", code,
           "Durations are the GPU's own per-dispatch times from the trace (under the profiler the "
           "host-side event figures of the small fp32 case are inflated by per-dispatch overhead; "
           "these are not). Launches are attributed to their workload by the elements their grid "
           "covers (NT threads x U items x 8 elements per workgroup, from the kernel's template "
           "arguments; the workloads' sizes all differ). The Laplace launches are split into the cold (rotated sets) and "
           f"warm (one set) timings by dispatch order ({per_timing} dispatches each). "
           "Per-matrix Llama launches are grouped by shape. The fp32 rows mix cold, warm, "
           "single-launch and graph-replayed dispatches. The suite's QSNR pass, which runs after "
           "the timed launches, is left out.\n",
           "| workload | kernel | dispatches | avg us | min us | max us | algorithmic bytes "
           "| GB/s at avg | % of 8 TB/s |", "|---|---|---|---|---|---|---|---|---|"]
    for (wl, k, n), v in groups.items():
        avg = sum(v) / len(v)
        b = bytes_for(k, n, "<false" in k) if n else None
        out.append(f"| {wl} | `{k}` | {len(v)} | {avg:.2f} | {min(v):.2f} | {max(v):.2f} | "
                   f"{int(b) if b else '-'} | {f'{b / avg / 1e3:.0f}' if b else '-'} | "
                   f"{f'{b / avg / 1e3 / HBM_PEAK_GBS * 100:.1f}' if b else '-'} |")
    for kname, multi, bpe, what in multis:
        per_pass = sum(multi) / passes
        b = (l3072 + l8192) * bpe
        out.append(f"| Llama-3.2-3B, the 196 weights as separate tensors: {what} "
                   f"per pass ({len(multi) // passes} launches) | `{kname}` | "
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
