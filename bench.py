"""Benchmark of the QLoRA NF4 linear hot path on one MI355X.

Step = one training step (forward + backward) of every projection of one
LLaMA-65B-shaped decoder layer (q, k, v, o 8192 -> 8192; gate, up 8192 ->
22016; down 22016 -> 8192), NF4 + double-quantised weights with a LoRA
adapter r = 64, alpha = 16 on each, 2048 tokens: per projection U = X·Aᵀ
(rank-r streaming kernel and its split reduction) and the dequant-GEMM with
the rank-r prologue, then V = dY·B and dB = s·dYᵀ·U (one streaming launch and
one reduction), the transposed dequant-GEMM for dX, and dA = s·Vᵀ·X
(streaming kernel and reduction).  6,754.24 GFLOP per step on
resident seeded synthetic inputs; `value` = algorithmic TFLOP/s of the step.
The roofline object is the forward dequant-GEMM over the layer's seven
launches, timed on the stream it runs on; `roofline_gemv` is the few-token
dequant-GEMV kernel (8192 -> 28672, 1 token) against HBM (its traffic from
the committed summary of the HBM-bound kernels' byte counters).  The same run also
measures, in `rows`, the LLaMA-7B MLP training step (4096 tokens, 4096 ->
11008, r = 64), the fused NF4 + double-quant quantiser and the dequantiser
(one matrix and the whole 224-matrix LLaMA-7B weight set), the few-token
forward at 1..8 tokens, the single 16-token 4096 x 4096 linear, the 32-bit
AdamW step over the 67M LoRA parameters of LLaMA-7B's attention projections,
the single-quantisation INT4 quantiser, decoder and error pass, the training
step with LoRA dropout (p = 0.05), and the adapter merge with
re-quantisation.

Prints ONE JSON line.  --gpus N > 1 is not supported (single-GPU build).
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# float64 fma on the vector ALU: 256 CUs x 64 lanes x 2 flop x 2.4 GHz
FP64_FMA_PEAK_TFLOPS = 78.6
GEMM_SOURCES = ["qlora_gemm.hip", "qlora_common.h", "qlora_kernels.h", "qlora_philox.h"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_gemm_fwd_llama65b_layer.txt")
CALIB_BYTES = 512 << 20  # plain device copy used to scale the byte counters


def gemm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "bit_nf4_quantized_blockwise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch of the forward dequant-GEMM from the committed
    counter summary, or None if absent or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    kv = {}
    for line in open(TRAFFIC_SUMMARY):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != gemm_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


HBM_SUMMARY = os.path.join(ROOT, "profiles", "traffic_hbm_bound_kernels.txt")


def read_gemv_traffic():
    """Counted HBM bytes per launch (read + write) of the few-token GEMV at one
    token on the 8192 -> 28672 weight, from the committed summary of the
    HBM-bound kernels, or None if absent or taken on a different kernel source."""
    if not os.path.exists(HBM_SUMMARY):
        return None
    lines = open(HBM_SUMMARY).read().splitlines()
    src = [ln.split("=", 1)[1].strip() for ln in lines if ln.startswith("kernel_source_sha256_16")]
    if not src or src[0] != hbm_source_hash():
        return None
    for ln in lines:
        if ln.startswith("few-token GEMV, 1 token:"):
            try:
                rd = ln.split("read", 1)[1].split("/", 1)[0]
                wr = ln.split("write", 1)[1].split("/", 1)[0]
                return float(rd) + float(wr)
            except (IndexError, ValueError):
                return None
    return None


def _layer_fwd_algo_bytes():
    """Algorithmic bytes of the layer's seven forward dequant-GEMM launches
    (weight storage, X, U, B and Y once each), summed."""
    tot = 0
    for K, N in LAYER65B_SHAPES:
        n = N * K
        tot += n // 2 + n // 64 + ((n // 64 + 255) // 256) * 4 + 2 * 2048 * K + 2 * 2048 * 64 \
            + 2 * N * 64 + 2 * 2048 * N
    return tot


def summarize_pmc(fetch_csv, write_csv, out_path):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the forward dequant-GEMM
    (the layer's seven launches of --pmc-pass, averaged per launch), each
    scaled by what the same counter reads for a device copy of CALIB_BYTES,
    written as a short text summary."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("gemm" if FWD_GEMM in name else "copy" if "copyBuffer" in name else None)
            if key:
                vals.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
                vals[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: (sum(v.values()) / len(v), len(v)) for k, v in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    kib = CALIB_BYTES / 1024.0
    f_scale = kib / f["copy"][0]
    w_scale = kib / w["copy"][0]
    fetch_b = f["gemm"][0] * f_scale * 1024.0
    write_b = w["gemm"][0] * w_scale * 1024.0
    algo = _layer_fwd_algo_bytes() / 7
    with open(out_path, "w") as fh:
        fh.write("# HBM traffic of the forward dequant-GEMM over the seven projections of one\n")
        fh.write("# LLaMA-65B layer (2048 tokens, r = 64), per launch (average of the seven shapes),\n")
        fh.write("# from rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by the same counter on a\n")
        fh.write(f"# device copy of {CALIB_BYTES} bytes.  Commands (from /tmp, TMPDIR=/tmp):\n")
        fh.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o f -- python3 <repo>/bench.py --pmc-pass\n")
        fh.write("#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_w> -o w -- python3 <repo>/bench.py --pmc-pass\n")
        fh.write("#   python3 <repo>/bench.py --summarize-pmc <dir_f>/f_counter_collection.csv "
                 "<dir_w>/w_counter_collection.csv <this file>\n")
        fh.write(f"kernel_source_sha256_16 = {gemm_source_hash()}\n")
        fh.write(f"gemm_dispatches = {f['gemm'][1]}\n")
        fh.write(f"fetch_kib_per_launch_raw = {f['gemm'][0]:.1f}\n")
        fh.write(f"write_kib_per_launch_raw = {w['gemm'][0]:.1f}\n")
        fh.write(f"copy_fetch_kib_raw = {f['copy'][0]:.1f}\n")
        fh.write(f"copy_write_kib_raw = {w['copy'][0]:.1f}\n")
        fh.write(f"fetch_scale = {f_scale:.4f}\n")
        fh.write(f"write_scale = {w_scale:.4f}\n")
        fh.write(f"fetch_bytes_per_launch = {fetch_b:.0f}\n")
        fh.write(f"write_bytes_per_launch = {write_b:.0f}\n")
        fh.write(f"traffic_bytes_per_launch = {fetch_b + write_b:.0f}\n")
        fh.write(f"algorithmic_bytes_per_launch = {algo:.0f}\n")
        fh.write(f"traffic_over_algorithmic = {(fetch_b + write_b) / algo:.3f}\n")
    print(open(out_path).read())


def summarize_stats(stats_csv, bench_log, out_path):
    """Short text summary of a rocprofv3 --kernel-trace --stats run of this
    script: calls and durations per kernel and launch grid (from the per-
    dispatch trace beside the stats file), with the bench line it printed.
    With --no-rows every forward dequant-GEMM launch is one of the layer's
    seven projections, each equally often, so their mean duration is the
    per-launch figure the roofline's event timing is compared with."""
    import csv
    import statistics

    trace_csv = stats_csv.replace("kernel_stats", "kernel_trace")
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        key = (r["Kernel_Name"], f"{r['Grid_Size_X']}x{r['Grid_Size_Y']}")
        groups.setdefault(key, []).append(dur)
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    line = [ln for ln in open(bench_log) if ln.startswith('{"metric"')][-1]
    d = json.loads(line)
    fwd = [x for k, v in groups.items() if FWD_GEMM in k[0] for x in v]
    with open(out_path, "w") as fh:
        fh.write("# rocprofv3 kernel statistics of bench.py (QLoRA linear fwd + bwd over the seven\n"
                 "# projections of one LLaMA-65B layer, 2048 tokens, r = 64, and the other rows of\n"
                 "# the bench line), one MI355X, per kernel and launch grid.\n")
        fh.write("# commands (from /tmp, TMPDIR=/tmp):\n")
        rows_flag = "" if d["rows"] and len(d["rows"]) > 1 else " --no-rows"
        fh.write("#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- "
                 f"python3 <repo>/bench.py --no-cpu-baseline{rows_flag} --steps 10 --warmup 2 > <log>\n")
        fh.write("#   python3 <repo>/bench.py --summarize-stats <dir>/bench_kernel_stats.csv "
                 "<log> <this file>\n")
        fh.write(f"# bench line under the profiler: value = {d['value']:.1f} TFLOP/s, "
                 f"ms_per_step = {d['ms_per_step']:.3f},\n")
        fh.write(f"#   forward dequant-GEMM per launch (events) = "
                 f"{d['roofline']['us_per_launch']:.1f} us\n")
        if fwd and rows_flag:
            fh.write(f"#   forward dequant-GEMM per launch (trace, all grids): {len(fwd)} calls, "
                     f"mean {statistics.mean(fwd):.1f} us\n")
        fh.write("\n")
        fh.write(f"{'kernel':<72} {'grid':>14} {'calls':>6} {'avg_us':>10} {'min_us':>10} "
                 f"{'max_us':>10} {'total_ms':>10}\n")
        for (name, grid), v in rows[:60]:
            fh.write(f"{name[:72]:<72} {grid:>14} {len(v):>6} {statistics.mean(v):>10.2f} "
                     f"{min(v):>10.2f} {max(v):>10.2f} {sum(v) / 1e3:>10.3f}\n")
    print(open(out_path).read())


FWD_GEMM = "gemm_kernel<256, 256, 2, 2, 0, true, 0, 0>"
DX_GEMM = "gemm_kernel<256, 256, 2, 2, 1, true, 0, 0>"


def summarize_counters(out_path, *csvs, kernel=FWD_GEMM, what="forward dequant-GEMM",
                       pass_flag="--pmc-pass", summary_flag="--summarize-counters",
                       workload="the LLaMA-65B layer's 7 projections: 2048 tokens, r = 64"):
    """Per-dispatch averages of the SQ counters of one GEMM kernel from
    rocprofv3 --pmc runs of a counter pass, with the ratios read off them."""
    import csv

    vals = {}
    for path in csvs:
        for r in csv.DictReader(open(path)):
            if kernel not in r["Kernel_Name"]:
                continue
            d = vals.setdefault(r["Counter_Name"], {})
            key = (path, r["Dispatch_Id"])  # a counter may appear in several runs
            d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    avg = {k: sum(v.values()) / len(v) for k, v in vals.items()}
    with open(out_path, "w") as fh:
        fh.write(f"# SQ counters of the {what} ({workload}),\n"
                 f"# per dispatch, averaged over the dispatches of {pass_flag}.  "
                 "Commands (from /tmp, TMPDIR=/tmp),\n# one rocprofv3 run per counter set:\n")
        fh.write("#   rocprofv3 --pmc <set> --output-format csv -d <dir_i> -o c -- python3 "
                 f"<repo>/bench.py {pass_flag}\n")
        fh.write(f"#   python3 <repo>/bench.py {summary_flag} <this file> "
                 "<dir_1>/c_counter_collection.csv ...\n")
        fh.write(f"kernel_source_sha256_16 = {gemm_source_hash()}\n")
        for k in sorted(avg):
            fh.write(f"{k} = {avg[k]:.6g}\n")
        if "SQ_INSTS_MFMA" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            fh.write(f"# matrix-pipe cycles per MFMA = "
                     f"{avg['SQ_VALU_MFMA_BUSY_CYCLES'] / avg['SQ_INSTS_MFMA']:.2f}\n")
        if "SQ_VALU_MFMA_COEXEC_CYCLES" in avg and "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
            fh.write(f"# share of matrix-pipe busy cycles with VALU work beside it = "
                     f"{avg['SQ_VALU_MFMA_COEXEC_CYCLES'] / avg['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}\n")
        if "SQ_WAIT_INST_ANY" in avg and "SQ_WAVE_CYCLES" in avg:
            fh.write(f"# wave cycles waiting on a dependency (s_waitcnt) = "
                     f"{avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.3f}, on LDS = "
                     f"{avg.get('SQ_WAIT_INST_LDS', 0.0) / avg['SQ_WAVE_CYCLES']:.3f}\n")
    print(open(out_path).read())


def pmc_pass_bwd():
    """Short run for counter collection: the backward of the LLaMA-7B MLP
    linear (input-gradient dequant-GEMM and adapter products) three times."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    dev = torch.device("cuda:0")
    wlc = wl.LLAMA7B_MLP
    inp = wlc.inputs()
    wq = q.quantize_weight(torch.from_numpy(inp["W"]).to(dev))
    X, A, B, dY = (inp[k].to(dev) for k in ("X", "A", "B", "dY"))
    U = q.lora_down(X, A)
    ws = torch.empty(q.workspace_size(1, wlc.M, wlc.n_out, wlc.k_in, wlc.r), dtype=torch.uint8,
                     device=dev)
    for _ in range(3):
        q.linear_bwd(wq, X, dY, A, B, U, wlc.alpha, workspace=ws)
    torch.cuda.synchronize()
    print("pmc bwd pass done", flush=True)


def pmc_pass():
    """Short run for counter collection: the forward dequant-GEMM of each of
    the LLaMA-65B layer's seven projections once (inputs drawn on the GPU:
    the counters do not depend on the values) and a device copy of
    CALIB_BYTES (the byte counters' calibration)."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(5)
    M, r = 2048, 64
    for K, N in LAYER65B_SHAPES:
        wq = q.quantize_weight(torch.randn(N, K, generator=gen, device=dev) * 0.02)
        bf = lambda *shape, s: (torch.randn(*shape, generator=gen, device=dev) * s).to(torch.bfloat16)
        X, A, B = bf(M, K, s=1.0), bf(r, K, s=0.01), bf(N, r, s=0.01)
        U = q.lora_down(X, A)
        q.nf4_matmul_fwd(wq, X, U, B, 16.0)
        torch.cuda.synchronize()
        del wq, X, A, B, U
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("pmc pass done", flush=True)


HBM_SOURCES = ["qlora_quant.hip", "qlora_gemv.hip", "qlora_adapter.hip", "qlora_aux.hip",
               "qlora_common.h", "qlora_kernels.h"]


def hbm_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in HBM_SOURCES:
        with open(os.path.join(ROOT, "bit_nf4_quantized_blockwise_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def pmc_pass_hbm():
    """Short run for the byte counters of the HBM-bound kernels: the fused
    quantiser (two launches) and the dequantiser on the 11008 x 4096 weight,
    the few-token forward (U launch + GEMV) at one token on the 8192 -> 28672
    weight, the one-launch forward of the single 16-token 4096 x 4096 linear
    (r = 8), the rank-r streaming kernels of the LLaMA-65B q projection (2048
    tokens, 8192 -> 8192, r = 64: U, then V and dB, then dA), three times
    each, and the calibration copy."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    dev = torch.device("cuda:0")
    # the few-token and q-projection weights are quantised first: the summary
    # takes the last three dispatches of each kernel
    g = wl.GEMV_70B
    gin = g.inputs(M=1)
    wg = q.quantize_weight(torch.from_numpy(gin["W"]).to(dev))
    p = wl.LLAMA65B_LAYER[0]
    pin = p.inputs()
    wp = q.quantize_weight(torch.from_numpy(pin["W"]).to(dev))
    sl = wl.SINGLE_LINEAR
    sin = sl.inputs()
    wsl = q.quantize_weight(torch.from_numpy(sin["W"]).to(dev))
    W = torch.from_numpy(wl.LLAMA7B_MLP.inputs(with_dy=False)["W"]).to(dev)
    for _ in range(3):
        o = q.quantize_nf4_dq(W, want_absmax=True)
    wq = q.NF4Tensor(o[0], o[1], o[2], W.shape[0], W.shape[1])
    out = torch.empty(W.shape, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        q.dequantize_nf4(wq, out=out)
    del W, out
    X, A, B = (gin[k].to(dev) for k in ("X", "A", "B"))
    for _ in range(3):
        q.linear_fwd(wg, X, A, B, g.alpha)
    del wg, X, A, B
    X, A, B = (sin[k].to(dev) for k in ("X", "A", "B"))
    for _ in range(3):
        q.linear_fwd(wsl, X, A, B, sl.alpha)
    del wsl, X, A, B
    X, A, B, dY = (pin[k].to(dev) for k in ("X", "A", "B", "dY"))
    for _ in range(3):
        U = q.lora_down(X, A)
        q.linear_bwd(wp, X, dY, A, B, U, p.alpha)
    del wp, X, A, B, dY, U
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("pmc hbm pass done", flush=True)


def summarize_hbm(out_path, fetch_csv, write_csv):
    """Per-launch FETCH_SIZE / WRITE_SIZE of the HBM-bound kernels (the last
    three dispatches of each), scaled by the copy calibration, against each
    kernel's algorithmic bytes."""
    import csv

    # qualified names: "quantize_nf4_kernel" alone would also match the dequantiser
    keys = {"qlora::quantize_nf4_kernel(": "quantise, first level",
            "qlora::double_quant_kernel(": "DQ, second level",
            "qlora::dequantize_nf4_kernel(": "dequantise",
            "qlora::lora_down_small_kernel(": "U = X·Aᵀ, 1 token",
            "qlora::nf4_gemv_kernel<": "few-token GEMV, 1 token",
            "qlora::nf4_small_fwd_kernel<": "one-launch forward, 16 tokens, 4096 x 4096, r = 8",
            "qlora::adapter_rows_kernel<2, false>(": "U = X·Aᵀ splits (q projection)",
            "qlora::adapter_dy_kernel<2>(": "V = dY·B and dB = s·dYᵀ·U splits, one launch",
            "qlora::adapter_cols_kernel<2, true>(": "dA = s·Vᵀ·X splits",
            "copyBuffer": "copy"}

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            key = next((k for k in keys if k in r["Kernel_Name"]), None)
            if key:
                vals.setdefault(key, {}).setdefault(int(r["Dispatch_Id"]), 0.0)
                vals[key][int(r["Dispatch_Id"])] += float(r["Counter_Value"])
        # the last three dispatches of each kernel are the measured ones (the
        # calibration copies run last; earlier copies and the quantisation of
        # the few-token weight move other buffers)
        for k in vals:
            last = sorted(vals[k])[-3:]
            vals[k] = {d: vals[k][d] for d in last}
        return {k: sum(v.values()) / len(v) for k, v in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    kib = CALIB_BYTES / 1024.0
    fs, ws_ = kib / f["copyBuffer"], kib / w["copyBuffer"]
    n = 11008 * 4096
    nb, ng = n // 64, (n // 64 + 255) // 256
    ng70, n70 = (28672 * 8192 // 64 + 255) // 256, 28672 * 8192
    n1 = 4096 * 4096
    ng1 = (n1 // 64 + 255) // 256
    algo = {
        "qlora::quantize_nf4_kernel(": (4 * n, n // 2 + 4 * nb),
        "qlora::double_quant_kernel(": (4 * nb, nb + 4 * ng),
        "qlora::dequantize_nf4_kernel(": (n // 2 + nb + 4 * ng, 2 * n),
        "qlora::lora_down_small_kernel(": (2 * 8192 + 2 * 16 * 8192, 2 * 16),
        "qlora::nf4_gemv_kernel<": (n70 // 2 + n70 // 64 + 4 * ng70 + 2 * 8192 + 2 * 16 * 28672 + 2 * 16,
                            2 * 28672),
        # weight storage, X, A and B read once; Y and U written once (every
        # workgroup reads all of X and A, from L2 after the first)
        "qlora::nf4_small_fwd_kernel<": (n1 // 2 + n1 // 64 + 4 * ng1 + 2 * 16 * 4096 + 2 * 8 * 4096
                                         + 2 * 4096 * 8, 2 * 16 * 4096 + 2 * 16 * 8),
        # q projection, M = 2048, K = N = 8192, r = 64: each product's operands
        # read once, its result written once (bf16 U and V, fp32 dA and dB)
        "qlora::adapter_rows_kernel<2, false>(": (2 * 2048 * 8192 + 2 * 64 * 8192, 2 * 2048 * 64),
        "qlora::adapter_dy_kernel<2>(": (2 * (2 * 2048 * 8192) + 2 * 8192 * 64 + 2 * 2048 * 64,
                                        2 * 2048 * 64 + 4 * 8192 * 64),
        "qlora::adapter_cols_kernel<2, true>(": (2 * 2048 * 8192 + 2 * 2048 * 64, 4 * 64 * 8192),
    }
    with open(out_path, "w") as fh:
        fh.write("# HBM traffic of the HBM-bound kernels: the fused quantiser (two launches) and the\n")
        fh.write("# dequantiser on the 11008 x 4096 weight, the few-token forward at 1 token on the\n")
        fh.write("# 8192 -> 28672 weight (r = 16), the one-launch forward of the single 16-token\n")
        fh.write("# 4096 x 4096 linear (r = 8), the rank-r streaming kernels of the LLaMA-65B q\n")
        fh.write("# projection (2048 tokens, r = 64; their writes are the fp32 partial sums of the\n")
        fh.write("# splits, summed by the next launch, against the result written once).\n")
        fh.write("# rocprofv3 FETCH_SIZE and WRITE_SIZE per launch\n")
        fh.write(f"# (the last three dispatches of each), each scaled by the same counter on a device copy of\n")
        fh.write(f"# {CALIB_BYTES} bytes.  Commands (from /tmp, TMPDIR=/tmp):\n")
        fh.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o f -- python3 <repo>/bench.py --pmc-pass-hbm\n")
        fh.write("#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_w> -o w -- python3 <repo>/bench.py --pmc-pass-hbm\n")
        fh.write("#   python3 <repo>/bench.py --summarize-hbm <this file> <dir_f>/f_counter_collection.csv "
                 "<dir_w>/w_counter_collection.csv\n")
        fh.write(f"kernel_source_sha256_16 = {hbm_source_hash()}\n")
        fh.write(f"fetch_scale = {fs:.4f}\nwrite_scale = {ws_:.4f}\n")
        fh.write("# kernel: counted read / write bytes per launch; algorithmic read / write; counted / algorithmic\n")
        for k, (ar, aw) in algo.items():
            if k not in f or k not in w:
                continue
            cr, cw = f[k] * fs * 1024.0, w[k] * ws_ * 1024.0
            fh.write(f"{keys[k]}: read {cr:.0f} / {ar}, write {cw:.0f} / {aw}, "
                     f"total {(cr + cw) / (ar + aw):.3f}\n")
        kq, kd = "qlora::quantize_nf4_kernel(", "qlora::double_quant_kernel("
        q2 = (f.get(kq, 0) + f.get(kd, 0)) * fs * 1024.0 + (w.get(kq, 0) + w.get(kd, 0)) * ws_ * 1024.0
        fh.write(f"quantise + DQ (both launches) counted {q2:.0f} against the fused algorithmic "
                 f"{4 * n + n // 2 + nb + 4 * ng} (ratio {q2 / (4 * n + n // 2 + nb + 4 * ng):.3f}; the "
                 "absmax hand-over is 8 B per 64 weights)\n")
    print(open(out_path).read())


def _events():
    import torch
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _c_call(fn, *args):
    """A library entry point with its arguments marshalled once, so a timing
    loop spends ~µs per call on the host and the GPU queue stays ahead of it."""
    import bit_nf4_quantized_blockwise_amd as q
    name = fn.__name__

    def call():
        s = fn(*args)
        if s != 0:
            raise q.QloraError(s, name)
    return call


def _rotate(calls):
    """One call per invocation, cycling through `calls` (inputs that together
    exceed the last-level cache, so each call streams from HBM)."""
    it = [0]

    def call():
        calls[it[0] % len(calls)]()
        it[0] += 1
    return call


def _time_ms(fn, iters, warmup=2):
    import torch
    for _ in range(warmup):
        fn()
    s, e = _events()
    torch.cuda.synchronize()
    s.record()
    for _ in range(iters):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="time only the training step")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="only run the forward dequant-GEMM and a calibration copy (counters)")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_TXT"),
                    help="write the HBM traffic summary from two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "BENCH_LOG", "OUT_TXT"),
                    help="write the kernel statistics summary of a rocprofv3 --stats run")
    ap.add_argument("--pmc-pass-bwd", action="store_true",
                    help="only run the backward (input-gradient GEMM) for counters")
    ap.add_argument("--summarize-counters-bwd", nargs="+", metavar="PATH",
                    help="OUT_TXT then the counter CSVs of rocprofv3 --pmc runs of --pmc-pass-bwd")
    ap.add_argument("--pmc-pass-hbm", action="store_true",
                    help="only run the HBM-bound kernels and a calibration copy (counters)")
    ap.add_argument("--summarize-hbm", nargs=3, metavar=("OUT_TXT", "FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="PATH",
                    help="OUT_TXT then the counter CSVs of rocprofv3 --pmc runs of --pmc-pass")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_stats:
        summarize_stats(*args.summarize_stats)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the build has no multi-GPU path "
              "(the linear shards by tokens with one all-reduce of dA, dB; not built)",
              file=sys.stderr)
        sys.exit(2)

    if args.pmc_pass:
        pmc_pass()
        return
    if args.pmc_pass_hbm:
        pmc_pass_hbm()
        return
    if args.pmc_pass_bwd:
        pmc_pass_bwd()
        return
    if args.summarize_counters_bwd:
        summarize_counters(*args.summarize_counters_bwd, kernel=DX_GEMM,
                           what="input-gradient dequant-GEMM", pass_flag="--pmc-pass-bwd",
                           workload="LLaMA-7B MLP: 4096 tokens, 4096 -> 11008, r = 64",
                           summary_flag="--summarize-counters-bwd")
        return
    if args.summarize_hbm:
        summarize_hbm(*args.summarize_hbm)
        return

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print("[bench] LLaMA-65B layer inputs (seeded, host)", file=sys.stderr, flush=True)
    layer = layer65b_setup(dev)

    def step():
        for P in layer:
            P["fwd"]()
            P["bwd"]()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    s, e = _events()
    s.record()
    for _ in range(args.steps):
        step()
    e.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = s.elapsed_time(e) / args.steps
    flops = sum(P["flops"] for P in layer)
    tflops = flops / (ms_step * 1e-3) / 1e12
    print(f"[bench] layer step {ms_step:.3f} ms, {tflops:.1f} TFLOP/s", file=sys.stderr,
          flush=True)

    # dominant kernel: the forward dequant-GEMM (Y = X·Ŵᵀ + s·U·Bᵀ), one launch
    # per projection through its own entry point, timed with events on the
    # stream it is launched on
    per, g_ms, g_flops = {}, 0.0, 0
    for P in layer:
        ms_p = _time_ms(P["gemm"], args.steps, warmup=3)
        per[P["name"]] = dict(step_ms=_time_ms(lambda: (P["fwd"](), P["bwd"]()), args.steps,
                                               warmup=2),
                              fwd_gemm_us=ms_p * 1e3,
                              fwd_gemm_TFLOPs=P["gemm_flops"] / (ms_p * 1e-3) / 1e12)
        per[P["name"]]["step_TFLOPs"] = P["flops"] / (per[P["name"]]["step_ms"] * 1e-3) / 1e12
        g_ms += ms_p
        g_flops += P["gemm_flops"]
    gemm_tflops = g_flops / (g_ms * 1e-3) / 1e12
    del layer
    torch.cuda.empty_cache()

    gemv = gemv_roofline(dev, args.steps)
    rows = {"llama65b_layer_projections": per}
    if not args.no_rows:
        rows["llama7b_mlp_4096x11008_r64_m4096"] = llama7b_mlp_rows(dev, args.steps, args.warmup)
        rows.update(other_rows(dev, args.steps))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline()

    out = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s (one LLaMA-65B decoder layer, 7 projections, "
                  "2048 tokens, r=64)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) fp32 weights -> NF4+DQ; bf16 N(0,1) X, dY; "
                "bf16 N(0,0.01) A, B; the parity tests' host recipe)",
        "config": {"workload": "llama65b_layer_7proj_r64_m2048", "tokens": 2048,
                   "projections": [[P_k, P_n] for P_k, P_n in LAYER65B_SHAPES], "r": 64,
                   "alpha": 16.0, "flops_per_step": flops},
        "roofline": {
            "bound": "mfma",
            "kernel": FWD_GEMM + " (forward dequant-GEMM, the layer's 7 launches)",
            "achieved": gemm_tflops,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / BF16_PEAK_TFLOPS,
            "us_per_launch": g_ms * 1e3 / 7,
            "flops_per_launch": g_flops / 7,
            "traffic": read_traffic(),
        },
        "roofline_gemv": gemv,
        "rows": rows,
        "cpu_baseline": cpu,
        "wall_s": wall,
    }
    print(json.dumps(out), flush=True)


LAYER65B_SHAPES = [(8192, 8192)] * 4 + [(8192, 22016)] * 2 + [(22016, 8192)]


def layer65b_setup(dev):
    """The seven projections of one LLaMA-65B-shaped decoder layer with the
    parity tests' seeded host inputs (weights drawn in threads), quantised on
    the GPU, with resident outputs and workspaces: a list of dicts holding
    fwd(), bwd() and gemm() (the forward dequant-GEMM alone) closures."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    with ThreadPoolExecutor(7) as ex:
        inps = list(ex.map(lambda w: w.inputs(), wl.LLAMA65B_LAYER))
    out = []
    for wlc, inp in zip(wl.LLAMA65B_LAYER, inps):
        M, K, N, r, alpha = wlc.M, wlc.k_in, wlc.n_out, wlc.r, wlc.alpha
        W = torch.from_numpy(inp["W"]).to(dev)
        wq = q.quantize_weight(W)
        del W
        X, A, B, dY = (inp[k].to(dev) for k in ("X", "A", "B", "dY"))
        ws_f = torch.empty(q.workspace_size(0, M, N, K, r), dtype=torch.uint8, device=dev)
        ws_b = torch.empty(q.workspace_size(1, M, N, K, r), dtype=torch.uint8, device=dev)
        Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        U = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
        dA = torch.empty(r, K, dtype=torch.float32, device=dev)
        dB = torch.empty(N, r, dtype=torch.float32, device=dev)
        P = dict(name=wlc.name, wq=wq, X=X, A=A, B=B, dY=dY, Y=Y, U=U, dX=dX, dA=dA, dB=dB,
                 flops=wlc.flops_fwd + wlc.flops_bwd, gemm_flops=2 * M * K * N + 2 * M * r * N)
        P["fwd"] = (lambda P=P, wlc=wlc, ws_f=ws_f: q.linear_fwd(
            P["wq"], P["X"], P["A"], P["B"], wlc.alpha, workspace=ws_f, Y=P["Y"], U=P["U"]))
        P["bwd"] = (lambda P=P, wlc=wlc, ws_b=ws_b: q.linear_bwd(
            P["wq"], P["X"], P["dY"], P["A"], P["B"], P["U"], wlc.alpha, workspace=ws_b,
            dX=P["dX"], dA=P["dA"], dB=P["dB"]))
        P["gemm"] = (lambda P=P, wlc=wlc, ws_f=ws_f: q.nf4_matmul_fwd(
            P["wq"], P["X"], P["U"], P["B"], wlc.alpha, workspace=ws_f, Y=P["Y"]))
        out.append(P)
    del inps
    return out


def gemv_roofline(dev, steps):
    """The few-token dequant-GEMV kernel alone (8192 -> 28672, r = 16, the
    adapter term fused; U given), one launch per call, five weight copies
    rotating past the 256 MB last-level cache.  Algorithmic bytes per launch:
    the NF4 + DQ weight, X, B, U and Y once each."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    g = wl.GEMV_70B
    gin = g.inputs(M=1, with_w=True)
    Wg = torch.from_numpy(gin["W"]).to(dev)
    copies = [q.quantize_weight(Wg if c == 0 else Wg * (1.0 + c * 1e-3)) for c in range(5)]
    del Wg
    Ag, Bg = gin["A"].to(dev), gin["B"].to(dev)
    res = {}
    for m in (1, 8):
        Xg = wl.bf16_normal(4, (m, g.k_in), 1.0, tensor=wl.T_X).to(dev)
        Ug = q.lora_down(Xg, Ag)
        ws = torch.empty(q.workspace_size(0, m, g.n_out, g.k_in, g.r), dtype=torch.uint8,
                         device=dev)
        Yg = torch.empty(m, g.n_out, dtype=torch.bfloat16, device=dev)
        calls = [(lambda w_=w_: q.nf4_matmul_fwd(w_, Xg, Ug, Bg, g.alpha, workspace=ws, Y=Yg))
                 for w_ in copies]
        ms = _time_ms(_rotate(calls), 50, warmup=5)
        nbytes = copies[0].nbytes + 2 * m * g.k_in + 2 * g.r * g.n_out + 2 * m * g.r \
            + 2 * m * g.n_out
        res[m] = dict(us=ms * 1e3, GBps=nbytes / ms / 1e6, bytes=nbytes)
    del copies
    torch.cuda.empty_cache()
    a = res[1]
    return {"bound": "hbm", "kernel": "nf4_gemv_kernel (8192 -> 28672, r = 16, 1 token)",
            "achieved": a["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": a["GBps"] / HBM_PEAK_GBS, "us_per_launch": a["us"],
            "bytes_per_launch": a["bytes"], "traffic": read_gemv_traffic(),
            "tokens_8": dict(GBps=res[8]["GBps"], frac=res[8]["GBps"] / HBM_PEAK_GBS,
                             us_per_launch=res[8]["us"])}


def llama7b_mlp_rows(dev, steps, warmup):
    """The LLaMA-7B MLP linear (4096 tokens, 4096 -> 11008, r = 64): the
    training step, its forward dequant-GEMM alone, and the forward and the
    backward on their own."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    wlc = wl.LLAMA7B_MLP
    M, K, N, r, alpha = wlc.M, wlc.k_in, wlc.n_out, wlc.r, wlc.alpha
    inp = wlc.inputs()
    W = torch.from_numpy(inp["W"]).to(dev)
    X, A, B, dY = (inp[k].to(dev) for k in ("X", "A", "B", "dY"))
    wq = q.quantize_weight(W)
    ws_f = torch.empty(q.workspace_size(0, M, N, K, r), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(q.workspace_size(1, M, N, K, r), dtype=torch.uint8, device=dev)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    U = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(r, K, dtype=torch.float32, device=dev)
    dB = torch.empty(N, r, dtype=torch.float32, device=dev)

    def step():
        q.linear_fwd(wq, X, A, B, alpha, workspace=ws_f, Y=Y, U=U)
        q.linear_bwd(wq, X, dY, A, B, U, alpha, workspace=ws_b, dX=dX, dA=dA, dB=dB)
    ms_step = _time_ms(step, steps, warmup=warmup)
    flops = wlc.flops_fwd + wlc.flops_bwd
    gemm_flops = 2 * M * K * N + 2 * M * r * N
    ms_gemm = _time_ms(lambda: q.nf4_matmul_fwd(wq, X, U, B, alpha, workspace=ws_f, Y=Y), steps,
                       warmup=3)
    ms_fwd = _time_ms(lambda: q.linear_fwd(wq, X, A, B, alpha, workspace=ws_f, Y=Y, U=U), steps)
    ms_bwd = _time_ms(lambda: q.linear_bwd(wq, X, dY, A, B, U, alpha, workspace=ws_b, dX=dX,
                                           dA=dA, dB=dB), steps)
    # the same step with LoRA dropout p = 0.05 on the adapter input
    Xdr = torch.empty_like(X)
    ws_d = torch.empty(q.workspace_size(2, M, N, K, r), dtype=torch.uint8, device=dev)
    it = [0]

    def step_dropout():
        it[0] += 1
        q.linear_fwd_dropout(wq, X, A, B, alpha, 0.05, 1234, it[0], workspace=ws_f, Y=Y, U=U,
                             Xd=Xdr)
        q.linear_bwd_dropout(wq, Xdr, dY, A, B, U, alpha, 0.05, 1234, it[0], workspace=ws_d,
                             dX=dX, dA=dA, dB=dB)
    ms_dr = _time_ms(step_dropout, steps)
    out = dict(ms=ms_step, TFLOPs=flops / (ms_step * 1e-3) / 1e12, flops_per_step=flops,
               fwd_ms=ms_fwd, bwd_ms=ms_bwd, fwd_gemm_us=ms_gemm * 1e3,
               fwd_gemm_TFLOPs=gemm_flops / (ms_gemm * 1e-3) / 1e12,
               fwd_gemm_frac=gemm_flops / (ms_gemm * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
               lora_dropout_0_05=dict(ms=ms_dr, TFLOPs=flops / (ms_dr * 1e-3) / 1e12,
                                      overhead_vs_plain=ms_dr / ms_step - 1.0))
    rows = {"train_step": out,
            "merge_adapter_11008x4096_r64": merge_row(W, B, A, alpha)}
    rows.update(variant_rows(W))
    rows.update(quant_rows(W, wq, dev))
    del W, X, A, B, dY, wq, ws_f, ws_b, Y, U, dX, dA, dB, Xdr, ws_d
    torch.cuda.empty_cache()
    return rows


def quant_rows(W, wq, dev):
    """The fused quantiser (NF4 + DQ) and the dequantiser on the 11008 x 4096
    weight: three / five input copies rotate past the last-level cache so every
    call streams from HBM."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q

    N, K = W.shape
    n = K * N
    qbytes = n * 4 + n // 2 + n // 64 + ((n // 64 + 255) // 256) * 4
    L = q.lib()
    st = q._stream(dev)
    Ws = [W] + [W * (1.0 + c * 1e-3) for c in (1, 2)]
    qouts = [q.quantize_nf4_dq(w_, want_absmax=True) for w_ in Ws]
    qcalls = [_c_call(L.qlora_quantize_nf4_dq, q._ptr(w_), n, q._ptr(o[0]), q._ptr(o[1]),
                      q._ptr(o[2]), q._ptr(o[3]), None, st) for w_, o in zip(Ws, qouts)]
    ms_q = _time_ms(_rotate(qcalls), 21, warmup=6)
    dbytes = n // 2 + n // 64 + ((n // 64 + 255) // 256) * 4 + 2 * n
    wqs = [q.NF4Tensor(o[0], o[1], o[2], N, K) for o in qouts] + \
        [q.quantize_weight(W * (1.0 + c * 1e-3)) for c in (3, 4)]
    del Ws, qouts
    wds = [torch.empty(N, K, dtype=torch.bfloat16, device=dev) for _ in wqs]
    wsts = [w_.c_struct() for w_ in wqs]
    dcalls = [_c_call(L.qlora_dequantize_nf4, ctypes.byref(sc), q._ptr(o), st)
              for sc, o in zip(wsts, wds)]
    ms_d = _time_ms(_rotate(dcalls), 20, warmup=5)
    return {"quantize_nf4_dq": dict(shape=[N, K], ms=ms_q, GBps=qbytes / ms_q / 1e6,
                                    hbm_frac=qbytes / ms_q / 1e6 / HBM_PEAK_GBS),
            "dequantize_nf4": dict(shape=[N, K], ms=ms_d, GBps=dbytes / ms_d / 1e6,
                                   hbm_frac=dbytes / ms_d / 1e6 / HBM_PEAK_GBS)}


def other_rows(dev, steps):
    """Few-token forward at 1..8 tokens (U launch + GEMV, end to end), the
    AdamW step, the single 16-token linear and the LLaMA-7B weight set."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    rows = {}
    g = wl.GEMV_70B
    gin = g.inputs(M=8)
    Wg = torch.from_numpy(gin["W"]).to(dev)
    copies = [q.quantize_weight(Wg if c == 0 else Wg * (1.0 + c * 1e-3)) for c in range(5)]
    del Wg
    Ag, Bg = gin["A"].to(dev), gin["B"].to(dev)
    gemv = {}
    for m in wl.GEMV_TOKENS:
        Xg = wl.bf16_normal(4, (m, g.k_in), 1.0, tensor=wl.T_X).to(dev)
        wsg = torch.empty(q.workspace_size(0, m, g.n_out, g.k_in, g.r), dtype=torch.uint8,
                          device=dev)
        Yg = torch.empty(m, g.n_out, dtype=torch.bfloat16, device=dev)
        Ug = torch.empty(m, g.r, dtype=torch.bfloat16, device=dev)
        calls = [(lambda w_=w_: q.linear_fwd(w_, Xg, Ag, Bg, g.alpha, workspace=wsg, Y=Yg, U=Ug))
                 for w_ in copies]
        ms = _time_ms(_rotate(calls), 50, warmup=5)
        gbytes = copies[0].nbytes + 2 * m * g.k_in + 2 * g.r * (g.k_in + g.n_out) \
            + 2 * m * g.n_out + 2 * m * g.r
        gemv[str(m)] = dict(us=ms * 1e3, GBps=gbytes / ms / 1e6,
                            hbm_frac=gbytes / ms / 1e6 / HBM_PEAK_GBS)
    rows["few_token_fwd_8192x28672_r16"] = gemv
    del copies, Ag, Bg
    torch.cuda.empty_cache()
    rows["adamw_step_llama7b_lora_r64"] = adamw_row(dev)
    rows["single_linear_4096x4096_r8_m16"] = single_linear_row(dev)
    rows["llama7b_weight_set_224_matrices"] = weight_set_row(dev)
    return rows


def single_linear_row(dev):
    """A single QLoRA linear, 4096 -> 4096, r = 8, alpha = 16, 16 tokens, forward
    only.  Algorithmic bytes: the NF4+DQ weight plus X, A, B, U and Y, once each
    (9,048,320 B).  64 weight copies (554 MB, over twice the 256 MB last-level
    cache) rotate, so every forward streams its weight from HBM.  Reported back
    to back (calls marshalled once, the queue kept full) and one launch at a
    time (the host waits for each forward)."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    wlc = wl.SINGLE_LINEAR
    M, K, N, r = wlc.M, wlc.k_in, wlc.n_out, wlc.r
    inp = wlc.inputs()
    W = torch.from_numpy(inp["W"]).to(dev)
    copies = [q.quantize_weight(W if c == 0 else W * (1.0 + c * 1e-4)) for c in range(64)]
    del W
    X, A, B = (inp[k].to(dev) for k in ("X", "A", "B"))
    ws = torch.empty(q.workspace_size(0, M, N, K, r), dtype=torch.uint8, device=dev)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    U = torch.empty(M, r, dtype=torch.bfloat16, device=dev)
    L, st = q.lib(), q._stream(dev)
    structs = [w_.c_struct() for w_ in copies]
    calls = [_c_call(L.qlora_linear_fwd, ctypes.byref(sc), q._ptr(X), M, q._ptr(A), q._ptr(B), r,
                     ctypes.c_float(wlc.alpha), q._ptr(Y), q._ptr(U), q._ptr(ws), ws.numel(), st)
             for sc in structs]
    it = [0]

    def fwd():
        calls[it[0] % len(calls)]()
        it[0] += 1
    ms_b2b = _time_ms(fwd, 256, warmup=64)
    single = []
    for _ in range(32):
        torch.cuda.synchronize()
        s, e = _events()
        s.record()
        fwd()
        e.record()
        torch.cuda.synchronize()
        single.append(s.elapsed_time(e))
    single.sort()
    ms_one = single[len(single) // 2]
    nbytes = copies[0].nbytes + 2 * M * K + 2 * r * (K + N) + 2 * M * N + 2 * M * r
    return dict(bytes=nbytes, us_back_to_back=ms_b2b * 1e3, GBps=nbytes / ms_b2b / 1e6,
                hbm_frac=nbytes / ms_b2b / 1e6 / HBM_PEAK_GBS, us_one_launch=ms_one * 1e3,
                TFLOPs=wlc.flops_fwd / (ms_b2b * 1e-3) / 1e12)


def weight_set_row(dev):
    """The LLaMA-7B weight set: 32 layers x (q, k, v, o 4096x4096; gate, up
    4096 -> 11008; down 11008 -> 4096) = 224 matrices, 6,476,005,376 weights,
    all resident in HBM.  One pass of the fused quantise + DQ over all 224
    (4.5159 B per weight: 29.25 GB) and one pass of the dequantiser to bf16
    (2.5159 B per weight: 16.29 GB), through the batch entry points (two and
    one launches per 48 matrices) and, for comparison, one call per matrix.
    The float32 inputs are drawn on the GPU
    (seeded torch normals times 0.02, 0.1 % of positions set to +-8 sigma):
    drawing 6.5 G values on the host would take minutes, and the time does not
    depend on the values."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    L, st = q.lib(), q._stream(dev)
    gen = torch.Generator(device=dev).manual_seed(wl.SEED + 2)
    mats = []
    for layer in range(wl.LLAMA7B_LAYERS):
        for name, n_out, k_in in wl.LLAMA7B_MATRICES:
            n = n_out * k_in
            w = torch.randn(n, generator=gen, device=dev) * 0.02
            pos = torch.rand(n, generator=gen, device=dev) < 1e-3
            w[pos] = torch.where(torch.rand(n, generator=gen, device=dev)[pos] < 0.5, -0.16, 0.16)
            del pos
            nb = n // 64
            mats.append(dict(
                w=w, n=n, n_out=n_out, k_in=k_in,
                packed=torch.empty(n // 2, dtype=torch.uint8, device=dev),
                qa=torch.empty(nb, dtype=torch.int8, device=dev),
                c2=torch.empty((nb + 255) // 256, dtype=torch.float32, device=dev),
                am=torch.empty(nb, dtype=torch.float32, device=dev),
                out=torch.empty(n_out, k_in, dtype=torch.bfloat16, device=dev)))
    total = sum(m["n"] for m in mats)
    qcalls = [_c_call(L.qlora_quantize_nf4_dq, q._ptr(m["w"]), m["n"], q._ptr(m["packed"]),
                      q._ptr(m["qa"]), q._ptr(m["c2"]), q._ptr(m["am"]), None, st) for m in mats]
    structs = [q.NF4Weight(m["packed"].data_ptr(), m["qa"].data_ptr(), m["c2"].data_ptr(),
                           m["n_out"], m["k_in"]) for m in mats]
    dcalls = [_c_call(L.qlora_dequantize_nf4, ctypes.byref(sc), q._ptr(m["out"]), st)
              for sc, m in zip(structs, mats)]

    jobs = (q.QuantJob * len(mats))(*[q.QuantJob(m["w"].data_ptr(), m["n"], m["packed"].data_ptr(),
                                                 m["qa"].data_ptr(), m["c2"].data_ptr(),
                                                 m["am"].data_ptr(), None) for m in mats])
    outs = (ctypes.c_void_p * len(mats))(*[m["out"].data_ptr() for m in mats])
    wsa = (q.NF4Weight * len(mats))(*structs)
    qbatch = _c_call(L.qlora_quantize_nf4_dq_batch, jobs, len(mats), st)
    dbatch = _c_call(L.qlora_dequantize_nf4_batch, wsa, outs, len(mats), st)

    def qpass():
        for c in qcalls:
            c()

    def dpass():
        for c in dcalls:
            c()
    ms_q = _time_ms(qbatch, 3, warmup=1)
    ms_d = _time_ms(dbatch, 3, warmup=1)
    ms_q1 = _time_ms(qpass, 3, warmup=1)
    ms_d1 = _time_ms(dpass, 3, warmup=1)
    nblk = total // 64
    qbytes = total * 4 + total // 2 + nblk + sum(((m["n"] // 64 + 255) // 256) * 4 for m in mats)
    dbytes = total // 2 + nblk + sum(((m["n"] // 64 + 255) // 256) * 4 for m in mats) + 2 * total
    del mats, qcalls, dcalls, structs, jobs, outs, wsa, qbatch, dbatch
    torch.cuda.empty_cache()
    return dict(matrices=32 * len(wl.LLAMA7B_MATRICES), weights=total,
                quantize_dq=dict(ms=ms_q, GB=qbytes / 1e9, GBps=qbytes / ms_q / 1e6,
                                 hbm_frac=qbytes / ms_q / 1e6 / HBM_PEAK_GBS,
                                 ms_one_call_per_matrix=ms_q1),
                dequantize=dict(ms=ms_d, GB=dbytes / 1e9, GBps=dbytes / ms_d / 1e6,
                                hbm_frac=dbytes / ms_d / 1e6 / HBM_PEAK_GBS,
                                ms_one_call_per_matrix=ms_d1))


def adamw_row(dev):
    """The 32-bit AdamW step with global-norm clipping over the LoRA factors of
    LLaMA-7B's four attention projections at r = 64: 32 layers x 4 matrices x
    (A and B), 256 tensors of 64 x 4096, 67,108,864 parameters.  Algorithmic
    bytes per parameter: the norm pass reads g (4); the update reads p, g, m, v
    (16) and writes p, m, v (12) and the bf16 copy (2): 34."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    n_t, size = wl.ADAMW_TENSORS, wl.ADAMW_TENSOR_SIZE
    gen = torch.Generator(device=dev).manual_seed(wl.SEED)
    mk = lambda s: torch.randn(n_t, size, generator=gen, device=dev) * s
    P, G, Mo, V = mk(0.01), mk(1e-3), mk(1e-4), mk(1e-6).abs()
    PB = torch.empty(n_t, size, dtype=torch.bfloat16, device=dev)
    lst = q.AdamWList(list(P), list(G), list(Mo), list(V), list(PB))
    ws = torch.empty(q.adamw_workspace_size(n_t), dtype=torch.uint8, device=dev)
    norm = torch.empty(1, dtype=torch.float32, device=dev)
    plan = q.AdamWPlan(list(P), list(G), list(Mo), list(V), list(PB))
    it = [1]

    def step_plan():  # the prepared list: one launch per pass
        q.adamw_step_plan(plan, it[0], grad_norm=norm)
        it[0] += 1

    def step_list():  # descriptors in the kernel arguments, 48 tensors per launch
        q.adamw_step_list(lst, it[0], grad_norm=norm, workspace=ws)
        it[0] += 1
    ms = _time_ms(step_plan, 20, warmup=5)
    ms_list = _time_ms(step_list, 20, warmup=5)
    nparam = n_t * size
    nbytes = 34 * nparam
    # the paged step: m and v in pinned host memory (the device keeps p and g),
    # read and written there by the update every step
    Mh, Vh = Mo.cpu().pin_memory(), V.cpu().pin_memory()

    def step_paged():
        q.adamw_step_paged(list(P), list(G), list(Mh), list(Vh), it[0], params_bf16=list(PB),
                           grad_norm=norm, workspace=ws)
        it[0] += 1
    ms_paged = _time_ms(step_paged, 5, warmup=2)
    moved = 2 * 2 * 4 * nparam  # m and v, in and out
    return dict(tensors=n_t, params=nparam, ms=ms, GBps=nbytes / ms / 1e6,
                hbm_frac=nbytes / ms / 1e6 / HBM_PEAK_GBS, ms_unprepared_list=ms_list,
                paged=dict(ms=ms_paged, host_link_GBps=moved / ms_paged / 1e6,
                           device_bytes_saved=8 * nparam))


def variant_rows(W):
    """Single quantisation with either code on the 11008 x 4096 weight: the
    INT4 quantiser (4 B read, 0.5 + 4/64 B written per weight), the single
    decode (0.5 + 4/64 B read, 2 B written), the squared-error pass (4 + 0.5 +
    4/64 B read), and the NF4-vs-INT4 mean squared error on that weight."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q

    n = W.numel()
    nb = (n + 63) // 64
    qbytes = 4 * n + n // 2 + 4 * nb
    dbytes = n // 2 + 4 * nb + 2 * n
    ebytes = 4 * n + n // 2 + 4 * nb
    rows, mse = {}, {}
    L = q.lib()
    st = q._stream(W.device)
    # five weight copies (901 MB) rotate, so every timed call streams from HBM
    Ws = [W] + [W * (1.0 + c * 1e-3) for c in (1, 2, 3, 4)]
    outs = [torch.empty(n, dtype=torch.bfloat16, device=W.device) for _ in Ws]
    ws = torch.empty(q.quant_error_workspace_size(n), dtype=torch.uint8, device=W.device)
    sse = torch.empty(1, dtype=torch.float64, device=W.device)
    for code in ("int4", "nf4"):
        cd = q.CODES[code]
        qs = [q.quantize_4bit(w_, code) for w_ in Ws]
        _c_call(L.qlora_quant_sq_error, q._ptr(W), n, cd, q._ptr(qs[0][0]), q._ptr(qs[0][1]),
                q._ptr(sse), q._ptr(ws), ws.numel(), st)()
        mse[code] = float(sse.cpu()[0]) / n
        if code == "int4":
            ms_e = _time_ms(_rotate([
                _c_call(L.qlora_quant_sq_error, q._ptr(w_), n, cd, q._ptr(p_), q._ptr(a_),
                        q._ptr(sse), q._ptr(ws), ws.numel(), st) for w_, (p_, a_) in zip(Ws, qs)]),
                20, warmup=5)
            scratch = [(torch.empty_like(p_), torch.empty_like(a_)) for p_, a_ in qs]
            ms_q = _time_ms(_rotate([
                _c_call(L.qlora_quantize_4bit, q._ptr(w_), n, cd, q._ptr(p2), q._ptr(a2), st)
                for w_, (p2, a2) in zip(Ws, scratch)]), 20, warmup=5)
            ms_d = _time_ms(_rotate([
                _c_call(L.qlora_dequantize_4bit, q._ptr(p_), q._ptr(a_), n, cd, q._ptr(o_), st)
                for (p_, a_), o_ in zip(qs, outs)]), 20, warmup=5)
            del scratch
            rows["quantize_int4_single"] = dict(shape=list(W.shape), ms=ms_q,
                                                GBps=qbytes / ms_q / 1e6,
                                                hbm_frac=qbytes / ms_q / 1e6 / HBM_PEAK_GBS)
            rows["dequantize_int4_single"] = dict(shape=list(W.shape), ms=ms_d,
                                                  GBps=dbytes / ms_d / 1e6,
                                                  hbm_frac=dbytes / ms_d / 1e6 / HBM_PEAK_GBS)
            rows["quant_sq_error_int4"] = dict(shape=list(W.shape), ms=ms_e,
                                               GBps=ebytes / ms_e / 1e6,
                                               hbm_frac=ebytes / ms_e / 1e6 / HBM_PEAK_GBS)
        del qs
    del Ws, outs
    rows["nf4_vs_int4_mse"] = dict(mse_nf4=mse["nf4"], mse_int4=mse["int4"],
                                   improvement_pct=(1 - mse["nf4"] / mse["int4"]) * 100)
    return rows


def merge_row(W, B, A, alpha):
    """Adapter merge at the 11008 x 4096 shape, r = 64: the merge kernel alone
    (2·n·r flop of float64 fma on the vector ALU, rounded once to bf16), the merge with
    re-quantisation, both bases, and how much of the adapter's delta survives
    re-quantisation on each path (its projection on the delta)."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q

    N, K = W.shape
    r = A.shape[0]
    s = alpha / r
    W16 = W.to(torch.bfloat16)
    wq = q.quantize_weight(W)
    merged = torch.empty(N, K, dtype=torch.bfloat16, device=W.device)
    ms_m = _time_ms(lambda: q.merge_adapter(W16, A, B, alpha, requantize=False, merged=merged), 10)
    ms_mq = _time_ms(lambda: q.merge_adapter(W16, A, B, alpha, merged=merged), 10)
    ms_m4 = _time_ms(lambda: q.merge_adapter(wq, A, B, alpha, merged=merged), 10)
    flops = 2.0 * N * K * r
    D = s * (B.float() @ A.float())
    base4 = q.dequantize_nf4(wq).float()
    out = {}
    for name, base in (("16bit", W16), ("4bit", wq)):
        _, rq = q.merge_adapter(base, A, B, alpha)
        d = q.dequantize_nf4(rq).float()
        ref = base4 if name == "4bit" else W16.float()
        out["delta_kept_" + name] = float(((d - ref) * D).sum() / (D * D).sum())
        out["rel_err_" + name] = float((d - (W16.float() + D)).norm() / (W16.float() + D).norm())
    return dict(r=r, ms_merge=ms_m, TFLOPs_merge=flops / (ms_m * 1e-3) / 1e12,
                alu_frac=flops / (ms_m * 1e-3) / 1e12 / FP64_FMA_PEAK_TFLOPS,
                ms_merge_requant_16bit=ms_mq, ms_merge_requant_4bit=ms_m4, **out)


def cpu_baseline():
    """The oracle, untuned, on the host cores, BLAS threads pinned to the
    stated count: decode the weight from its NF4 + DQ storage, then the
    float64 forward and backward, on a bounded sample of the layer step (its
    q projection, 8192 -> 8192, all 2048 tokens, repeated for about 10 s),
    plus the rate of one thread on 256 of those tokens and the oracle's wall
    time on the other workloads."""
    import torch
    from threadpoolctl import threadpool_limits

    import workloads as wl
    from oracle.linear import linear_bwd, linear_fwd, lora_scale
    from oracle.quant import bf16_to_f64, dequantize_nf4, double_quant, quantize_nf4

    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    wlc = wl.LLAMA65B_LAYER[0]
    inp = wlc.inputs()
    packed, absmax = quantize_nf4(inp["W"].ravel())
    qa, c2 = double_quant(absmax)
    f64 = lambda t: t.to(torch.float64).numpy()
    X, A, B, dY = (f64(inp[k]) for k in ("X", "A", "B", "dY"))
    s = lora_scale(wlc.alpha, wlc.r)
    shape = (wlc.n_out, wlc.k_in)

    def one(Xs, dYs):
        w64 = bf16_to_f64(dequantize_nf4(packed, qa, c2, inp["W"].size)).reshape(shape)
        linear_fwd(Xs, w64, A, B, s)
        linear_bwd(Xs, dYs, w64, A, B, s)

    flops = wlc.flops_fwd + wlc.flops_bwd
    with threadpool_limits(cores):
        reps, t0 = 0, time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 10.0:
            one(X, dY)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
    m1 = 256
    f1 = flops * m1 / wlc.M
    with threadpool_limits(1):
        t0 = time.perf_counter()
        one(X[:m1], dY[:m1])
        dt1 = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds_per_sample": dt, "repeats": reps,
            "sample": f"the q projection of the layer step ({wlc.name}: decode from NF4 + DQ, "
                      "float64 forward + backward, all 2048 tokens) repeated for about 10 s, "
                      f"numpy/OpenBLAS pinned to {cores} threads; the layer step is 12.0x its flops",
            "one_thread": {"TFLOPs": f1 / dt1 / 1e12, "seconds": dt1,
                           "sample": f"the same projection on {m1} of the 2048 tokens, 1 thread "
                                     "(decode of the whole weight included)"},
            "per_config": oracle_per_config(cores)}


def oracle_per_config(cores):
    """The oracle's wall time on the other workloads (BLAS pinned to `cores`
    threads): measured in full where that takes a few seconds, else on a
    stated sample and extrapolated (labelled)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import workloads as wl
    from oracle.linear import linear_bwd, linear_fwd, lora_scale
    from oracle.quant import bf16_to_f64, dequantize_nf4, double_quant, quantize_nf4

    f64 = lambda t: t.to(torch.float64).numpy()
    out = {}
    with threadpool_limits(cores):
        # single linear: quantise + DQ, decode and the 16-token forward, in full
        w1 = wl.SINGLE_LINEAR
        inp = w1.inputs()
        t0 = time.perf_counter()
        p1, a1 = quantize_nf4(inp["W"].ravel())
        q1, c1 = double_quant(a1)
        w64 = bf16_to_f64(dequantize_nf4(p1, q1, c1, inp["W"].size)).reshape(w1.n_out, w1.k_in)
        linear_fwd(f64(inp["X"]), w64, f64(inp["A"]), f64(inp["B"]), lora_scale(w1.alpha, w1.r))
        out["single_linear_4096x4096_r8_m16"] = dict(
            seconds=time.perf_counter() - t0, what="quantise + DQ + decode + forward, in full")
        # LLaMA-7B MLP training step: decode + forward + backward, in full
        w3 = wl.LLAMA7B_MLP
        inp = w3.inputs()
        p3, a3 = quantize_nf4(inp["W"].ravel())
        q3, c3 = double_quant(a3)
        X, A, B, dY = (f64(inp[k]) for k in ("X", "A", "B", "dY"))
        t0 = time.perf_counter()
        w64 = bf16_to_f64(dequantize_nf4(p3, q3, c3, inp["W"].size)).reshape(w3.n_out, w3.k_in)
        linear_fwd(X, w64, A, B, lora_scale(w3.alpha, w3.r))
        linear_bwd(X, dY, w64, A, B, lora_scale(w3.alpha, w3.r))
        dt = time.perf_counter() - t0
        out["llama7b_mlp_4096x11008_r64_m4096"] = dict(
            seconds=dt, TFLOPs=(w3.flops_fwd + w3.flops_bwd) / dt / 1e12,
            what="decode + float64 forward + backward, all 4096 tokens, in full")
        del X, A, B, dY, w64
        # weight set: one 4096 x 4096 matrix (with its outliers), scaled to 6.48 G weights
        w = wl.llama7b_weight(0, 0).ravel()
        t0 = time.perf_counter()
        p2, a2 = quantize_nf4(w)
        q2, c2_ = double_quant(a2)
        tq = time.perf_counter() - t0
        t0 = time.perf_counter()
        dequantize_nf4(p2, q2, c2_, w.size)
        td = time.perf_counter() - t0
        total = sum(n * k for _, n, k in wl.LLAMA7B_MATRICES) * wl.LLAMA7B_LAYERS
        out["llama7b_weight_set_224_matrices"] = dict(
            seconds_quantize_dq=tq * total / w.size, seconds_dequantize=td * total / w.size,
            what=f"extrapolated from layer 0's q matrix ({w.size} weights) to {total} weights")
        # few-token forward: 1024 of the 28672 output rows of the 8192 -> 28672 weight
        # (the first rows of the same seeded stream), M = 1, scaled to all rows
        g = wl.GEMV_70B
        rows = 1024
        wr = wl.rng(g.workload, 0, 0, wl.T_W).standard_normal(rows * g.k_in, dtype=np.float32)
        wr *= np.float32(0.02)
        gin = g.inputs(M=1, with_dy=False, with_w=False)
        t0 = time.perf_counter()
        p4, a4 = quantize_nf4(wr)
        q4, c4 = double_quant(a4)
        w4 = bf16_to_f64(dequantize_nf4(p4, q4, c4, wr.size)).reshape(rows, g.k_in)
        linear_fwd(f64(gin["X"]), w4, f64(gin["A"]), f64(gin["B"][:rows]),
                   lora_scale(g.alpha, g.r))
        dt = time.perf_counter() - t0
        out["few_token_fwd_8192x28672_r16"] = dict(
            seconds_quantize_and_forward_m1=dt * g.n_out / rows,
            what=f"extrapolated from {rows} of {g.n_out} output rows (quantise + DQ + decode "
                 "+ forward of one token)")
    return out


if __name__ == "__main__":
    main()
