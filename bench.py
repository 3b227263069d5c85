"""Benchmark of the QLoRA NF4 linear hot path on one MI355X.

Step = one training step of the frozen-NF4 QLoRA linear at the LLaMA-7B MLP
shape (4096 tokens, 4096 -> 11008, r = 64, alpha = 16): forward (U = X·Aᵀ, then
the dequant-GEMM with the LoRA prologue) and backward (V = dY·B, the
transposed dequant-GEMM for dX, dA and dB), on resident synthetic inputs.
`value` = algorithmic TFLOP/s of that step.  The same run also measures the
other rows of the hot path: the fused NF4 + double-quant quantiser and the
dequantiser (GB/s over the weight), and the few-token forward at 8192 -> 28672
(GB/s over the weight it streams, M = 1..8, weight copies rotated past the
256 MB Infinity Cache), the 32-bit AdamW step with gradient clipping over
the 67M LoRA parameters of LLaMA-7B's attention projections (GB/s), and the
single-quantisation INT4 quantiser, decoder and error pass with the
NF4-vs-INT4 error on the 11008 x 4096 weight, the training step with LoRA
dropout (p = 0.05) on the adapter input, and the adapter merge with
re-quantisation at that shape.

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
# float32 fma on the vector ALU without packed-float32 instructions (the
# library is built without them): 256 CUs x 64 lanes x 2 flop x 2.4 GHz
FP32_FMA_PEAK_TFLOPS = 78.6
GEMM_SOURCES = ["qlora_gemm.hip", "qlora_common.h", "qlora_kernels.h", "qlora_philox.h"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "traffic_gemm_fwd_llama7b_mlp.txt")
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


def summarize_pmc(fetch_csv, write_csv, out_path):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the forward dequant-GEMM,
    each scaled by what the same counter reads for a device copy of
    CALIB_BYTES, written as a short text summary."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = ("gemm" if "gemm_kernel<256, 256, 2, 2, 0, true, 0, 0>" in name else
                   "copy" if "copyBuffer" in name else None)
            if key:
                vals.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
                vals[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
        return {k: sum(v.values()) / len(v) for k, v in vals.items()}

    f = per_kernel(fetch_csv, "FETCH_SIZE")
    w = per_kernel(write_csv, "WRITE_SIZE")
    kib = CALIB_BYTES / 1024.0
    f_scale = kib / f["copy"]
    w_scale = kib / w["copy"]
    fetch_b = f["gemm"] * f_scale * 1024.0
    write_b = w["gemm"] * w_scale * 1024.0
    M, K, N, r = 4096, 4096, 11008, 64
    algo = N * K // 2 + N * K // 64 + ((N * K // 64 + 255) // 256) * 4 + 2 * M * K \
        + 2 * M * r + 2 * N * r + 2 * M * N
    with open(out_path, "w") as fh:
        fh.write("# HBM traffic of the forward dequant-GEMM (LLaMA-7B MLP: 4096 tokens, 4096 -> 11008,\n")
        fh.write("# r = 64), from rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by the same counter\n")
        fh.write(f"# on a device copy of {CALIB_BYTES} bytes.  Commands (from /tmp, TMPDIR=/tmp):\n")
        fh.write("#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir_f> -o f -- python3 <repo>/bench.py --pmc-pass\n")
        fh.write("#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir_w> -o w -- python3 <repo>/bench.py --pmc-pass\n")
        fh.write("#   python3 <repo>/bench.py --summarize-pmc <dir_f>/f_counter_collection.csv "
                 "<dir_w>/w_counter_collection.csv <this file>\n")
        fh.write(f"kernel_source_sha256_16 = {gemm_source_hash()}\n")
        fh.write(f"fetch_kib_per_launch_raw = {f['gemm']:.1f}\n")
        fh.write(f"write_kib_per_launch_raw = {w['gemm']:.1f}\n")
        fh.write(f"copy_fetch_kib_raw = {f['copy']:.1f}\n")
        fh.write(f"copy_write_kib_raw = {w['copy']:.1f}\n")
        fh.write(f"fetch_scale = {f_scale:.4f}\n")
        fh.write(f"write_scale = {w_scale:.4f}\n")
        fh.write(f"fetch_bytes_per_launch = {fetch_b:.0f}\n")
        fh.write(f"write_bytes_per_launch = {write_b:.0f}\n")
        fh.write(f"traffic_bytes_per_launch = {fetch_b + write_b:.0f}\n")
        fh.write(f"algorithmic_bytes_per_launch = {algo}\n")
        fh.write(f"traffic_over_algorithmic = {(fetch_b + write_b) / algo:.3f}\n")
    print(open(out_path).read())


def summarize_stats(stats_csv, bench_log, out_path):
    """Short text summary of a rocprofv3 --kernel-trace --stats run of this
    script: per-kernel calls and durations, with the bench line it printed."""
    import csv

    rows = list(csv.DictReader(open(stats_csv)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    line = [ln for ln in open(bench_log) if ln.startswith('{"metric"')][-1]
    d = json.loads(line)
    with open(out_path, "w") as fh:
        fh.write("# rocprofv3 kernel statistics of bench.py (LLaMA-7B MLP QLoRA linear: 4096 "
                 "tokens,\n# 4096 -> 11008, r = 64, alpha = 16, and the other rows of the "
                 "bench line), one MI355X.\n")
        fh.write("# commands (from /tmp, TMPDIR=/tmp):\n")
        fh.write("#   rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- "
                 "python3 <repo>/bench.py --no-cpu-baseline --steps 10 --warmup 2 > <log>\n")
        fh.write("#   python3 <repo>/bench.py --summarize-stats <dir>/bench_kernel_stats.csv "
                 "<log> <this file>\n")
        fh.write(f"# bench line under the profiler: value = {d['value']:.1f} TFLOP/s, "
                 f"ms_per_step = {d['ms_per_step']:.3f},\n")
        fh.write(f"#   forward dequant-GEMM (events) = {d['roofline']['ms'] * 1e3:.1f} us\n\n")
        fh.write(f"{'kernel':<80} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} "
                 f"{'total_ms':>10}\n")
        for r in rows:
            fh.write(f"{r['Name'][:80]:<80} {int(r['Calls']):>6} "
                     f"{float(r['AverageNs']) / 1e3:>10.2f} {float(r['MinNs']) / 1e3:>10.2f} "
                     f"{float(r['MaxNs']) / 1e3:>10.2f} "
                     f"{float(r['TotalDurationNs']) / 1e6:>10.3f}\n")
    print(open(out_path).read())


def summarize_counters(out_path, *csvs):
    """Per-dispatch averages of the SQ counters of the forward dequant-GEMM from
    rocprofv3 --pmc runs of --pmc-pass, with the ratios read off them."""
    import csv

    vals = {}
    for path in csvs:
        for r in csv.DictReader(open(path)):
            if "gemm_kernel<256, 256, 2, 2, 0, true, 0, 0>" not in r["Kernel_Name"]:
                continue
            d = vals.setdefault(r["Counter_Name"], {})
            key = (path, r["Dispatch_Id"])  # a counter may appear in several runs
            d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    avg = {k: sum(v.values()) / len(v) for k, v in vals.items()}
    with open(out_path, "w") as fh:
        fh.write("# SQ counters of the forward dequant-GEMM (LLaMA-7B MLP: 4096 tokens, 4096 -> "
                 "11008, r = 64),\n# per dispatch, averaged over the dispatches of --pmc-pass.  "
                 "Commands (from /tmp, TMPDIR=/tmp),\n# one rocprofv3 run per counter set:\n")
        fh.write("#   rocprofv3 --pmc <set> --output-format csv -d <dir_i> -o c -- python3 "
                 "<repo>/bench.py --pmc-pass\n")
        fh.write("#   python3 <repo>/bench.py --summarize-counters <this file> "
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


def pmc_pass():
    """Short run for counter collection: the forward dequant-GEMM a few times
    and a device copy of CALIB_BYTES (the byte counters' calibration)."""
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    dev = torch.device("cuda:0")
    wlc = wl.LLAMA7B_MLP
    inp = wlc.inputs(with_dy=False)
    wq = q.quantize_weight(torch.from_numpy(inp["W"]).to(dev))
    X, A, B = (inp[k].to(dev) for k in ("X", "A", "B"))
    ws = torch.empty(q.workspace_size(0, wlc.M, wlc.n_out, wlc.k_in, wlc.r), dtype=torch.uint8,
                     device=dev)
    U = q.lora_down(X, A)
    Y = torch.empty(wlc.M, wlc.n_out, dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        q.nf4_matmul_fwd(wq, X, U, B, wlc.alpha, workspace=ws, Y=Y)
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("pmc pass done", flush=True)


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

    import numpy as np
    import torch

    import bit_nf4_quantized_blockwise_amd as q
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
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
    flops = wlc.flops_fwd + wlc.flops_bwd
    tflops = flops / (ms_step * 1e-3) / 1e12

    # dominant kernel: the forward dequant-GEMM (one launch: Y = X·Ŵᵀ + s·U·Bᵀ)
    gemm_flops = 2 * M * K * N + 2 * M * r * N
    ms_gemm = _time_ms(lambda: q.nf4_matmul_fwd(wq, X, U, B, alpha, workspace=ws_f, Y=Y),
                       args.steps, warmup=args.warmup)
    gemm_tflops = gemm_flops / (ms_gemm * 1e-3) / 1e12
    # the input-gradient GEMM, timed through the backward (reported for context)
    ms_bwd = _time_ms(lambda: q.linear_bwd(wq, X, dY, A, B, U, alpha, workspace=ws_b, dX=dX,
                                           dA=dA, dB=dB), args.steps)
    ms_fwd = _time_ms(lambda: q.linear_fwd(wq, X, A, B, alpha, workspace=ws_f, Y=Y, U=U),
                      args.steps)

    rows = {}
    if not args.no_rows:
        n = K * N
        # quantiser (fused NF4 + DQ): reads 4 B, writes 0.5 + 1/64 + 4/16384 B per weight
        qbytes = n * 4 + n // 2 + n // 64 + ((n // 64 + 255) // 256) * 4
        L = q.lib()
        st = q._stream(dev)
        pk_, qa_, c2_, am_ = q.quantize_nf4_dq(W, want_absmax=True)
        ms_q = _time_ms(_c_call(L.qlora_quantize_nf4_dq, q._ptr(W), n, q._ptr(pk_), q._ptr(qa_),
                                q._ptr(c2_), q._ptr(am_), st), 20, warmup=5)
        # dequantiser: reads the NF4 storage, writes bf16
        dbytes = n // 2 + n // 64 + ((n // 64 + 255) // 256) * 4 + 2 * n
        wd = torch.empty(N, K, dtype=torch.bfloat16, device=dev)
        wst = wq.c_struct()
        ms_d = _time_ms(_c_call(L.qlora_dequantize_nf4, ctypes.byref(wst), q._ptr(wd), st), 20,
                        warmup=5)
        rows["quantize_nf4_dq"] = dict(shape=[N, K], ms=ms_q, GBps=qbytes / ms_q / 1e6,
                                       hbm_frac=qbytes / ms_q / 1e6 / HBM_PEAK_GBS)
        rows["dequantize_nf4"] = dict(shape=[N, K], ms=ms_d, GBps=dbytes / ms_d / 1e6,
                                      hbm_frac=dbytes / ms_d / 1e6 / HBM_PEAK_GBS)
        del wd
        # few-token forward, 8192 -> 28672, r = 16; 5 weight copies (> 2x the MALL)
        g = wl.GEMV_70B
        gin = g.inputs(M=8)
        copies = []
        Wg = torch.from_numpy(gin["W"]).to(dev)
        for c in range(5):
            copies.append(q.quantize_weight(Wg if c == 0 else Wg * (1.0 + c * 1e-3)))
        del Wg
        Ag, Bg = gin["A"].to(dev), gin["B"].to(dev)
        gemv = {}
        for m in wl.GEMV_TOKENS:
            Xg = wl.bf16_normal(4, (m, g.k_in), 1.0, tensor=wl.T_X).to(dev)
            wsg = torch.empty(q.workspace_size(0, m, g.n_out, g.k_in, g.r), dtype=torch.uint8,
                              device=dev)
            Yg = torch.empty(m, g.n_out, dtype=torch.bfloat16, device=dev)
            Ug = torch.empty(m, g.r, dtype=torch.bfloat16, device=dev)
            it = [0]

            def fwd():
                w_ = copies[it[0] % len(copies)]
                it[0] += 1
                q.linear_fwd(w_, Xg, Ag, Bg, g.alpha, workspace=wsg, Y=Yg, U=Ug)
            ms = _time_ms(fwd, 50, warmup=5)
            gbytes = copies[0].nbytes + 2 * m * g.k_in + 2 * g.r * (g.k_in + g.n_out) \
                + 2 * m * g.n_out + 2 * m * g.r
            gemv[str(m)] = dict(us=ms * 1e3, GBps=gbytes / ms / 1e6,
                                hbm_frac=gbytes / ms / 1e6 / HBM_PEAK_GBS)
        rows["few_token_fwd_8192x28672_r16"] = gemv
        del copies, Ag, Bg
        # the same training step with LoRA dropout p = 0.05 on the adapter input
        Xdr = torch.empty_like(X)
        ws_d = torch.empty(q.workspace_size(2, M, N, K, r), dtype=torch.uint8, device=dev)
        it = [0]

        def step_dropout():
            it[0] += 1
            q.linear_fwd_dropout(wq, X, A, B, alpha, 0.05, 1234, it[0], workspace=ws_f, Y=Y, U=U,
                                 Xd=Xdr)
            q.linear_bwd_dropout(wq, Xdr, dY, A, B, U, alpha, 0.05, 1234, it[0], workspace=ws_d,
                                 dX=dX, dA=dA, dB=dB)
        ms_dr = _time_ms(step_dropout, args.steps)
        rows["train_step_lora_dropout_0.05"] = dict(ms=ms_dr, TFLOPs=flops / (ms_dr * 1e-3) / 1e12,
                                                    overhead_vs_plain=ms_dr / ms_step - 1.0)
        del Xdr, ws_d
        rows["adamw_step_llama7b_lora_r64"] = adamw_row(dev)
        rows.update(variant_rows(W))
        rows["merge_adapter_11008x4096_r64"] = merge_row(W, B, A, alpha)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, wlc)

    out = {
        "metric": "QLoRA linear fwd+bwd TFLOP/s (LLaMA-7B MLP 4096x11008, 4096 tokens, r=64)",
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
        "data": "synthetic (seeded N(0,0.02) fp32 weight -> NF4+DQ; bf16 N(0,1) X, dY; "
                "bf16 N(0,0.01) A, B)",
        "config": {"workload": wlc.name, "tokens": M, "k_in": K, "n_out": N, "r": r,
                   "alpha": alpha, "flops_per_step": flops,
                   "fwd_ms": ms_fwd, "bwd_ms": ms_bwd},
        "roofline": {
            "bound": "mfma",
            "kernel": "gemm_kernel<256, 256, 2, 2, 0, true, 0, 0> (forward dequant-GEMM)",
            "achieved": gemm_tflops,
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": gemm_tflops / BF16_PEAK_TFLOPS,
            "ms": ms_gemm,
            "traffic": read_traffic(),
        },
        "rows": rows,
        "cpu_baseline": cpu,
        "wall_s": wall,
    }
    print(json.dumps(out), flush=True)


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
    return dict(tensors=n_t, params=nparam, ms=ms, GBps=nbytes / ms / 1e6,
                hbm_frac=nbytes / ms / 1e6 / HBM_PEAK_GBS, ms_unprepared_list=ms_list)


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
    out = torch.empty(n, dtype=torch.bfloat16, device=W.device)
    ws = torch.empty(q.quant_error_workspace_size(n), dtype=torch.uint8, device=W.device)
    sse = torch.empty(1, dtype=torch.float64, device=W.device)
    for code in ("int4", "nf4"):
        packed, absmax = q.quantize_4bit(W, code)
        cd = q.CODES[code]
        ms_e = _time_ms(_c_call(L.qlora_quant_sq_error, q._ptr(W), n, cd, q._ptr(packed),
                                q._ptr(absmax), q._ptr(sse), q._ptr(ws), ws.numel(), st), 20,
                        warmup=5)
        mse[code] = float(sse.cpu()[0]) / n
        if code == "int4":
            p2 = torch.empty_like(packed)
            a2 = torch.empty_like(absmax)
            ms_q = _time_ms(_c_call(L.qlora_quantize_4bit, q._ptr(W), n, cd, q._ptr(p2), q._ptr(a2),
                                    st), 20, warmup=5)
            ms_d = _time_ms(_c_call(L.qlora_dequantize_4bit, q._ptr(packed), q._ptr(absmax), n, cd,
                                    q._ptr(out), st), 20, warmup=5)
            rows["quantize_int4_single"] = dict(shape=list(W.shape), ms=ms_q,
                                                GBps=qbytes / ms_q / 1e6,
                                                hbm_frac=qbytes / ms_q / 1e6 / HBM_PEAK_GBS)
            rows["dequantize_int4_single"] = dict(shape=list(W.shape), ms=ms_d,
                                                  GBps=dbytes / ms_d / 1e6,
                                                  hbm_frac=dbytes / ms_d / 1e6 / HBM_PEAK_GBS)
            rows["quant_sq_error_int4"] = dict(shape=list(W.shape), ms=ms_e,
                                               GBps=ebytes / ms_e / 1e6,
                                               hbm_frac=ebytes / ms_e / 1e6 / HBM_PEAK_GBS)
    rows["nf4_vs_int4_mse"] = dict(mse_nf4=mse["nf4"], mse_int4=mse["int4"],
                                   improvement_pct=(1 - mse["nf4"] / mse["int4"]) * 100)
    return rows


def merge_row(W, B, A, alpha):
    """Adapter merge at the 11008 x 4096 shape, r = 64: the merge kernel alone
    (2·n·r flop of float32 fma on the vector ALU, fixed order), the merge with
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
                alu_frac=flops / (ms_m * 1e-3) / 1e12 / FP32_FMA_PEAK_TFLOPS,
                ms_merge_requant_16bit=ms_mq, ms_merge_requant_4bit=ms_m4, **out)


def cpu_baseline(inp, wlc):
    """The oracle, untuned, on the host cores: decode the weight from its NF4 +
    DQ storage and run the float64 forward and backward for the whole batch."""
    import numpy as np
    import torch

    from oracle.linear import linear_bwd, linear_fwd, lora_scale
    from oracle.quant import bf16_to_f64, dequantize_nf4, double_quant, quantize_nf4

    cores = len(os.sched_getaffinity(0))
    packed, absmax = quantize_nf4(inp["W"].ravel())
    qa, c2 = double_quant(absmax)
    f64 = lambda t: t.to(torch.float64).numpy()
    X, A, B, dY = (f64(inp[k]) for k in ("X", "A", "B", "dY"))
    s = lora_scale(wlc.alpha, wlc.r)
    reps, t0 = 0, time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < 10.0:  # about 10 s of host work
        w64 = bf16_to_f64(dequantize_nf4(packed, qa, c2, inp["W"].size)).reshape(wlc.n_out,
                                                                                 wlc.k_in)
        Y, U = linear_fwd(X, w64, A, B, s)
        dX, dA, dB = linear_bwd(X, dY, w64, A, B, s)
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    flops = wlc.flops_fwd + wlc.flops_bwd
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds_per_step": dt, "steps": reps,
            "sample": f"full steps of {wlc.name} repeated for about 10 s: decode + fp64 "
                      "forward + backward, all 4096 tokens (numpy, float64)"}


if __name__ == "__main__":
    main()
